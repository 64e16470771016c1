"""bench.py's default step counts (host logic, no GPU).

A default run times about two seconds of back-to-back launches: long enough
for an outside utilisation sampler to see the work and for the per-launch
spread to average out, short enough that the GPU is not held for long.
"""
import argparse

import bench
from software_pipelining_fmha_amd import inputs

HEADLINE = inputs.WORKLOADS[inputs.HEADLINE].name


def steps(which="fwd", dtype="f16", workload=HEADLINE):
    return bench._default_steps(argparse.Namespace(which=which, dtype=dtype, workload=workload))


def expected_seconds(n, flops, tflops):
    return n * flops / (tflops * 1e12)


def test_headline_lines_time_about_two_seconds():
    w = inputs.WORKLOADS[inputs.HEADLINE]
    for which, dtype, factor in (("fwd", "f16", 1.0), ("fwd", "fp8", 1.0), ("bwd", "f16", 2.5)):
        n = steps(which, dtype)
        rate = bench.USUAL_TFLOPS["fp8" if dtype == "fp8" else which]
        assert 1.5 <= expected_seconds(n, w.flops * factor, rate) <= 2.5, (which, dtype, n)
        assert n >= 20


def test_fp8_name_without_prefix_resolves():
    assert steps("fwd", "fp8", HEADLINE) == steps("fwd", "fp8", "fp8_" + HEADLINE)


def test_small_workloads_are_capped_and_gemm_keeps_its_count():
    assert steps(workload=inputs.WORKLOADS[0].name) == bench.MAX_DEFAULT_STEPS
    assert steps(which="gemm") == 100
    assert steps(which="wsmodel") == 20


def test_command_line_defaults_and_explicit_counts():
    a = bench.parse_args([])
    assert (a.steps, a.warmup) == (steps(), 10)
    a = bench.parse_args(["--dtype", "fp8"])
    assert (a.steps, a.warmup) == (steps("fwd", "fp8"), 20)
    a = bench.parse_args(["--pass", "bwd"])
    assert (a.steps, a.warmup) == (steps("bwd"), 5)
    a = bench.parse_args(["--pass", "gemm", "--steps", "7", "--warmup", "3"])
    assert (a.steps, a.warmup) == (7, 3)
