"""The warp-specialised GEMM's host side on the CPU: the model's
recurrences in libfmha.so against the oracle's event simulation, the launch
time, two-point calibration and the chooser, and the GEMM entry point's
argument checks (no GPU call is made)."""
import itertools
import os
import random
import re

import pytest

from oracle import ws_sim
from software_pipelining_fmha_amd import fmha, ws_gemm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ws_gemm.h")
A = 1 << 20  # fake, aligned "device addresses" (never dereferenced)


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ws_\w+)\s*\(", text, re.M)))


def test_header_declares_the_exports():
    assert declared_functions() == sorted(ws_gemm.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ws_gemm.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def dyadic(rng):
    return rng.randint(1, 64) / 8.0


@pytest.mark.parametrize("seed", range(40))
def test_recurrences_match_event_simulation(seed):
    """Same stage start times, end and MATH wait as the oracle's event-driven
    run of the DMA and MATH agents (dyadic durations: sums are exact)."""
    rng = random.Random(seed)
    S = rng.randint(0, 40)
    ring = rng.randint(1, 6)
    ta, tb, tm = dyadic(rng), dyadic(rng), dyadic(rng)
    sa, sb, sm, end, wait = ws_gemm.stage_times(S, ring, ta, tb, tm)
    ref = ws_sim.simulate_wave(S, ring, ta, tb, tm)
    assert sa == ref.load_a and sb == ref.load_b and sm == ref.math
    assert end == ref.math_end and wait == ref.math_wait


def test_recurrences_reject_bad_arguments():
    with pytest.raises(ValueError):
        ws_gemm.stage_times(-1, 2, 1.0, 1.0, 1.0)
    with pytest.raises(ValueError):
        ws_gemm.stage_times(4, 0, 1.0, 1.0, 1.0)


def make_params(thr=2048.0, lat=0.5, cthr=2.0 ** 20, clat=0.125, epi=1.0, init=3.0, units=256):
    p = ws_gemm.ModelParams()
    p.load_throughput, p.load_latency = thr, lat
    p.compute_throughput, p.compute_latency = cthr, clat
    p.t_epilogue, p.t_init, p.n_units = epi, init, units
    return p


@pytest.mark.parametrize("M,N,K", [(1024, 1024, 1024), (512, 256, 1024), (8192, 8192, 8192),
                                   (1000, 72, 200)])
def test_launch_time_matches_oracle(M, N, K):
    p = make_params()
    for tm, tn, tk, ring in ws_gemm.configs():
        got = ws_gemm.launch_time(p, M, N, K, tm, tn, tk, ring)
        ref = ws_sim.launch_time(M, N, K, tm, tn, tk, ring, p.n_units, p.load_throughput,
                                 p.load_latency, p.compute_throughput, p.compute_latency,
                                 p.t_epilogue, p.t_init)
        assert got == pytest.approx(ref, rel=1e-12)


def test_two_point_matches_oracle():
    got = ws_gemm.two_point(8192.0, 5.5, 16384.0, 9.75)
    assert got == pytest.approx(ws_sim.two_point(8192.0, 5.5, 16384.0, 9.75), rel=1e-14)
    with pytest.raises(ValueError):
        ws_gemm.two_point(1.0, 2.0, 1.0, 3.0)


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (1024, 512, 1024), (8192, 8192, 8192)])
def test_chooser_picks_the_smallest_prediction(M, N, K):
    p = make_params()
    pick = ws_gemm.choose(M, N, K, p)
    times = {c: ws_sim.launch_time(M, N, K, *c, p.n_units, p.load_throughput, p.load_latency,
                                   p.compute_throughput, p.compute_latency, p.t_epilogue,
                                   p.t_init) for c in ws_gemm.configs()}
    best = min(times.values())
    assert times[pick] <= best * (1 + 1e-9)
    # of equal predictions for the picked tile, the deepest ring that the
    # stages can fill (or the shallowest, if none is that shallow)
    same = [c for c in times if c[:3] == pick[:3] and times[c] <= best * (1 + 1e-9)]
    stages = -(-K // pick[2])
    fill = [c[3] for c in same if c[3] <= stages]
    assert pick[3] == (max(fill) if fill else min(c[3] for c in same))


def test_chooser_ring_never_deeper_than_the_stages():
    """K = 256 on T_K = 128 is two stages: rings 3 and 4 predict what ring 2
    does, and the pick stays at two slots or fewer."""
    p = make_params()
    for M, N in ((256, 1024), (64, 64), (1024, 1024)):
        tm, tn, tk, ring = ws_gemm.choose(M, N, 256, p)
        assert ring <= -(-256 // tk)


def test_config_list():
    cfgs = ws_gemm.configs()
    assert len(cfgs) == len(set(cfgs)) == 34
    for tm, tn, tk, ring in cfgs:
        assert tm in (64, 128, 256) and tn in (64, 128) and tk in (64, 128) and 1 <= ring <= 4
        assert ring * (tm * tk + tk * tn) * 2 + 64 <= 160 * 1024
    # the page's tile space, T_M, T_N, T_K in {64, 128}, with two or more slots
    for tm, tn, tk in itertools.product((64, 128), repeat=3):
        assert (tm, tn, tk, 2) in cfgs


def test_trace_words():
    assert ws_gemm.trace_words(256, 256, 1024, 128, 128, 64) == 4 * (16 + 1) * 5
    assert ws_gemm.trace_words(0, 256, 1024, 128, 128, 64) == 0


def gemm_call(a=A, b=2 * A, c=4 * A, M=256, N=256, K=256, cfg=(128, 128, 64, 2)):
    return ws_gemm.lib().ws_gemm(a, b, c, M, N, K, *cfg, None, None, None)


@pytest.mark.parametrize("which", ["a", "b", "c"])
def test_gemm_null_pointer_is_invalid(which):
    assert gemm_call(**{which: 0}) == fmha.FMHA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("field", ["M", "N", "K"])
def test_gemm_negative_size_is_invalid(field):
    assert gemm_call(**{field: -1}) == fmha.FMHA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("field", ["M", "N"])
def test_gemm_empty_output_is_ok(field):
    assert gemm_call(a=0, b=0, c=0, **{field: 0}) == fmha.FMHA_OK


@pytest.mark.parametrize("N,K", [(12, 64), (64, 20)])
def test_gemm_rows_not_16_bytes_is_unsupported(N, K):
    assert gemm_call(N=N, K=K) == fmha.FMHA_ERR_UNSUPPORTED


@pytest.mark.parametrize("which", ["a", "b", "c"])
def test_gemm_misaligned_is_unsupported(which):
    base = {"a": A, "b": 2 * A, "c": 4 * A}[which]
    assert gemm_call(**{which: base + 8}) == fmha.FMHA_ERR_UNSUPPORTED


def test_gemm_unknown_variant_is_unsupported():
    assert gemm_call(cfg=(128, 128, 64, 5)) == fmha.FMHA_ERR_UNSUPPORTED
    assert gemm_call(cfg=(32, 128, 64, 2)) == fmha.FMHA_ERR_UNSUPPORTED


def test_gemm_too_large_is_unsupported():
    assert gemm_call(M=1 << 20, K=1 << 10) == fmha.FMHA_ERR_UNSUPPORTED


def test_gemm_output_overlapping_input_is_invalid():
    assert gemm_call(c=A + 256) == fmha.FMHA_ERR_INVALID_ARGUMENT
