"""Benchmark of the fused attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--pass fwd|bwd]

A step is one fmha_fwd launch over the whole batch. The default workload is
FP16, B=4, H=32, N=16384, d=128, non-causal; the Twill (section 6.2, Fig. 7)
and Tawa (section V-D) evaluations use this shape at their longest sequence.
Inputs are seeded synthetic N(0,1) draws and are already resident in HBM
when the timed region starts. Throughput counts 4*B*H*N^2*d FLOPs per step,
halved for causal.

Prints one JSON line. It includes the MFMA roofline of the kernel (average
launch time from HIP events on the launch stream) and, on rank 0, the CPU
oracle timed on a bounded row sample. The oracle's rows also check the
timed output.

--dtype fp8 times fmha_fwd_fp8 instead, on the FP8 workloads (the same
shapes and draws quantized per tensor to OCP E4M3), against the MFMA's dense
FP8 peak.

--pass bwd times one fmha_bwd call per step instead (its three kernels: the
row dot products D, dK/dV, dQ) on the same workload plus a seeded output
gradient, after one untimed forward pass that supplies O and lse. It counts
the usual 2.5x the forward's FLOPs (five matrix products of 2*N^2*d per
head), although the kernels execute seven (S and dP are formed again for
dQ).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from software_pipelining_fmha_amd import inputs  # noqa: E402

METRIC = "FMHA fwd TFLOPS (fp16, B4 H32 d128, N=16384) and % of MFMA peak"
PEAK_FP16_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
KERNEL_SOURCES = ("software_pipelining_fmha_amd/csrc/fmha_fwd_kernel.hpp",
                  "software_pipelining_fmha_amd/csrc/fmha_api.hip")
BWD_SOURCES = ("software_pipelining_fmha_amd/csrc/fmha_bwd_kernel.hpp",)
FP8_SOURCES = ("software_pipelining_fmha_amd/csrc/fmha_fwd_fp8_kernel.hpp",)
GEMM_SOURCES = ("software_pipelining_fmha_amd/csrc/ws_gemm_kernel.hpp",
                "software_pipelining_fmha_amd/csrc/ws_gemm_api.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_fmha_fwd_b4h32n16384d128.txt")


_COMMENT = re.compile(r"/\*.*?\*/|//[^\n]*", re.S)


def _source_digest(paths) -> str:
    """Digest of the code in `paths` with comments and whitespace removed, so
    that a profile stays matched to its kernel across comment-only edits."""
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            code = _COMMENT.sub(" ", f.read())
        h.update(" ".join(code.split()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def kernel_digest() -> str:
    return _source_digest(KERNEL_SOURCES)


def fp8_digest() -> str:
    return _source_digest(FP8_SOURCES + KERNEL_SOURCES)


def gemm_digest() -> str:
    return _source_digest(GEMM_SOURCES)


def bwd_digest() -> str:
    return _source_digest(BWD_SOURCES + KERNEL_SOURCES[1:])


def _recorded_counters(workload: str) -> dict:
    """key=value pairs of the committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source and this workload; else {}."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    kv = {}
    for line in open(TRAFFIC_FILE):
        if line.startswith("#"):
            continue
        for item in line.split():
            if "=" in item:
                key, val = item.split("=", 1)
                kv[key.strip()] = val.strip()
    if kv.get("kernel_digest") != kernel_digest() or kv.get("workload") != workload:
        return {}
    return kv


def recorded_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, or None."""
    try:
        return float(_recorded_counters(workload)["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def recorded_mfma_utilisation(workload: str):
    """MFMA busy fraction and SCLK (GHz) from the committed counter summary
    (SQ_VALU_MFMA_BUSY_CYCLES over the active cycles of all SIMDs, and
    GRBM_GUI_ACTIVE over the kernel time), or None."""
    kv = _recorded_counters(workload)
    try:
        return {"mfma_busy": float(kv["mfma_busy_frac_at_measured_clock"]),
                "sclk_ghz": float(kv["sclk_from_GRBM_GUI_ACTIVE_GHz"]),
                "source": os.path.relpath(TRAFFIC_FILE, ROOT)}
    except (KeyError, ValueError):
        return None


def cpu_threads() -> int:
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_baseline(q, k, v, w, scale, o_gpu, lse_gpu, target_s: float):
    """Time the CPU oracle on a seeded row sample of the same workload, and
    compare those rows with the GPU output."""
    import oracle

    threads = cpu_threads()
    idx = inputs.WORKLOADS.index(w)
    rows0 = inputs.workload_rows(idx) if w.sampled_rows else inputs.sample_rows(
        w.B, w.H, w.N, 256, (inputs.SEED_BASE + idx) ^ inputs.SAMPLE_SEED_XOR)
    t0 = time.perf_counter()
    o_ref, l_ref = oracle.fmha_rows(q, k, v, rows0, causal=w.causal, scale=scale, threads=threads)
    t_first = time.perf_counter() - t0
    b, h, i = rows0.T
    err_o = float(np.abs(o_gpu[b, h, i].astype(np.float64) - o_ref).max())
    err_l = float(np.abs(lse_gpu[b, h, i].astype(np.float64) - l_ref).max())
    # the same rows on one thread
    t0 = time.perf_counter()
    oracle.fmha_rows(q, k, v, rows0, causal=w.causal, scale=scale, threads=1)
    t_one = time.perf_counter() - t0
    vis0 = (rows0[:, 2] + 1).astype(np.float64) if w.causal else np.full(len(rows0), float(w.N))
    flops0 = float((4.0 * w.d * vis0).sum())

    # grow the sample to about target_s seconds of oracle work
    n = int(min(w.B * w.H * w.N, max(len(rows0), len(rows0) * target_s / max(t_first, 1e-3))))
    rows = inputs.sample_rows(w.B, w.H, w.N, n, 4242 + idx)
    t0 = time.perf_counter()
    oracle.fmha_rows(q, k, v, rows, causal=w.causal, scale=scale, threads=threads)
    dt = time.perf_counter() - t0
    vis = (rows[:, 2] + 1).astype(np.float64) if w.causal else np.full(len(rows), float(w.N))
    flops = float((4.0 * w.d * vis).sum())
    return {
        "value": flops / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
        "sample": "%d seeded (b,h,i) rows of %s, every visible key per row; %.1f s wall"
                  % (len(rows), w.name, dt),
        "seconds": dt,
        "single_thread": {"value": flops0 / t_one / 1e12, "unit": "TFLOPS",
                          "sample": "the %d parity rows; %.1f s wall" % (len(rows0), t_one)},
    }, {"rows": int(len(rows0)), "max_abs_o": err_o, "max_abs_lse": err_l,
        "pass": bool(err_o <= 2e-3 and err_l <= 1e-3)}


BWD_U = 2.0 ** -11


def bwd_cpu_baseline(q, k, v, do, w, scale, grads, target_s: float):
    """Time the CPU oracle's backward on a bounded sample of one head of the
    workload (dq rows, and dk/dv rows, whose head costs one forward pass),
    and check those rows of the GPU gradients with the parity tests' bar."""
    import oracle

    threads = cpu_threads()
    idx = inputs.WORKLOADS.index(w)
    rng = np.random.default_rng(4343 + idx)
    b, h = 0, int(rng.integers(w.H))
    n = int(min(w.N, 2048))
    qi = np.sort(rng.choice(w.N, size=n, replace=False))
    kj = np.sort(rng.choice(w.N, size=n, replace=False))
    qrows = np.array([(b, h, i) for i in qi], dtype=np.int64)
    krows = np.array([(b, h, j) for j in kj], dtype=np.int64)
    t0 = time.perf_counter()
    ref = oracle.fmha_bwd_rows(q, k, v, do, qrows, krows, causal=w.causal, scale=scale,
                               threads=threads, rss=True)
    dt = time.perf_counter() - t0
    worst = 0.0
    for name, (got, rows, r, rs, ds, c) in {
            "dq": (grads[0], qrows, ref[0], ref[3], ref[6], 3),
            "dk": (grads[1], krows, ref[1], ref[4], ref[7], 21),
            "dv": (grads[2], krows, ref[2], ref[5], 0.0, 0)}.items():
        g = got[rows[:, 0], rows[:, 1], rows[:, 2]].astype(np.float64)
        tol = 8 * BWD_U * rs + 2 * BWD_U * np.abs(r) + c * BWD_U * ds + 2.0 ** -16
        worst = max(worst, float((np.abs(g - r) / tol).max()))
    # Algorithmic work attributed to the sample: each (query, key) pair carries
    # 10 d FLOPs (five products); a dq row covers half of its row's pairs and a
    # dk/dv row half of its column's.
    vis_q = (qi + 1) if w.causal else np.full(n, w.N)
    vis_k = (w.N - kj) if w.causal else np.full(n, w.N)
    flops = 5.0 * w.d * float(vis_q.sum() + vis_k.sum())
    return {
        "value": flops / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
        "sample": "head (b=%d, h=%d) of %s: %d dq rows and %d dk/dv rows (the latter need one "
                  "forward pass over the head); %.1f s wall" % (b, h, w.name, n, n, dt),
    }, {"rows": 2 * n, "max_err_over_bar": worst, "pass": bool(worst <= 1.0)}


def bench_bwd(args, w, idx, q, k, v, scale, tq, tk, tv, dev, stream):
    import torch

    from software_pipelining_fmha_amd import fmha

    do = inputs.workload_dout(idx)
    tdo = torch.from_numpy(do).to(dev)
    o, lse = fmha.forward(tq, tk, tv, causal=w.causal, scale=float(scale), stream=stream)
    dq, dk, dv = (torch.empty_like(tq) for _ in range(3))
    ws = torch.empty((2 * w.B * w.H * w.N,), dtype=torch.float32, device=dev)

    def step():
        fmha.backward(tq, tk, tv, o, lse, tdo, causal=w.causal, scale=float(scale), dq=dq, dk=dk,
                      dv=dv, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = [s_.elapsed_time(e) for s_, e in zip(starts, ends)]
    avg_ms = float(np.mean(call_ms))
    ms_per_step = wall * 1e3 / args.steps
    flops = 2.5 * w.flops
    result = {
        "metric": "FMHA bwd TFLOPS (fp16, %s) and %% of MFMA peak" % w.name,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "bwd", "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "k_gain": w.k_gain, "layout": "BHNd",
                   "flops_per_step": flops, "seed": inputs.SEED_BASE + idx,
                   "dout_seed": inputs.SEED_BASE + idx + inputs.DOUT_SEED_OFFSET},
        "roofline": {"bound": "mfma", "achieved": round(flops / (avg_ms * 1e-3) / 1e12, 2),
                     "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (avg_ms * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 4),
                     "traffic": None, "timed_unit": "one fmha_bwd call (3 kernels)",
                     "call_ms_avg": round(avg_ms, 4), "call_ms_median": round(float(np.median(call_ms)), 4),
                     "call_ms_min": round(min(call_ms), 4),
                     "kernel_digest": bwd_digest()},
    }
    if not args.no_cpu_baseline:
        grads = [x.cpu().numpy() for x in (dq, dk, dv)]
        cb, parity = bwd_cpu_baseline(q, k, v, do, w, scale, grads, args.cpu_seconds)
        result["cpu_baseline"] = cb
        result["parity"] = parity
    print(json.dumps(result), flush=True)
    if "parity" in result and not result["parity"]["pass"]:
        return 1
    return 0


def bench_fp8(args) -> int:
    import torch

    from software_pipelining_fmha_amd import fmha

    names = [w.name for w in inputs.FP8_WORKLOADS]
    name = args.workload if args.workload in names else "fp8_" + args.workload
    if name not in names:
        print("no FP8 workload named %s (have %s)" % (args.workload, ", ".join(names)), file=sys.stderr)
        return 2
    idx = names.index(name)
    w = inputs.FP8_WORKLOADS[idx]
    dev = torch.device("cuda:0")
    (q8, k8, v8), sc, scale = inputs.fp8_workload_inputs(idx)
    tq, tk, tv = (torch.from_numpy(x).to(dev) for x in (q8, k8, v8))
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float16, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        fmha.forward_fp8(tq, tk, tv, sc, causal=w.causal, scale=float(scale), out=o, lse=lse,
                         stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s_.elapsed_time(e) for s_, e in zip(starts, ends)]
    avg_ms = float(np.mean(launch_ms))
    ms_per_step = wall * 1e3 / args.steps
    achieved = w.flops / (avg_ms * 1e-3) / 1e12
    result = {
        "metric": "FMHA fwd TFLOPS (fp8 e4m3, %s) and %% of MFMA peak" % w.name,
        "value": round(w.flops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "k_gain": w.k_gain, "layout": "BHNd", "flops_per_step": w.flops,
                   "seed": inputs.SEED_BASE + inputs.FP8_SEED_OFFSET + idx,
                   "descales": [float(x) for x in sc]},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": None,
                     "kernel_ms_avg": round(avg_ms, 4), "kernel_ms_median": round(float(np.median(launch_ms)), 4),
                     "kernel_ms_min": round(min(launch_ms), 4),
                     "kernel_digest": fp8_digest()},
    }
    if not args.no_cpu_baseline:
        import oracle

        threads = cpu_threads()
        rows = inputs.fp8_workload_rows(idx) if w.sampled_rows else inputs.sample_rows(
            w.B, w.H, w.N, 256, 4545 + idx)
        t1 = time.perf_counter()
        ref = oracle.fmha_fp8_rows(q8, k8, v8, sc, rows, causal=w.causal, scale=scale,
                                   threads=threads, rss=True)
        dt = time.perf_counter() - t1
        b, h, i = rows.T
        og = o.cpu().numpy()[b, h, i].astype(np.float64)
        lg = lse.cpu().numpy()[b, h, i].astype(np.float64)
        e = 2.0 ** -11
        bar_o = 7 * ref[2] + e * ref[4] + 2.0 ** -10 * np.abs(ref[0]) + 2.0 ** -16
        bar_l = 7 * ref[3] + e * ref[5] + 2.0 ** -20 * np.abs(ref[1]) + 2.0 ** -16
        worst = max(float((np.abs(og - ref[0]) / bar_o).max()), float((np.abs(lg - ref[1]) / bar_l).max()))
        vis = (rows[:, 2] + 1).astype(np.float64) if w.causal else np.full(len(rows), float(w.N))
        result["cpu_baseline"] = {
            "value": float((4.0 * w.d * vis).sum()) / dt / 1e12, "unit": "TFLOPS", "cores": threads,
            "kind": "oracle",
            "sample": "%d seeded (b,h,i) rows of %s with tolerance scales; %.1f s wall" % (len(rows), w.name, dt)}
        result["parity"] = {"rows": int(len(rows)), "max_err_over_bar": worst, "pass": bool(worst <= 1.0)}
    print(json.dumps(result), flush=True)
    if "parity" in result and not result["parity"]["pass"]:
        return 1
    return 0


def _gemm_time(torch, fn, stream, reps: int):
    """Median and all HIP-event times (ms) of `reps` launches of fn()."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for s_, e in ev:
        s_.record(stream)
        fn()
        e.record(stream)
    torch.cuda.synchronize()
    ts = [s_.elapsed_time(e) for s_, e in ev]
    return float(np.median(ts)), ts


def bench_gemm(args) -> int:
    """The warp-specialised GEMM at one workload: C = A B, fp16, timed per
    launch with HIP events on the launch stream."""
    import torch

    from software_pipelining_fmha_amd import ws_gemm

    names = [w.name for w in inputs.GEMM_WORKLOADS]
    name = args.workload if args.workload in names else inputs.GEMM_WORKLOADS[inputs.GEMM_HEADLINE].name
    idx = names.index(name)
    w = inputs.GEMM_WORKLOADS[idx]
    dev = torch.device("cuda:0")
    a, b = inputs.gemm_workload_inputs(idx)
    ta, tb = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    c = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    cfg = tuple(int(x) for x in args.gemm_config.split(",")) if args.gemm_config else \
        ws_gemm.choose(w.M, w.N, w.K)
    stream = torch.cuda.current_stream(dev)
    flops = 2.0 * w.M * w.N * w.K

    def step():
        ws_gemm.gemm(ta, tb, out=c, config=cfg, status=status, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # whole-job rate: K launches back to back, synchronised on both sides
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-launch kernel time (HIP events on the launch stream) for the roofline
    med, ts = _gemm_time(torch, step, stream, args.steps)
    if int(status.item()) != 0:
        print("a semaphore wait gave up", file=sys.stderr)
        return 1
    avg_ms = float(np.mean(ts))
    ms_per_step = wall * 1e3 / args.steps
    achieved = flops / (avg_ms * 1e-3) / 1e12
    # context: the library GEMM on the same operands (hipBLASLt through torch)
    lib_ms, _ = _gemm_time(torch, lambda: torch.matmul(ta, tb), stream, max(5, args.steps // 2))
    result = {
        "metric": "WS GEMM TFLOPS (fp16, %s) and %% of MFMA peak" % w.name,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "tile": list(cfg[:3]),
                   "ring": cfg[3], "chosen_by": "explicit" if args.gemm_config else "model",
                   "flops_per_step": flops, "seed": inputs.GEMM_SEED_BASE + idx},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                     "traffic": None, "kernel_ms_avg": round(avg_ms, 4),
                     "kernel_ms_min": round(min(ts), 4), "kernel_digest": gemm_digest()},
        "context": {"torch_matmul_tflops": round(flops / (lib_ms * 1e-3) / 1e12, 2)},
    }
    if not args.no_cpu_baseline:
        import oracle

        threads = cpu_threads()
        rows = inputs.gemm_sample_rows(w.M, cfg[0], 96 if w.M > 2048 else w.M, seed=idx)
        t1 = time.perf_counter()
        ref, cabs = oracle.gemm_rows(a, b, rows, threads=threads, magnitude=True)
        dt = time.perf_counter() - t1
        got = c.cpu().numpy()[rows].astype(np.float64)
        bar = 2.0 ** -11 * np.abs(ref) + (w.K + 2) * 2.0 ** -24 * cabs + 2.0 ** -24
        worst = float((np.abs(got - ref) / bar).max())
        result["cpu_baseline"] = {
            "value": 2.0 * len(rows) * w.N * w.K / dt / 1e12, "unit": "TFLOPS", "cores": threads,
            "kind": "oracle",
            "sample": "%d rows of C (tile edges first) of %s; %.1f s wall" % (len(rows), w.name, dt)}
        result["parity"] = {"rows": int(len(rows)), "max_err_over_bar": worst, "pass": bool(worst <= 1.0)}
    print(json.dumps(result), flush=True)
    if "parity" in result and not result["parity"]["pass"]:
        return 1
    return 0


def bench_wsmodel(args) -> int:
    """The analytic model of the warp-specialised GEMM on this GPU: two-point
    calibration from the kernel's own stage trace, then predicted against
    measured launch time over the page's problem space (M, N, K in {256,
    512, 1024}, T_M, T_N, T_K in {64, 128}, every compiled ring depth), and
    the chooser's pick against the measured best per problem."""
    import itertools

    import torch

    from software_pipelining_fmha_amd import ws_gemm

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    tick_us = 0.01  # wall_clock64 runs at 100 MHz

    def operands(M, N, K, seed):
        a, b = inputs.draw_gemm(M, N, K, seed)
        return (torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev),
                torch.empty((M, N), dtype=torch.float16, device=dev))

    # ---- calibration: ring depth 1, so a stage's loads and MATH never overlap
    calib = {}
    for cfg, (M, N, K) in (((64, 64, 64, 1), (1024, 1024, 1024)),
                           ((128, 128, 128, 1), (2048, 2048, 1024))):
        ta, tb, c = operands(M, N, K, 8000 + cfg[0])
        S = -(-K // cfg[2])
        tiles = (M // cfg[0]) * (N // cfg[1])
        trace = torch.zeros(ws_gemm.trace_words(M, N, K, *cfg[:3]), dtype=torch.int64, device=dev)
        for _ in range(3):
            ws_gemm.gemm(ta, tb, out=c, config=cfg, trace=trace, stream=stream)
        med, _ = _gemm_time(torch, lambda: ws_gemm.gemm(ta, tb, out=c, config=cfg, trace=trace,
                                                        stream=stream), stream, 5)
        t = trace.cpu().numpy().reshape(tiles, S + 1, 5).astype(np.float64) * tick_us
        st = t[:, :S, :]
        span = t[:, S, 1].max() - t[:, S, 0].min()
        # A MATH wave's stage span [2]..[4] also holds, before its last
        # MFMAs, the wait for the next stage ([3] release .. next [2]); with
        # one slot that wait is the whole next load, so it is taken out.
        math = st[:, :, 4] - st[:, :, 2]
        math[:, :-1] -= st[:, 1:, 2] - st[:, :-1, 3]
        calib[cfg] = {
            "load": float(np.mean(st[:, :, 1] - st[:, :, 0])),
            "math": float(np.mean(math)),
            "epi": float(np.mean(t[:, S, 1] - st[:, S - 1, 4])),
            "init": float(med * 1e3 - span),
        }
    c1, c2 = calib[(64, 64, 64, 1)], calib[(128, 128, 128, 1)]
    # A and B load together per stage: T_LOAD_A + T_LOAD_B = (T_M T_K + T_K T_N) / thr + 2 lat
    thr, lat2 = ws_gemm.two_point(64 * 64 + 64 * 64, c1["load"], 128 * 128 + 128 * 128, c2["load"])
    cthr, clat = ws_gemm.two_point(64.0 ** 3, c1["math"], 128.0 ** 3, c2["math"])
    p = ws_gemm.ModelParams()
    p.load_throughput, p.load_latency = thr, lat2 / 2
    p.compute_throughput, p.compute_latency = cthr, clat
    p.t_epilogue = (c1["epi"] + c2["epi"]) / 2
    p.t_init = (c1["init"] + c2["init"]) / 2
    p.n_units = cus

    # ---- validation over the page's space
    sizes = (256, 512, 1024)
    cfgs = [c_ for c_ in ws_gemm.configs() if c_[0] in (64, 128)]
    rows, errs, regrets = [], [], []
    for M, N, K in itertools.product(sizes, repeat=3):
        ta, tb, c = operands(M, N, K, 8100 + M + 3 * N + 7 * K)
        meas = {}
        for cfg in cfgs:
            fn = lambda: ws_gemm.gemm(ta, tb, out=c, config=cfg, stream=stream)  # noqa: E731
            for _ in range(2):
                fn()
            med, _ = _gemm_time(torch, fn, stream, 9)
            meas[cfg] = med * 1e3
            pred = ws_gemm.launch_time(p, M, N, K, *cfg)
            errs.append((pred - meas[cfg]) / meas[cfg])
            rows.append((M, N, K) + cfg + (meas[cfg], pred))
        pick = ws_gemm.choose(M, N, K, p)
        regrets.append(meas[pick] / min(meas.values()) - 1.0)
    errs = np.array(errs)
    result = {
        "metric": "WS model mean |prediction error| over the page's GEMM space", "unit": "%",
        "value": round(100 * float(np.mean(np.abs(errs))), 2), "higher_is_better": False,
        "n_gpus": 1, "data": "synthetic",
        "config": {"workload": "M,N,K in {256,512,1024}; T_M,T_N,T_K in {64,128}; rings 1-4",
                   "launches": len(rows)},
        "max_abs_error_pct": round(100 * float(np.max(np.abs(errs))), 2),
        "median_error_pct": round(100 * float(np.median(errs)), 2),
        "within_10pct": round(float(np.mean(np.abs(errs) <= 0.10)), 3),
        "chooser_regret_mean_pct": round(100 * float(np.mean(regrets)), 2),
        "chooser_regret_max_pct": round(100 * float(np.max(regrets)), 2),
        "calibration": {"load_throughput_elem_per_us": thr, "load_latency_us": lat2 / 2,
                        "compute_throughput_mac_per_us": cthr, "compute_latency_us": clat,
                        "t_epilogue_us": p.t_epilogue, "t_init_us": p.t_init, "n_units": cus,
                        "points": {"%dx%dx%d_r%d" % k: v for k, v in calib.items()}},
        "kernel_digest": gemm_digest(),
    }
    if args.model_table:
        with open(args.model_table, "w") as f:
            f.write("M N K T_M T_N T_K ring measured_us predicted_us\n")
            for r in rows:
                f.write("%d %d %d %d %d %d %d %.3f %.3f\n" % r)
    print(json.dumps(result), flush=True)
    return 0


def copy_calibration(mib: int, steps: int) -> int:
    """A plain copy kernel of known size: `steps` launches that each read and
    write mib MiB."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(max(1, steps)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n * 4, "copy_bytes_written_per_launch": n * 4,
                      "launches": max(1, steps)}), flush=True)
    return 0


# Default length of the timed region. A couple of seconds of back-to-back
# launches is long enough for an outside utilisation sampler to see and for
# the per-launch spread to average out; a 60-s run of the FP16 headline held
# the same rate as its first seconds.
TIMED_SECONDS = 2.0
MAX_DEFAULT_STEPS = 4000
# TFLOPS each pass reaches at its headline shape (counted FLOPs), used only to
# size the default step count.
USUAL_TFLOPS = {"fwd": 1200.0, "fp8": 2300.0, "bwd": 800.0}


def _default_steps(args) -> int:
    if args.which == "gemm":
        return 100
    fp8 = args.dtype == "fp8"
    pool = inputs.FP8_WORKLOADS if fp8 else inputs.WORKLOADS
    name = args.workload if (not fp8 or args.workload.startswith("fp8_")) else "fp8_" + args.workload
    w = next((x for x in pool if x.name == name), None)
    if w is None or args.which not in ("fwd", "bwd"):
        return 20
    flops = w.flops * (2.5 if args.which == "bwd" else 1.0)
    rate = USUAL_TFLOPS["fp8" if fp8 else args.which] * 1e12
    return int(min(MAX_DEFAULT_STEPS, max(20, round(TIMED_SECONDS * rate / flops))))


def parse_args(argv=None) -> argparse.Namespace:
    """The command line, with the per-pass default step and warm-up counts
    filled in."""
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: about %.0f s of work at the pass's usual rate, "
                         "20 to %d steps; 100 for --pass gemm)" % (TIMED_SECONDS, MAX_DEFAULT_STEPS))
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default 10; 20 for --dtype fp8, 50 for --pass gemm, "
                         "5 for --pass bwd)")
    ap.add_argument("--workload", default=inputs.WORKLOADS[inputs.HEADLINE].name,
                    choices=[w.name for w in inputs.WORKLOADS] + [w.name for w in inputs.FP8_WORKLOADS]
                    + [w.name for w in inputs.GEMM_WORKLOADS])
    ap.add_argument("--dtype", choices=["f16", "fp8"], default="f16",
                    help="f16 (default) or the FP8 (E4M3) forward pass")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd", "gemm", "wsmodel"],
                    default="fwd",
                    help="time the attention forward pass (default) or backward pass, the "
                         "warp-specialised GEMM, or validate the GEMM's analytic model")
    ap.add_argument("--gemm-config", default="",
                    help="T_M,T_N,T_K,ring for --pass gemm (default: the model's pick)")
    ap.add_argument("--model-table", default="",
                    help="--pass wsmodel: also write every measured/predicted launch here")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of attention, run a plain device copy of this many MiB "
                         "per step (calibrates rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args(argv)
    # The clocks ramp over the first launches: about 50 ms for the GEMM and
    # the FP8 forward (which run below the power limit), a few launches for
    # the FP16 forward. The default warm-up covers the ramp, so that the
    # timed steps see the steady state.
    if args.steps is None:
        args.steps = _default_steps(args)
    if args.warmup is None:
        if args.which == "gemm":
            args.warmup = 50
        elif args.which == "bwd":
            args.warmup = 5
        elif args.dtype == "fp8":
            args.warmup = 20
        else:
            args.warmup = 10
    return args


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the attention forward pass here is a "
              "single-GPU kernel with no cross-GPU path (asked for --gpus %d)" % args.gpus,
              file=sys.stderr)
        return 2

    import torch

    if args.copy_mib:
        return copy_calibration(args.copy_mib, args.steps)

    from software_pipelining_fmha_amd import fmha

    fmha.lib()  # fail loudly before any work if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.which == "gemm":
        return bench_gemm(args)
    if args.which == "wsmodel":
        return bench_wsmodel(args)
    if args.dtype == "fp8":
        if args.which != "fwd":
            print("the FP8 path is forward only", file=sys.stderr)
            return 2
        return bench_fp8(args)
    w = next(x for x in inputs.WORKLOADS if x.name == args.workload)
    idx = inputs.WORKLOADS.index(w)
    q, k, v, scale = inputs.workload_inputs(idx)
    tq, tk, tv = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    o = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.which == "bwd":
        return bench_bwd(args, w, idx, q, k, v, scale, tq, tk, tv, dev, stream)

    def step():
        fmha.forward(tq, tk, tv, causal=w.causal, scale=float(scale), out=o, lse=lse,
                     stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_ms = float(np.mean(launch_ms))
    ms_per_step = wall * 1e3 / args.steps
    value = w.flops / (ms_per_step * 1e-3) / 1e12
    achieved = w.flops / (avg_ms * 1e-3) / 1e12

    result = {
        "metric": METRIC if idx == inputs.HEADLINE else
        "FMHA fwd TFLOPS (fp16, %s) and %% of MFMA peak" % w.name, "value": round(value, 2), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "k_gain": w.k_gain, "layout": "BHNd",
                   "flops_per_step": w.flops, "seed": inputs.SEED_BASE + idx},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                     "traffic": recorded_traffic(w.name),
                     "counters": recorded_mfma_utilisation(w.name),
                     "kernel_ms_avg": round(avg_ms, 4), "kernel_ms_median": round(float(np.median(launch_ms)), 4),
                     "kernel_ms_min": round(min(launch_ms), 4),
                     "kernel_digest": kernel_digest()},
    }
    if not args.no_cpu_baseline:
        o_host, lse_host = o.cpu().numpy(), lse.cpu().numpy()
        try:
            cb, parity = cpu_baseline(q, k, v, w, scale, o_host, lse_host, args.cpu_seconds)
            cb.pop("seconds")
        except Exception as e:  # the GPU measurement stands; the line says why the CPU leg is missing
            cb = {"value": None, "unit": "TFLOPS", "kind": "oracle", "error": "%s: %s" % (type(e).__name__, e)}
            parity = {"pass": None, "error": "the CPU oracle did not run"}
        result["cpu_baseline"] = cb
        result["parity"] = parity
    print(json.dumps(result), flush=True)
    if "parity" in result and result["parity"]["pass"] is False:
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
