"""Parity of the warp-specialised GEMM (ws_gemm, through the C ABI) with the
CPU oracle C = A x B in fp64.

Bar, per element: |C - C_ref| <= 2^-11 |C_ref| + (K + 2) 2^-24 Cabs + 2^-24,
with Cabs = sum_k |A[m][k] B[k][n]| from the oracle. Products of binary16
values are exact in fp32; any order of K fp32 additions errs by at most
about K 2^-24 Cabs; the final rounding to binary16 adds at most 2^-11 of
the value, or 2^-25 below the normal range.

Also checked: every compiled variant on a ragged shape, the page's problem
sizes, sampled rows (the first and last row of every tile) at M = N = K =
8192, zero K, determinism across ring depths, the status word, and the
ordering constraints in the per-stage trace that the semaphores enforce.
"""
import numpy as np
import pytest

import oracle
from software_pipelining_fmha_amd import inputs, ws_gemm

pytestmark = pytest.mark.gpu


def run(a, b, config=(0, 0, 0, 0), trace_words=0):
    import torch
    ta = torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    tb = torch.from_numpy(np.ascontiguousarray(b)).to("cuda:0")
    M, N = a.shape[0], b.shape[1]
    c = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    trace = torch.zeros(trace_words, dtype=torch.int64, device="cuda:0") if trace_words else None
    ws_gemm.gemm(ta, tb, out=c, config=config, trace=trace, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "a semaphore wait gave up"
    out = c.cpu().numpy()
    return (out, trace.cpu().numpy()) if trace_words else out


def check(c, a, b, rows, label):
    ref, cabs = oracle.gemm_rows(a, b, rows, magnitude=True)
    got = c[rows].astype(np.float64)
    assert np.isfinite(got).all(), label + ": unwritten or non-finite output"
    K = a.shape[1]
    bar = 2.0 ** -11 * np.abs(ref) + (K + 2) * 2.0 ** -24 * cabs + 2.0 ** -24
    err = np.abs(got - ref)
    print("%s: rows=%d max|dC|=%.3e err/bar %.3f" % (label, len(rows), err.max(),
                                                     (err / bar).max()), flush=True)
    assert (err <= bar).all(), "%s: error above the bar" % label


@pytest.mark.parametrize("cfg", ws_gemm.configs(), ids=lambda c: "t%dx%dx%d_r%d" % c)
def test_every_variant_ragged_shape(cfg, device):
    M, N, K = 200, 136, 264
    print("gemm variant %s M=%d N=%d K=%d" % (cfg, M, N, K), flush=True)
    a, b = inputs.draw_gemm(M, N, K, seed=7000 + sum(cfg))
    c = run(a, b, cfg)
    check(c, a, b, np.arange(M), "variant %s" % (cfg,))


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (512, 1024, 256), (1024, 512, 1024),
                                   (1024, 1024, 1024)])
@pytest.mark.parametrize("cfg", [(64, 64, 64, 2), (128, 64, 128, 2), (128, 128, 64, 3),
                                 (128, 128, 128, 2)], ids=lambda c: "t%dx%dx%d_r%d" % c)
def test_page_problem_sizes(M, N, K, cfg, device):
    print("gemm %s M=%d N=%d K=%d" % (cfg, M, N, K), flush=True)
    a, b = inputs.draw_gemm(M, N, K, seed=7100 + M + 3 * N + 7 * K)
    c = run(a, b, cfg)
    check(c, a, b, np.arange(M), "page size")


@pytest.mark.parametrize("idx", range(len(inputs.GEMM_WORKLOADS)),
                         ids=[w.name for w in inputs.GEMM_WORKLOADS])
def test_gemm_workload_parity(idx, device):
    """The model's own pick (all-zero config), as the bench runs it."""
    w = inputs.GEMM_WORKLOADS[idx]
    print("gemm workload %s" % w.name, flush=True)
    a, b = inputs.gemm_workload_inputs(idx)
    cfg = ws_gemm.choose(w.M, w.N, w.K)
    c = run(a, b)
    assert not np.isnan(c).any(), "unwritten output"
    rows = inputs.gemm_sample_rows(w.M, cfg[0], 128, seed=idx) if w.M > 1024 else np.arange(w.M)
    check(c, a, b, rows, "%s %s" % (w.name, cfg))


def test_large_tile_edges_every_column(device):
    """M = N = K = 4096 with the largest tile: rows at both edges of every
    tile row, all columns (every tile column and its edges)."""
    M = N = K = 4096
    cfg = (256, 128, 64, 3)
    a, b = inputs.draw_gemm(M, N, K, seed=7300)
    c = run(a, b, cfg)
    assert not np.isnan(c).any()
    rows = inputs.gemm_sample_rows(M, cfg[0], 40, seed=5)
    check(c, a, b, rows, "4096 tile edges")


def test_zero_k_writes_zeros(device):
    a = np.zeros((100, 0), np.float16)
    b = np.zeros((0, 64), np.float16)
    c = run(a, b, (128, 64, 64, 2))
    assert (c == 0).all()


@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (3, 8, 520), (300, 8, 8)])
def test_degenerate_shapes(M, N, K, device):
    a, b = inputs.draw_gemm(M, N, K, seed=7400 + M + N + K)
    for cfg in [(64, 64, 64, 1), (256, 128, 64, 3), (128, 128, 128, 2)]:
        c = run(a, b, cfg)
        check(c, a, b, np.arange(M), "degenerate %dx%dx%d %s" % (M, N, K, cfg))


def test_ring_depth_does_not_change_bits(device):
    """The ring only changes when stages load, not the order of the sums."""
    a, b = inputs.draw_gemm(384, 256, 1024, seed=7500)
    outs = [run(a, b, (128, 128, 64, r)).view(np.uint16) for r in (1, 2, 3, 4)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    again = run(a, b, (128, 128, 64, 2)).view(np.uint16)
    assert np.array_equal(again, outs[0])


@pytest.mark.parametrize("cfg", [(128, 128, 64, 1), (128, 128, 64, 3), (64, 64, 128, 2),
                                 (128, 128, 128, 2)], ids=lambda c: "t%dx%dx%d_r%d" % c)
def test_trace_obeys_the_semaphores(cfg, device):
    """Per workgroup and stage i: DMA wave 0 issues a stage before it
    lands, MATH wave 0 starts it after it landed, releases it after it
    started and finishes its MFMAs after that; stage i is issued only after
    stage i - ring was released (by MATH wave 0 at least)."""
    M, N, K = 512, 512, 1024
    tm, tn, tk, ring = cfg
    S = -(-K // tk)
    words = ws_gemm.trace_words(M, N, K, tm, tn, tk)
    a, b = inputs.draw_gemm(M, N, K, seed=7600)
    c, tr = run(a, b, cfg, trace_words=words)
    check(c, a, b, np.arange(0, M, 7), "traced %s" % (cfg,))
    tiles = (M // tm) * (N // tn)
    t = tr.reshape(tiles, S + 1, 5)
    st = t[:, :S, :]
    assert (st > 0).all()
    assert (st[:, :, 1] >= st[:, :, 0]).all()   # landed after issued
    assert (st[:, :, 2] >= st[:, :, 1]).all()   # MATH starts after landed
    assert (st[:, :, 3] >= st[:, :, 2]).all()   # released after started
    assert (st[:, :, 4] >= st[:, :, 3]).all()   # MFMAs end after the release
    assert (st[:, 1:, 2] >= st[:, :-1, 3]).all()  # next stage starts after this release
    if S > ring:
        assert (st[:, ring:, 0] >= st[:, :-ring, 3]).all()  # slot reuse waits for release
    assert (t[:, S, 1] >= st[:, S - 1, 3]).all()
    assert sorted(t[:, S, 2].tolist()) == list(range(tiles))


def test_model_choice_runs_and_matches_explicit(device):
    M, N, K = 1024, 768, 512
    a, b = inputs.draw_gemm(M, N, K, seed=7700)
    cfg = ws_gemm.choose(M, N, K)
    auto = run(a, b)
    explicit = run(a, b, cfg)
    assert np.array_equal(auto.view(np.uint16), explicit.view(np.uint16))
