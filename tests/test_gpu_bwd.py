"""Parity of the HIP backward path (fmha_bwd, through the C ABI) with the
CPU oracle's gradients of sum(dO * O).

Bar, per gradient element g with oracle value g_ref (fp64 from the fp16
inputs q, k, v, dO):
    |g - g_ref| <= 8u rss + 2u |g_ref| + c u ds + 2^-16,   u = 2^-11,
with c = 3 for dq, 21 for dk and ds = 0 for dv. The oracle reports, per
element, rss (root-sum-square of the terms summed into it) and ds (how far
the element moves per unit relative error in the forward output O through
D_i = dO_i . O_i). The derivation:
- each term is formed from one fp16-rounded factor (P or dS, relative error
  <= u/2 each, independent from term to term) and the forward's lse (an
  error of order 1e-5 per query row); the sum is fp32 and the result is
  rounded once to fp16 (u/2 relative, inside 2u |g_ref|). By Hoeffding's
  bound, independent errors |e_t| <= u |a_t| sum past 7 u rss with
  probability below 1e-10;
- D_i is formed from the fp16 forward output: |dD_i| <= 3u w_i (rounding of
  O plus the forward's own fp16 weights, each <= u sum_j P_ij |v_j| per
  entry). It moves dq_i by at most 3u ds_q (one direction for all terms)
  and dk_j by a sum of independent per-query shifts, at most 7 * 3u ds_k;
- the floor covers elements whose terms cancel exactly (a single visible
  key gives dS = 0): there the GPU keeps the fp32 residue of dP - D, two
  sums of d fp16 products in different orders, a few 2^-24 times
  sum_c |dO_c v_c| (about 100 here) times scale * |q| < 0.6.
A CPU model of exactly this arithmetic stays below 0.3 of the bar, and a
key tile left out of the sums exceeds it.

The forward outputs o and lse fed to the backward come from the GPU forward
pass (fmha_fwd), as in training.
"""
import math

import numpy as np
import pytest

import oracle
from software_pipelining_fmha_amd import fmha, inputs

pytestmark = pytest.mark.gpu

U = 2.0 ** -11


def torch_mod():
    import torch
    return torch


def to_dev(*arrays):
    torch = torch_mod()
    return [torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0") for a in arrays]


def run_bwd(q, k, v, do, causal, scale, stream=None):
    """fmha_fwd then fmha_bwd on the GPU; gradients start as NaN."""
    torch = torch_mod()
    tq, tk, tv, tdo = to_dev(q, k, v, do)
    o, lse = fmha.forward(tq, tk, tv, causal=causal, scale=float(scale))
    grads = [torch.full_like(tq, float("nan")) for _ in range(3)]
    fmha.backward(tq, tk, tv, o, lse, tdo, causal=causal, scale=float(scale),
                  dq=grads[0], dk=grads[1], dv=grads[2], stream=stream)
    torch.cuda.synchronize()
    return [g.cpu().numpy() for g in grads]


def check(name, got, ref, rss, label, ds=None):
    got = got.astype(np.float64)
    assert np.isfinite(got).all(), "%s %s: non-finite gradient" % (label, name)
    err = np.abs(got - ref)
    tol = 8 * U * rss + 2 * U * np.abs(ref) + 2.0 ** -16
    if ds is not None:
        tol = tol + {"dq": 3, "dk": 21}[name] * U * ds
    worst = np.argmax(err / tol)
    print("%s %s: n=%d max|err|=%.3e max err/tol=%.3f (max|ref|=%.3e)" % (
        label, name, err.size, err.max(), (err / tol).flat[worst], np.abs(ref).max()), flush=True)
    assert (err <= tol).all(), "%s %s: err %.3e > tol %.3e at %d" % (
        label, name, err.flat[worst], tol.flat[worst], worst)


def check_all_rows(q, k, v, do, causal, scale, label):
    dq, dk, dv = run_bwd(q, k, v, do, causal, scale)
    ref = oracle.fmha_bwd_all(q, k, v, do, causal=causal, scale=scale, rss=True)
    check("dq", dq, ref[0], ref[3], label, ref[6])
    check("dk", dk, ref[1], ref[4], label, ref[7])
    check("dv", dv, ref[2], ref[5], label)


SMALL = [(2, 3, n, d, c) for n in (1, 2, 31, 32, 33, 127, 128, 129, 200, 333)
         for d in (64, 128) for c in (False, True)]


@pytest.mark.parametrize("B,H,N,d,causal", SMALL)
def test_small_and_ragged_shapes_every_row(B, H, N, d, causal, device):
    print("bwd small B=%d H=%d N=%d d=%d causal=%d" % (B, H, N, d, causal), flush=True)
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=3000 + 7 * N + d + causal)
    do = inputs.draw_dout(B, H, N, d, seed=4000 + N + d + causal)
    check_all_rows(q, k, v, do, causal, np.float32(1 / math.sqrt(d)), "small")


@pytest.mark.parametrize("d,causal", [(64, False), (64, True), (128, False), (128, True)])
@pytest.mark.parametrize("scale", [0.0, -0.088388, -0.5])
def test_zero_and_negative_scale(scale, d, causal, device):
    """Any finite scale: masks apply after the exponent is scaled, so masked
    keys keep weight 0 for scale <= 0 too (scale = 0 gives dq = dk = 0)."""
    B, H, N = 1, 3, 200
    print("bwd scale=%g d=%d causal=%d" % (scale, d, causal), flush=True)
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=3500 + d + causal)
    do = inputs.draw_dout(B, H, N, d, seed=3600 + d + causal)
    check_all_rows(q, k, v, do, causal, np.float32(scale), "scale %g" % scale)


@pytest.mark.parametrize("idx", [0, 1], ids=[inputs.WORKLOADS[i].name for i in (0, 1)])
def test_workload_every_row(idx, device):
    """The tiny workload, and B4 H32 N1024 d128 on 4 of its 128 heads (each
    head is independent; the oracle's cost grows with the head count)."""
    w = inputs.WORKLOADS[idx]
    print("bwd workload %s" % w.name, flush=True)
    q, k, v, scale = inputs.workload_inputs(idx)
    do = inputs.workload_dout(idx)
    if w.B * w.H > 4:
        sel = np.random.default_rng(idx).choice(w.B * w.H, size=4, replace=False)
        pick = lambda x: x.reshape(w.B * w.H, w.N, w.d)[sel][None]
        q, k, v, do = (np.ascontiguousarray(pick(x)) for x in (q, k, v, do))
    check_all_rows(q, k, v, do, w.causal, scale, w.name)


@pytest.mark.parametrize("idx", [2, 3, 4], ids=[inputs.WORKLOADS[i].name for i in (2, 3, 4)])
def test_workload_sampled_rows(idx, device):
    """Full-size workloads in the launch configuration bench.py times: dq on
    the workload's sampled (b, h, i) rows, dk and dv on 32 sampled key rows
    of each of 2 seeded heads (each such head costs the oracle one forward
    pass over it)."""
    w = inputs.WORKLOADS[idx]
    print("bwd workload %s (sampled)" % w.name, flush=True)
    q, k, v, scale = inputs.workload_inputs(idx)
    do = inputs.workload_dout(idx)
    dq, dk, dv = run_bwd(q, k, v, do, w.causal, scale)
    qrows = inputs.workload_rows(idx)
    rng = np.random.default_rng(idx + 77)
    heads = rng.choice(w.B * w.H, size=2, replace=False)
    keys = [np.sort(np.concatenate([[0, w.N - 1], rng.choice(w.N, size=30, replace=False)]))
            for _ in heads]
    krows = np.array([(hh // w.H, hh % w.H, j) for hh, ks in zip(heads, keys) for j in ks])
    ref = oracle.fmha_bwd_rows(q, k, v, do, qrows, krows, causal=w.causal, scale=scale, rss=True)
    b, h, i = qrows.T
    check("dq", dq[b, h, i], ref[0], ref[3], w.name, ref[6])
    b, h, j = krows.T
    check("dk", dk[b, h, j], ref[1], ref[4], w.name, ref[7])
    check("dv", dv[b, h, j], ref[2], ref[5], w.name)


@pytest.mark.parametrize("causal,k_gain", [(False, 1.0), (True, 3.0)])
def test_head_dim_64_at_full_size(causal, k_gain, device):
    """The d = 64 backward kernels at B4 H32 N4096 (the d = 128 checks' launch
    configuration, at the other head dim): dq on 256 seeded rows, dk and dv
    on 32 key rows of each of 2 seeded heads, including keys 0 and N-1."""
    B, H, N, d = 4, 32, 4096, 64
    print("bwd d=64 full size causal=%d k_gain=%g" % (causal, k_gain), flush=True)
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=6500 + causal, k_gain=k_gain)
    do = inputs.draw_dout(B, H, N, d, seed=6600 + causal)
    scale = np.float32(1 / math.sqrt(d))
    dq, dk, dv = run_bwd(q, k, v, do, causal, scale)
    qrows = inputs.sample_rows(B, H, N, 256, seed=66 + causal)
    rng = np.random.default_rng(67 + causal)
    heads = rng.choice(B * H, size=2, replace=False)
    keys = [np.sort(np.concatenate([[0, N - 1], rng.choice(np.arange(1, N - 1), size=30, replace=False)]))
            for _ in heads]
    krows = np.array([(hh // H, hh % H, j) for hh, ks in zip(heads, keys) for j in ks])
    ref = oracle.fmha_bwd_rows(q, k, v, do, qrows, krows, causal=causal, scale=scale, rss=True)
    b, h, i = qrows.T
    check("dq", dq[b, h, i], ref[0], ref[3], "d=64 full size", ref[6])
    b, h, j = krows.T
    check("dk", dk[b, h, j], ref[1], ref[4], "d=64 full size", ref[7])
    check("dv", dv[b, h, j], ref[2], ref[5], "d=64 full size")


@pytest.mark.parametrize("causal", [False, True])
def test_full_size_key_and_value_gradient_sums(causal, device):
    """Every row of a full-size problem (B4 H32 N8192 d128): per head
    sum_j dk_j = 0 and sum_j dv_j = sum_i dO_i (the weights of each query sum
    to 1). Both sums are taken over the fp16 outputs in fp64; the bound is
    the fp16 rounding of each summed element plus the relative error bar
    above, scaled by sum_j |g_j|."""
    B, H, N, d = 4, 32, 8192, 128
    print("bwd gradient sums N=%d causal=%d" % (N, causal), flush=True)
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=5150 + causal)
    do = inputs.draw_dout(B, H, N, d, seed=5250 + causal)
    _, dk, dv = run_bwd(q, k, v, do, causal, np.float32(1 / math.sqrt(d)))
    dk, dv = dk.astype(np.float64), dv.astype(np.float64)
    sk = np.abs(dk.sum(axis=2))
    sv = np.abs(dv.sum(axis=2) - do.astype(np.float64).sum(axis=2))
    bk = 4 * U * np.abs(dk).sum(axis=2) + 1e-6
    bv = 4 * U * np.abs(dv).sum(axis=2) + 1e-6
    print("max |sum dk| / bound = %.3f, max |sum dv - sum dO| / bound = %.3f" % (
        (sk / bk).max(), (sv / bv).max()), flush=True)
    assert (sk <= bk).all() and (sv <= bv).all()


@pytest.mark.parametrize("causal", [True, False])
def test_deterministic_bitwise(causal, device):
    q, k, v = inputs.draw_qkv(2, 4, 1000, 128, seed=61)
    do = inputs.draw_dout(2, 4, 1000, 128, seed=62)
    a = run_bwd(q, k, v, do, causal, np.float32(0.088388))
    b = run_bwd(q, k, v, do, causal, np.float32(0.088388))
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint16), y.view(np.uint16))


def test_causal_workload_repeats_bitwise(device):
    """Three backward passes of the causal K x3 workload (B4 H32 N8192) give
    the same bits: a read of a ring slot before every wave's share of its
    LDS-DMA has landed, or any other race between waves, would show here as
    run-to-run differences."""
    idx = [i for i, w in enumerate(inputs.WORKLOADS) if w.causal][0]
    q, k, v, scale = inputs.workload_inputs(idx)
    do = inputs.workload_dout(idx)
    a = run_bwd(q, k, v, do, True, scale)
    for _ in range(2):
        b = run_bwd(q, k, v, do, True, scale)
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint16), y.view(np.uint16))


def test_non_default_stream(device):
    torch = torch_mod()
    q, k, v = inputs.draw_qkv(1, 2, 300, 64, seed=63)
    do = inputs.draw_dout(1, 2, 300, 64, seed=64)
    ref = run_bwd(q, k, v, do, False, np.float32(0.125))
    got = run_bwd(q, k, v, do, False, np.float32(0.125), stream=torch.cuda.Stream())
    for x, y in zip(ref, got):
        assert np.array_equal(x.view(np.uint16), y.view(np.uint16))


def test_guard_bands_untouched(device):
    """dq, dk, dv and the workspace are written only inside their extents."""
    torch = torch_mod()
    B, H, N, d = 1, 2, 333, 128
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=65)
    do = inputs.draw_dout(B, H, N, d, seed=66)
    tq, tk, tv, tdo = to_dev(q, k, v, do)
    o, lse = fmha.forward(tq, tk, tv, causal=True)
    pad, n = 4096, B * H * N * d
    bufs = [torch.full((n + 2 * pad,), 1234.0, dtype=torch.float16, device="cuda:0") for _ in range(3)]
    wsb = torch.full((2 * B * H * N + 2 * pad,), -55.0, dtype=torch.float32, device="cuda:0")
    views = [x[pad:pad + n].view(B, H, N, d) for x in bufs]
    fmha.backward(tq, tk, tv, o, lse, tdo, causal=True, dq=views[0], dk=views[1], dv=views[2],
                  workspace=wsb[pad:pad + 2 * B * H * N])
    torch.cuda.synchronize()
    for x in bufs:
        c = x.cpu().numpy()
        assert (c[:pad] == np.float16(1234.0)).all() and (c[-pad:] == np.float16(1234.0)).all()
        assert np.isfinite(c[pad:-pad]).all()
    w = wsb.cpu().numpy()
    assert (w[:pad] == -55.0).all() and (w[-pad:] == -55.0).all()


def test_workspace_holds_row_dot_products(device):
    """On return the workspace's first B*H*N values are D_i = dO_i . O_i."""
    torch = torch_mod()
    q, k, v = inputs.draw_qkv(1, 2, 200, 64, seed=67)
    do = inputs.draw_dout(1, 2, 200, 64, seed=68)
    tq, tk, tv, tdo = to_dev(q, k, v, do)
    o, lse = fmha.forward(tq, tk, tv)
    ws = torch.empty((2 * 400,), dtype=torch.float32, device="cuda:0")
    fmha.backward(tq, tk, tv, o, lse, tdo, workspace=ws)
    torch.cuda.synchronize()
    ref = (o.double().cpu() * tdo.double().cpu()).sum(-1).numpy().ravel()
    np.testing.assert_allclose(ws[:400].cpu().numpy(), ref, rtol=1e-5, atol=1e-5)


def test_empty_problem_launches_nothing(device):
    torch = torch_mod()
    q = torch.empty((0, 2, 16, 64), dtype=torch.float16, device="cuda:0")
    lse = torch.empty((0, 2, 16), dtype=torch.float32, device="cuda:0")
    dq, dk, dv = fmha.backward(q, q.clone(), q.clone(), q.clone(), lse, q.clone())
    torch.cuda.synchronize()
    assert dq.numel() == 0
