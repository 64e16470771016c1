"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar: max |O - O_oracle| <= 2e-3 and max |lse - lse_oracle| <= 1e-3, for
fp16 inputs, on every checked row.

Workloads: FP16, batch 4, 32 heads, head dim 128, sequence lengths 1K-16K.
Twill, section 6.2, and Tawa, section V-D, evaluate this shape. Inputs are
seeded i.i.d. N(0,1) draws. Small shapes are compared on every row. At full
size the test compares the sampled rows the oracle computes one by one. A
uniform-key property holds at any size and checks every row's O and lse in
closed form.
"""
import math

import numpy as np
import pytest

import oracle
from software_pipelining_fmha_amd import fmha, inputs

pytestmark = pytest.mark.gpu

TOL_O = 2e-3
TOL_LSE = 1e-3


def torch_mod():
    import torch
    return torch


def to_dev(*arrays):
    torch = torch_mod()
    return [torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0") for a in arrays]


def run(q, k, v, causal, scale, fill_nan=True, stream=None):
    """fmha_fwd on the GPU. Outputs start as NaN so unwritten rows show."""
    torch = torch_mod()
    tq, tk, tv = to_dev(q, k, v)
    B, H, N, d = q.shape
    o = torch.full((B, H, N, d), float("nan") if fill_nan else 0.0, dtype=torch.float16,
                   device="cuda:0")
    lse = torch.full((B, H, N), float("nan") if fill_nan else 0.0, dtype=torch.float32,
                     device="cuda:0")
    fmha.forward(tq, tk, tv, causal=causal, scale=float(scale), out=o, lse=lse, stream=stream)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def check_rows(o_gpu, lse_gpu, rows, o_ref, lse_ref, label):
    b, h, i = rows[:, 0], rows[:, 1], rows[:, 2]
    og = o_gpu[b, h, i].astype(np.float64)
    lg = lse_gpu[b, h, i].astype(np.float64)
    assert np.isfinite(og).all() and np.isfinite(lg).all(), label + ": non-finite output"
    eo = np.abs(og - o_ref).max()
    el = np.abs(lg - lse_ref).max()
    print("%s: rows=%d max|dO|=%.3e max|dlse|=%.3e" % (label, len(rows), eo, el), flush=True)
    assert eo <= TOL_O, "%s: O error %.3e" % (label, eo)
    assert el <= TOL_LSE, "%s: lse error %.3e" % (label, el)


@pytest.mark.parametrize("idx", range(len(inputs.WORKLOADS)),
                         ids=[w.name for w in inputs.WORKLOADS])
def test_workload_parity(idx, device):
    w = inputs.WORKLOADS[idx]
    print("workload %s" % w.name, flush=True)
    q, k, v, scale = inputs.workload_inputs(idx)
    o, lse = run(q, k, v, w.causal, scale)
    assert not np.isnan(o).any() and not np.isnan(lse).any(), "unwritten or NaN output"
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = inputs.workload_rows(idx)
    o_ref, lse_ref = oracle.fmha_rows(q, k, v, rows, causal=w.causal, scale=scale)
    check_rows(o, lse, rows, o_ref, lse_ref, w.name)


RAGGED = [(2, 3, n, d, c) for n in (1, 2, 63, 65, 127, 129, 200, 333) for d in (64, 128)
          for c in (False, True)]


@pytest.mark.parametrize("B,H,N,d,causal", RAGGED)
def test_ragged_and_small_shapes(B, H, N, d, causal, device):
    print("ragged B=%d H=%d N=%d d=%d causal=%d" % (B, H, N, d, causal), flush=True)
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=1000 + N * 7 + d + causal)
    scale = np.float32(1 / math.sqrt(d))
    o, lse = run(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.fmha_all(q, k, v, causal=causal, scale=scale)
    rows = np.argwhere(np.ones((B, H, N), bool))
    check_rows(o, lse, rows, o_ref.reshape(-1, d), lse_ref.reshape(-1), "ragged")


@pytest.mark.parametrize("N,causal", [(16384, False), (8192, True)])
def test_full_size_uniform_keys_every_row(N, causal, device):
    """With every key row equal, O_i is the mean of the visible value rows and
    lse_i = scale*q_i.u + ln|J_i|. Every (b, h, i) row of the full-size
    workload is checked. Outputs start as NaN, so a tile the grid misses
    would fail."""
    B, H, d = 4, 32, 128
    print("uniform-K full size N=%d causal=%d" % (N, causal), flush=True)
    q, _, v = inputs.draw_qkv(B, H, N, d, seed=777 + N)
    u = np.random.default_rng(5).standard_normal((B, H, 1, d)).astype(np.float16)
    k = np.ascontiguousarray(np.broadcast_to(u, (B, H, N, d)))
    scale = np.float32(1 / math.sqrt(d))
    o, lse = run(q, k, v, causal, scale)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    s = float(scale) * np.einsum("bhnd,bhd->bhn", q.astype(np.float64), u[:, :, 0].astype(np.float64))
    if causal:
        cnt = np.arange(1, N + 1, dtype=np.float64)
        mean = np.cumsum(v.astype(np.float64), axis=2) / cnt[None, None, :, None]
        lse_ref = s + np.log(cnt)[None, None, :]
    else:
        mean = np.broadcast_to(v.astype(np.float64).mean(axis=2, keepdims=True), v.shape)
        lse_ref = s + math.log(N)
    eo = np.abs(o.astype(np.float64) - mean).max()
    el = np.abs(lse.astype(np.float64) - lse_ref).max()
    print("uniform-K: max|dO|=%.3e max|dlse|=%.3e" % (eo, el), flush=True)
    assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.parametrize("d,causal", [(64, False), (128, False), (64, True), (128, True)])
def test_late_scores_far_above_first_key_tile(d, causal, device):
    """For one block of query rows, the best key past the first 64 scores
    more than 2^28 above every key of the first 64. A weight formed against
    the first tile's row max overflows fp16 there, so these rows take the
    running-max path; the other rows of their workgroup are recomputed with
    them. Every row is compared with the oracle."""
    B, H, N = 1, 2, 700
    print("late large scores d=%d causal=%d" % (d, causal), flush=True)
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=31 + d + causal)
    q[:, 0, 300:340, 7] = 16
    k[:, 0, 64:, 7] = 16
    scale = np.float32(1 / math.sqrt(d))
    o, lse = run(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.fmha_all(q, k, v, causal=causal, scale=scale)
    s = float(scale) * np.einsum("nd,md->nm", q[0, 0, 300:340].astype(np.float64),
                                 k[0, 0].astype(np.float64))
    gap = (s[:, 64:].max(axis=1) - s[:, :64].max(axis=1)) / math.log(2)
    assert gap.min() > 17, "inputs do not reach the overflow case"
    rows = np.argwhere(np.ones((B, H, N), bool))
    check_rows(o, lse, rows, o_ref.reshape(-1, d), lse_ref.reshape(-1), "late-large")


@pytest.mark.parametrize("d", [64, 128])
def test_overflow_rerun_with_many_tiles(d, device):
    """More query tiles than compute units, so each workgroup runs several
    and stages the next tile's Q while finishing the current one. Rows
    500..539 of every head in batch 0 overflow the fast pass (a late key
    2^28 above the first key tile), so their tiles rerun exactly; the rerun
    refills the K ring that held the staged Q, and the next tile must still
    see its own Q. The overflow rows and both edges of every tile match the
    oracle."""
    torch = torch_mod()
    B, H, N = 3, 31, 1000
    bm = fmha.fmha_query_tile(d)
    tiles = B * H * (-(-N // bm))
    assert tiles > torch.cuda.get_device_properties(0).multi_processor_count
    print("overflow rerun, many tiles d=%d tiles=%d" % (d, tiles), flush=True)
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=1900 + d)
    q[0, :, 500:540, 7] = 16
    k[0, :, 64:, 7] = 16
    scale = np.float32(1 / math.sqrt(d))
    o, lse = run(q, k, v, False, scale)
    assert not np.isnan(o).any() and not np.isnan(lse).any(), "unwritten output"
    rows = list(map(tuple, tile_edge_rows(B, H, N, bm, seed=1900 + d)))
    rows += [(0, h, i) for h in (0, 17, 30) for i in (500, 519, 539)]
    rows = np.array(rows, dtype=np.int64)
    o_ref, lse_ref = oracle.fmha_rows(q, k, v, rows, causal=False, scale=scale)
    check_rows(o, lse, rows, o_ref, lse_ref, "overflow rerun, many tiles")


@pytest.mark.parametrize("d", [64, 128])
def test_late_scores_just_inside_fp16_weights(d, device):
    """Keys past the first tile score 2^13 to 2^15 above the first tile's
    max: the weights stay finite but reach thousands, with no rescale."""
    B, H, N = 1, 1, 640
    print("late scores inside fp16 d=%d" % d, flush=True)
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=57 + d)
    q = (q.astype(np.float32) * 0.05).astype(np.float16)
    k = (k.astype(np.float32) * 0.05).astype(np.float16)
    scale = np.float32(1 / math.sqrt(d))
    target = 14.0 * math.log(2)  # natural-log gap
    q[..., 3] = 8
    k[:, :, 64:, 3] = np.float16(target / (8 * float(scale)))
    o, lse = run(q, k, v, False, scale)
    o_ref, lse_ref = oracle.fmha_all(q, k, v, causal=False, scale=scale)
    s = float(scale) * np.einsum("nd,md->nm", q[0, 0].astype(np.float64), k[0, 0].astype(np.float64))
    gap = (s[:, 64:].max(axis=1) - s[:, :64].max(axis=1)) / math.log(2)
    assert 12 < gap.min() and gap.max() < 15.5, (gap.min(), gap.max())
    rows = np.argwhere(np.ones((B, H, N), bool))
    check_rows(o, lse, rows, o_ref.reshape(-1, d), lse_ref.reshape(-1), "late-inside")


@pytest.mark.parametrize("d", [64, 128])
def test_one_hot_scores_select_one_value_row(d, device):
    N = 300
    q = np.zeros((1, 2, N, d), np.float16)
    k = np.zeros((1, 2, N, d), np.float16)
    v = inputs.draw_qkv(1, 2, N, d, seed=9)[2]
    jstar = 217
    q[..., 5] = 64
    k[:, :, jstar, 5] = 64
    scale = np.float32(1 / math.sqrt(d))
    o, lse = run(q, k, v, False, scale)
    assert np.array_equal(o, np.broadcast_to(v[:, :, jstar:jstar + 1], o.shape))
    assert np.abs(lse - 4096 * float(scale)).max() <= TOL_LSE


def tile_edge_rows(B, H, N, bm, seed):
    """Per (b, h, query tile): its first row, its last row and one row
    between them."""
    rng = np.random.default_rng(seed)
    out = []
    for b in range(B):
        for h in range(H):
            for t0 in range(0, N, bm):
                t1 = min(t0 + bm, N) - 1
                out += [(b, h, t0), (b, h, t1), (b, h, int(rng.integers(t0, t1 + 1)))]
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("d,causal", [(64, False), (64, True), (128, False), (128, True)])
def test_persistent_passes_cover_every_tile(d, causal, device):
    """More query tiles than compute units, and a count that is not a
    multiple of 8: workgroups walk several tiles each, odd passes in
    reverse, and the last pass is partial. Every output is written (the NaN
    fill is gone), and rows at both edges of every tile match the oracle."""
    torch = torch_mod()
    B, H, N = 3, 31, 1000
    bm = fmha.fmha_query_tile(d)
    tiles = B * H * (-(-N // bm))
    assert tiles > torch.cuda.get_device_properties(0).multi_processor_count and tiles % 8
    print("persistent cover d=%d causal=%d tiles=%d" % (d, causal, tiles), flush=True)
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=1700 + d + causal)
    scale = np.float32(1 / math.sqrt(d))
    o, lse = run(q, k, v, causal, scale)
    assert not np.isnan(o).any() and not np.isnan(lse).any(), "unwritten output"
    rows = tile_edge_rows(B, H, N, bm, seed=d + causal)
    o_ref, lse_ref = oracle.fmha_rows(q, k, v, rows, causal=causal, scale=scale)
    check_rows(o, lse, rows, o_ref, lse_ref, "persistent cover")


@pytest.mark.parametrize("B,H,N,causal", [(1, 1, 600, False), (1, 3, 1024, True), (3, 5, 1000, False)])
def test_one_workgroup_per_tile_grid_not_a_multiple_of_8(B, H, N, causal, device):
    """Fewer query tiles than compute units and not a multiple of 8 (3, 12
    and 60 tiles): one workgroup per tile and a single pass, the grid on
    which the reversed walk of an odd pass falls below the tile count.
    Every output is written and every row matches the oracle."""
    d = 128
    bm = fmha.fmha_query_tile(d)
    tiles = B * H * (-(-N // bm))
    assert tiles < 256 and tiles % 8
    print("one workgroup per tile: tiles=%d causal=%d" % (tiles, causal), flush=True)
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=1900 + tiles)
    scale = np.float32(1 / math.sqrt(d))
    o, lse = run(q, k, v, causal, scale)
    assert not np.isnan(o).any() and not np.isnan(lse).any(), "unwritten output"
    o_ref, lse_ref = oracle.fmha_all(q, k, v, causal=causal, scale=scale)
    assert np.abs(o.astype(np.float64) - o_ref).max() <= TOL_O
    assert np.abs(lse.astype(np.float64) - lse_ref).max() <= TOL_LSE


@pytest.mark.parametrize("d", [64, 128])
def test_causal_first_row_is_first_value_row(d, device):
    q, k, v = inputs.draw_qkv(2, 2, 257, d, seed=12)
    scale = np.float32(1 / math.sqrt(d))
    o, lse = run(q, k, v, True, scale)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    s0 = float(scale) * np.einsum("bhd,bhd->bh", q[:, :, 0].astype(np.float64),
                                  k[:, :, 0].astype(np.float64))
    assert np.abs(lse[:, :, 0] - s0).max() <= TOL_LSE


def test_key_permutation_invariance(device):
    q, k, v = inputs.draw_qkv(1, 4, 1000, 128, seed=13)
    scale = np.float32(1 / math.sqrt(128))
    o, lse = run(q, k, v, False, scale)
    perm = np.random.default_rng(3).permutation(1000)
    o2, lse2 = run(q, k[:, :, perm], v[:, :, perm], False, scale)
    assert np.abs(o.astype(np.float64) - o2).max() <= TOL_O
    assert np.abs(lse.astype(np.float64) - lse2).max() <= TOL_LSE


def test_deterministic_bitwise(device):
    q, k, v, scale = inputs.workload_inputs(1)
    a = run(q, k, v, False, scale)
    b = run(q, k, v, False, scale)
    assert np.array_equal(a[0].view(np.uint16), b[0].view(np.uint16))
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_causal_workload_repeats_bitwise(device):
    """Three launches of the causal K x3 workload (B4 H32 N8192: diagonal
    tiles with masked keys and waves that sit out their last key tiles) give
    the same bits: a read of an LDS slot before every wave's share of it has
    landed, or any other race between waves, would show here as run-to-run
    differences."""
    idx = [i for i, w in enumerate(inputs.WORKLOADS) if w.causal][0]
    q, k, v, scale = inputs.workload_inputs(idx)
    a = run(q, k, v, True, scale)
    for _ in range(2):
        b = run(q, k, v, True, scale)
        assert np.array_equal(a[0].view(np.uint16), b[0].view(np.uint16))
        assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_non_default_stream(device):
    torch = torch_mod()
    q, k, v = inputs.draw_qkv(2, 2, 500, 128, seed=14)
    scale = np.float32(1 / math.sqrt(128))
    ref = run(q, k, v, True, scale)
    s = torch.cuda.Stream()
    got = run(q, k, v, True, scale, stream=s)
    assert np.array_equal(ref[0].view(np.uint16), got[0].view(np.uint16))


@pytest.mark.parametrize("B,H,N,causal", [(2, 2, 333, True), (3, 31, 1000, False)])
def test_guard_bands_untouched(B, H, N, causal, device):
    """Writes stay inside o and lse: sentinels around both are unchanged.
    The second case runs several tiles per workgroup with a ragged last
    query tile (its rows past N are dropped stores and zero Q loads)."""
    torch = torch_mod()
    d = 128
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=15)
    tq, tk, tv = to_dev(q, k, v)
    pad = 4096
    ob = torch.full((B * H * N * d + 2 * pad,), 12345.0, dtype=torch.float16, device="cuda:0")
    lb = torch.full((B * H * N + 2 * pad,), -777.0, dtype=torch.float32, device="cuda:0")
    o = ob[pad:pad + B * H * N * d].view(B, H, N, d)
    lse = lb[pad:pad + B * H * N].view(B, H, N)
    fmha.forward(tq, tk, tv, causal=causal, scale=0.088388, out=o, lse=lse)
    torch.cuda.synchronize()
    obc, lbc = ob.cpu().numpy(), lb.cpu().numpy()
    assert (obc[:pad] == np.float16(12345.0)).all() and (obc[-pad:] == np.float16(12345.0)).all()
    assert (lbc[:pad] == -777.0).all() and (lbc[-pad:] == -777.0).all()
    assert np.isfinite(obc[pad:-pad]).all()


@pytest.mark.parametrize("d,causal", [(64, True), (64, False), (128, True), (128, False)])
@pytest.mark.parametrize("scale", [0.02, 0.5, 0.0, -0.0, -0.088388, -0.5])
def test_other_scale_values(scale, d, causal, device):
    """Any finite scale: small and large positive ones, zero (uniform weights
    over the visible keys) and negative ones (the smallest q.k wins)."""
    N = 190 if d == 64 else 333
    print("scale=%g d=%d causal=%d" % (scale, d, causal), flush=True)
    q, k, v = inputs.draw_qkv(1, 3, N, d, seed=16 + d + causal)
    scale = np.float32(scale)
    o, lse = run(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.fmha_all(q, k, v, causal=causal, scale=scale)
    rows = np.argwhere(np.ones((1, 3, N), bool))
    check_rows(o, lse, rows, o_ref.reshape(-1, d), lse_ref.reshape(-1), "scale")


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_is_the_mean_of_visible_values(causal, device):
    """scale = 0 at a full-size shape with every row checked in closed form:
    O_i is the mean of the visible value rows and lse_i = ln |J_i|."""
    B, H, N, d = 4, 32, 2048, 128
    print("zero scale B=%d H=%d N=%d causal=%d" % (B, H, N, causal), flush=True)
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=808 + causal)
    o, lse = run(q, k, v, causal, np.float32(0.0))
    if causal:
        cnt = np.arange(1, N + 1, dtype=np.float64)
        mean = np.cumsum(v.astype(np.float64), axis=2) / cnt[None, None, :, None]
        lse_ref = np.broadcast_to(np.log(cnt)[None, None, :], lse.shape)
    else:
        mean = np.broadcast_to(v.astype(np.float64).mean(axis=2, keepdims=True), v.shape)
        lse_ref = np.full(lse.shape, math.log(N))
    eo = np.abs(o.astype(np.float64) - mean).max()
    el = np.abs(lse.astype(np.float64) - lse_ref).max()
    print("zero scale: max|dO|=%.3e max|dlse|=%.3e" % (eo, el), flush=True)
    assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.parametrize("causal,k_gain", [(False, 1.0), (True, 3.0)])
def test_head_dim_64_at_full_size(causal, k_gain, device):
    """The d = 64 kernels at B4 H32 N4096 (512 query tiles, two persistent
    passes): 256 seeded rows plus, for causal, the tile-edge rows of 4 heads
    at the d = 64 kernel's own tile sizes. The causal case draws K scaled by 3
    (sharp rows, the exact pass's lazy rescale) as the d = 128 causal
    workload does."""
    B, H, N, d = 4, 32, 4096, 64
    print("d=64 full size causal=%d k_gain=%g" % (causal, k_gain), flush=True)
    q, k, v = inputs.draw_qkv(B, H, N, d, seed=6400 + causal, k_gain=k_gain)
    scale = np.float32(1 / math.sqrt(d))
    o, lse = run(q, k, v, causal, scale)
    assert not np.isnan(o).any() and not np.isnan(lse).any(), "unwritten output"
    rows = inputs.sample_rows(B, H, N, 256, seed=64 + causal)
    if causal:
        bm, bn = fmha.fmha_query_tile(d), fmha.fmha_key_tile(d)
        extra = inputs.boundary_rows(B, H, N, 4, seed=65, tiles=(32, bn, 128, bm))
        assert {bm - 1, bm, bn - 1, bn} <= set(extra[:, 2].tolist())
        rows = np.unique(np.concatenate([rows, extra]), axis=0)
    o_ref, lse_ref = oracle.fmha_rows(q, k, v, rows, causal=causal, scale=scale)
    check_rows(o, lse, rows, o_ref, lse_ref, "d=64 full size")


def test_empty_problem_launches_nothing(device):
    torch = torch_mod()
    q = torch.empty((0, 2, 16, 64), dtype=torch.float16, device="cuda:0")
    o, lse = fmha.forward(q, q.clone(), q.clone(), causal=False)
    torch.cuda.synchronize()
    assert o.numel() == 0 and lse.numel() == 0
