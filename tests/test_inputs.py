"""The seeded input generator and row sampler (CPU)."""
import json
import os

import numpy as np

import oracle
from software_pipelining_fmha_amd import inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_workloads_match_the_pages_shapes():
    # FP16, batch 4, 32 heads, head dim 128: Twill section 6.2; Tawa V-D
    for w in inputs.WORKLOADS[1:]:
        assert (w.B, w.H, w.d) == (4, 32, 128)
    assert inputs.WORKLOADS[inputs.HEADLINE].N == 16384
    w = inputs.WORKLOADS[4]
    assert w.causal and w.k_gain == 3.0 and w.N == 8192
    assert inputs.WORKLOADS[3].flops == 4.0 * 4 * 32 * 16384**2 * 128
    assert w.flops == 4.0 * 4 * 32 * 8192**2 * 128 / 2


def test_digests_are_stable():
    gold = json.load(open(os.path.join(GOLD, "inputs_sha256.json")))
    for idx in (0, 1):
        w = inputs.WORKLOADS[idx]
        q, k, v, scale = inputs.workload_inputs(idx)
        g = gold[w.name]
        assert inputs.sha256(q) == g["q"] and inputs.sha256(k) == g["k"]
        assert inputs.sha256(v) == g["v"] and float(scale) == g["scale"]
        assert q.dtype == np.float16 and q.shape == (w.B, w.H, w.N, w.d)


def test_draw_is_fp32_normal_rounded_once():
    q, k, v = inputs.draw_qkv(1, 1, 8, 4, 5, k_gain=3.0)
    rng = np.random.default_rng(5)
    zq = rng.standard_normal((1, 1, 8, 4), dtype=np.float32)
    zk = rng.standard_normal((1, 1, 8, 4), dtype=np.float32)
    assert np.array_equal(q, zq.astype(np.float16))
    assert np.array_equal(k, (zk * np.float32(3)).astype(np.float16))


def test_sample_rows_distinct_in_range_reproducible():
    a = inputs.sample_rows(4, 32, 16384, 256, 77)
    b = inputs.sample_rows(4, 32, 16384, 256, 77)
    assert np.array_equal(a, b) and a.shape == (256, 3)
    assert len({tuple(r) for r in a}) == 256
    assert (a[:, 0] < 4).all() and (a[:, 1] < 32).all() and (a[:, 2] < 16384).all()
    assert (a >= 0).all()


def test_causal_rows_include_tile_edges():
    """The causal workload checks, in 4 seeded heads, rows 0, 1, BN-1, BN,
    BM-1, BM and N-1 of the forward kernel's tiles (BN = 64 keys, BM = 256
    queries), and the wave (32) and wave-group (128) edges."""
    rows = inputs.workload_rows(4)
    edges = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 8191}
    heads = {}
    for b, h, i in rows.tolist():
        heads.setdefault((b, h), set()).add(i)
    full = [hd for hd, ii in heads.items() if edges <= ii]
    assert len(full) >= 4
    assert len(rows) >= 256 + 4 * len(edges) - 4
    for idx in range(len(inputs.FP8_WORKLOADS)):
        if inputs.FP8_WORKLOADS[idx].causal:
            assert edges <= set(inputs.fp8_workload_rows(idx)[:, 2].tolist())


def test_tiny_oracle_regression_fixture():
    gold = json.load(open(os.path.join(GOLD, "tiny_oracle.json")))
    q, k, v, scale = inputs.workload_inputs(0)
    for causal in (False, True):
        g = gold["causal" if causal else "full"]
        o, lse = oracle.fmha_all(q, k, v, causal=causal, scale=scale)
        assert [float.hex(float(x)) for x in lse[0, 0]] == g["lse"]
        for i, row in g["o_rows"].items():
            assert [float.hex(float(x)) for x in o[0, 0, int(i)]] == row
