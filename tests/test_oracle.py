"""Pins for the CPU oracle (`oracle/`), run on the CPU.

The pages print no worked attention example, so no value here comes from
them. Each test pins the oracle to something other than itself:
- a library routine (numpy's binary16 decode, scipy's softmax and logsumexp);
- an independent pure-Python brute force;
- a closed form or an invariant of softmax(scale * Q K^T) V.
Together they are meant to catch a plausible slip anywhere in it: a dropped
term, a wrong sign or index, a transposed operand, a wrong causal edge, or
the wrong log base.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle

RNG = np.random.default_rng(1234)


def half(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def rand_qkv(B, H, N, d, seed, lo=-2.0, hi=2.0, grid=None):
    r = np.random.default_rng(seed)
    out = []
    for _ in range(3):
        x = r.uniform(lo, hi, size=(B, H, N, d))
        if grid:
            x = np.round(x * grid) / grid
        out.append(half(x))
    return out


def f64(x):
    return x.astype(np.float64)


# --- binary16 decode ---------------------------------------------------------

def test_half_decode_exhaustive_matches_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(got, ref, equal_nan=True)
    # bit-level check incl. signed zeros
    assert np.array_equal(got.view(np.uint64)[~np.isnan(ref)],
                          ref.view(np.uint64)[~np.isnan(ref)])


# --- library special cases ---------------------------------------------------

@pytest.mark.parametrize("scale", [0.37, -0.37, 0.0])
@pytest.mark.parametrize("causal", [False, True])
def test_identity_values_expose_softmax_matrix(causal, scale):
    """With V = I (N <= d) each output row is the softmax row itself. It is
    compared with scipy's softmax and logsumexp of scale * Q K^T. Q != K, so
    a transposed product fails. Any finite scale is allowed: a negative one
    favours the smallest q.k, zero gives uniform weights."""
    N, d = 12, 16
    q, k, _ = rand_qkv(1, 1, N, d, 7)
    v = np.zeros((1, 1, N, d), dtype=np.float16)
    v[0, 0, :, :N] = np.eye(N, dtype=np.float16)
    scale = np.float32(scale)
    o, lse = oracle.fmha_all(q, k, v, causal=causal, scale=scale)
    s = float(scale) * (f64(q[0, 0]) @ f64(k[0, 0]).T)
    if causal:
        s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    p = softmax(s, axis=1)
    np.testing.assert_allclose(o[0, 0, :, :N], p, rtol=0, atol=1e-14)
    assert np.all(o[0, 0, :, N:] == 0)
    np.testing.assert_allclose(o[0, 0, :, :N].sum(1), 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], logsumexp(s, axis=1), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_multihead_rows_match_library_reference(causal):
    """softmax(scale*QK^T) V per head with scipy/numpy. Covers the (b, h, i)
    indexing over several batches and heads."""
    B, H, N, d = 2, 3, 40, 16
    q, k, v = rand_qkv(B, H, N, d, 11)
    scale = np.float32(1 / math.sqrt(d))
    o, lse = oracle.fmha_all(q, k, v, causal=causal, scale=scale)
    for b in range(B):
        for h in range(H):
            s = float(scale) * (f64(q[b, h]) @ f64(k[b, h]).T)
            if causal:
                s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
            ref = softmax(s, axis=1) @ f64(v[b, h])
            np.testing.assert_allclose(o[b, h], ref, rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[b, h], logsumexp(s, axis=1),
                                       rtol=0, atol=1e-13)


def test_large_scores_do_not_overflow():
    """Scores up to ~1e5: exp without max-subtraction would overflow.
    logsumexp from scipy fixes the answer."""
    N, d = 9, 8
    q, k, v = rand_qkv(1, 1, N, d, 5, lo=-100, hi=100)
    o, lse = oracle.fmha_all(q, k, v, causal=False, scale=np.float32(1.0))
    s = f64(q[0, 0]) @ f64(k[0, 0]).T
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    np.testing.assert_allclose(lse[0, 0], logsumexp(s, axis=1), rtol=1e-15, atol=0)
    np.testing.assert_allclose(o[0, 0], softmax(s, axis=1) @ f64(v[0, 0]),
                               rtol=0, atol=1e-12)


# --- brute force -------------------------------------------------------------

def brute_row(q, k, v, i, causal, scale):
    """Pure Python: weights exp(s_j) / sum exp(s_k), no max subtraction."""
    N, d = len(k), len(q[0])
    js = range(i + 1) if causal else range(N)
    s = {j: scale * math.fsum(float(q[i][c]) * float(k[j][c]) for c in range(d))
         for j in js}
    w = {j: math.exp(s[j]) for j in js}
    z = math.fsum(w.values())
    o = [math.fsum(w[j] * float(v[j][c]) for j in js) / z for c in range(d)]
    return o, math.log(z)


@pytest.mark.parametrize("N,d", [(1, 1), (3, 2), (7, 5), (16, 8)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [0.5, -0.5])
def test_brute_force_tiny(N, d, causal, scale):
    q, k, v = rand_qkv(1, 1, N, d, 100 + N * d, lo=-1.5, hi=1.5)
    scale = np.float32(scale)
    o, lse = oracle.fmha_all(q, k, v, causal=causal, scale=scale)
    for i in range(N):
        ro, rl = brute_row(q[0, 0], k[0, 0], v[0, 0], i, causal, float(scale))
        np.testing.assert_allclose(o[0, 0, i], ro, rtol=0, atol=1e-13)
        assert abs(lse[0, 0, i] - rl) < 1e-13


# --- closed forms ------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_uniform_keys_give_mean_of_values(causal):
    B, H, N, d = 1, 2, 33, 8
    q, k, v = rand_qkv(B, H, N, d, 21)
    k[:] = k[:, :, :1, :]  # every key row equal to the first
    scale = np.float32(0.25)
    o, lse = oracle.fmha_all(q, k, v, causal=causal, scale=scale)
    for h in range(H):
        for i in range(N):
            n = i + 1 if causal else N
            np.testing.assert_allclose(o[0, h, i], f64(v[0, h, :n]).mean(0),
                                       rtol=0, atol=1e-14)
            s = float(scale) * float(f64(q[0, h, i]) @ f64(k[0, h, 0]))
            assert abs(lse[0, h, i] - (s + math.log(n))) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_gives_mean_of_visible_values(causal):
    """scale = 0: every visible score is 0, so O_i is the mean of the visible
    value rows and lse_i = ln |J_i| whatever Q and K hold."""
    B, H, N, d = 2, 2, 37, 8
    q, k, v = rand_qkv(B, H, N, d, 23, lo=-50, hi=50)
    o, lse = oracle.fmha_all(q, k, v, causal=causal, scale=np.float32(0.0))
    if causal:
        cnt = np.arange(1, N + 1, dtype=np.float64)
        mean = np.cumsum(f64(v), axis=2) / cnt[None, None, :, None]
        lse_ref = np.broadcast_to(np.log(cnt), (B, H, N))
    else:
        mean = np.broadcast_to(f64(v).mean(axis=2, keepdims=True), v.shape)
        lse_ref = np.full((B, H, N), math.log(N))
    np.testing.assert_allclose(o, mean, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-14)


def test_negative_scale_is_positive_scale_on_negated_queries():
    """(-q).k * |scale| = q.k * scale term by term, and binary16 negation is
    exact, so the two calls see the same scores bit for bit."""
    q, k, v = rand_qkv(2, 2, 50, 16, 29)
    a = oracle.fmha_all(q, k, v, causal=True, scale=np.float32(-0.3))
    b = oracle.fmha_all(-q, k, v, causal=True, scale=np.float32(0.3))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = oracle.fmha_all(q, k, v, causal=True, scale=np.float32(0.3))
    assert not np.allclose(a[0], c[0])


@pytest.mark.parametrize("d", [64, 128])
def test_one_hot_scores_select_one_value_row(d):
    """q_i = 64 e_c and k_{j*} = 64 e_c, other keys zero. The score gap is
    4096*scale, so the output is v_{j*} to within e^-362."""
    N = 50
    q = np.zeros((1, 1, N, d), np.float16)
    k = np.zeros((1, 1, N, d), np.float16)
    v = rand_qkv(1, 1, N, d, 3)[2]
    c, jstar = 5, 17
    q[0, 0, :, c] = 64
    k[0, 0, jstar, c] = 64
    scale = np.float32(1 / math.sqrt(d))
    o, lse = oracle.fmha_all(q, k, v, causal=False, scale=scale)
    for i in range(N):
        assert np.array_equal(o[0, 0, i], f64(v[0, 0, jstar]))
        assert lse[0, 0, i] == pytest.approx(4096 * float(scale), abs=1e-12)


def test_causal_first_row_is_first_value_row():
    q, k, v = rand_qkv(2, 2, 20, 8, 31)
    scale = np.float32(0.3)
    o, lse = oracle.fmha_all(q, k, v, causal=True, scale=scale)
    for b in range(2):
        for h in range(2):
            assert np.array_equal(o[b, h, 0], f64(v[b, h, 0]))
            s0 = float(scale) * math.fsum(f64(q[b, h, 0]) * f64(k[b, h, 0]))
            assert abs(lse[b, h, 0] - s0) < 1e-14


def test_causal_last_row_equals_full_row():
    q, k, v = rand_qkv(1, 3, 25, 8, 41)
    scale = np.float32(0.2)
    oc, lc = oracle.fmha_all(q, k, v, causal=True, scale=scale)
    of, lf = oracle.fmha_all(q, k, v, causal=False, scale=scale)
    assert np.array_equal(oc[:, :, -1], of[:, :, -1])
    assert np.array_equal(lc[:, :, -1], lf[:, :, -1])


def test_causal_row_sees_exactly_keys_up_to_itself():
    """Changing key/value rows after i leaves row i alone; changing row i
    itself changes it (the edge is j <= i, not j < i)."""
    N, d, i = 16, 8, 6
    q, k, v = rand_qkv(1, 1, N, d, 51)
    scale = np.float32(0.5)
    o0, l0 = oracle.fmha_rows(q, k, v, [[0, 0, i]], causal=True, scale=scale)
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, i + 1:] = half(9.0)
    v2[0, 0, i + 1:] = half(-7.0)
    o1, l1 = oracle.fmha_rows(q, k2, v2, [[0, 0, i]], causal=True, scale=scale)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    k3, v3 = k.copy(), v.copy()
    k3[0, 0, i] = half(3.0)
    v3[0, 0, i] = half(5.0)
    o2, l2 = oracle.fmha_rows(q, k3, v3, [[0, 0, i]], causal=True, scale=scale)
    assert not np.allclose(o0, o2) and not np.allclose(l0, l2)


# --- invariants --------------------------------------------------------------

def test_key_permutation_invariance():
    q, k, v = rand_qkv(1, 2, 37, 16, 61)
    scale = np.float32(0.25)
    o, lse = oracle.fmha_all(q, k, v, causal=False, scale=scale)
    perm = np.random.default_rng(9).permutation(37)
    op, lp = oracle.fmha_all(q, k[:, :, perm], v[:, :, perm], causal=False, scale=scale)
    np.testing.assert_allclose(op, o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lp, lse, rtol=0, atol=1e-13)


def test_key_shift_moves_lse_only():
    """K + 1 u^T adds scale*q.u to every score of a row. O is unchanged and
    lse grows by scale*q.u. Inputs on a 1/8 grid keep K + u exact in fp16."""
    N, d = 21, 8
    q, k, v = rand_qkv(1, 1, N, d, 71, grid=8)
    u = half(np.round(np.random.default_rng(2).uniform(-2, 2, d) * 8) / 8)
    k2 = half(f64(k) + f64(u))
    assert np.array_equal(f64(k2), f64(k) + f64(u))  # exact shift
    scale = np.float32(0.5)
    o, lse = oracle.fmha_all(q, k, v, causal=False, scale=scale)
    o2, lse2 = oracle.fmha_all(q, k2, v, causal=False, scale=scale)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    shift = float(scale) * (f64(q[0, 0]) @ f64(u))
    np.testing.assert_allclose(lse2[0, 0] - lse[0, 0], shift, rtol=0, atol=1e-12)


def test_values_affine_map_through():
    """a V + 1 c^T gives a O + 1 c^T: the weights are convex."""
    N, d = 19, 8
    q, k, v = rand_qkv(1, 1, N, d, 81, grid=8)
    c = half(np.arange(d) / 8.0 - 0.5)
    v2 = half(2.0 * f64(v) + f64(c))
    assert np.array_equal(f64(v2), 2.0 * f64(v) + f64(c))
    scale = np.float32(0.4)
    for causal in (False, True):
        o, lse = oracle.fmha_all(q, k, v, causal=causal, scale=scale)
        o2, lse2 = oracle.fmha_all(q, k, v2, causal=causal, scale=scale)
        np.testing.assert_allclose(o2, 2.0 * o + f64(c), rtol=0, atol=1e-13)
        assert np.array_equal(lse, lse2)


def test_constant_values_give_constant_output():
    q, k, _ = rand_qkv(1, 1, 30, 8, 91)
    v = np.full((1, 1, 30, 8), 1.5, np.float16)
    o, _ = oracle.fmha_all(q, k, v, causal=True, scale=np.float32(0.7))
    np.testing.assert_allclose(o, 1.5, rtol=0, atol=1e-15)


def test_lse_is_natural_log_of_scaled_scores():
    """Two keys with scaled scores 0 and ln 3 give lse = ln 4 in base e,
    not log2(4) and not the unscaled value."""
    q = np.zeros((1, 1, 2, 1), np.float16)
    k = np.zeros((1, 1, 2, 1), np.float16)
    v = np.zeros((1, 1, 2, 1), np.float16)
    q[..., 0] = 1.0
    k[0, 0, 1, 0] = 2.0
    scale = np.float32(math.log(3.0) / 2.0)
    _, lse = oracle.fmha_all(q, k, v, causal=False, scale=scale)
    expect = math.log(1.0 + math.exp(2.0 * float(scale)))
    np.testing.assert_allclose(lse[0, 0], expect, rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 0] - math.log(4.0)) < 1e-7


# --- mechanics ---------------------------------------------------------------

def test_thread_count_does_not_change_bits():
    q, k, v = rand_qkv(2, 2, 64, 16, 101)
    a = oracle.fmha_all(q, k, v, causal=True, scale=np.float32(0.25), threads=1)
    b = oracle.fmha_all(q, k, v, causal=True, scale=np.float32(0.25), threads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rows_subset_matches_full():
    q, k, v = rand_qkv(2, 3, 24, 8, 111)
    scale = np.float32(0.3)
    of, lf = oracle.fmha_all(q, k, v, causal=True, scale=scale)
    rows = np.array([[1, 2, 23], [0, 0, 0], [1, 0, 5]])
    o, lse = oracle.fmha_rows(q, k, v, rows, causal=True, scale=scale)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(o[r], of[b, h, i]) and lse[r] == lf[b, h, i]


def test_bad_rows_rejected():
    q, k, v = rand_qkv(1, 1, 4, 2, 1)
    with pytest.raises(RuntimeError):
        oracle.fmha_rows(q, k, v, [[0, 0, 4]], causal=False, scale=1.0)
    with pytest.raises(TypeError):
        oracle.fmha_rows(q.astype(np.float32), k, v, [[0, 0, 0]], causal=False,
                         scale=1.0)


def test_planted_mistakes_are_caught():
    """Each plausible slip, planted in a copy of the definition written
    here, moves the V = I softmax matrix away from scipy's. So the library
    pin above has the power to catch them in the oracle."""
    N, d = 6, 8
    q, k, _ = rand_qkv(1, 1, N, d, 121)
    Q, K = f64(q[0, 0]), f64(k[0, 0])
    scale = 0.41
    ref = softmax(scale * Q @ K.T, axis=1)
    slips = {
        "transposed product": softmax(scale * K @ Q.T, axis=1),
        "scale dropped": softmax(Q @ K.T, axis=1),
        "sign flipped": softmax(-scale * Q @ K.T, axis=1),
        "normalised over queries": softmax(scale * Q @ K.T, axis=0),
        "strict causal edge": softmax(np.where(np.tril(np.ones((N, N)), -1) > 0,
                                               scale * Q @ K.T, -1e300), axis=1),
    }
    for name, bad in slips.items():
        assert np.abs(bad - ref).max() > 1e-3, name
