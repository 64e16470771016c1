"""Pins for the oracle's backward pass (`oracle.fmha_bwd_rows`), run on the CPU.

The gradients are those of L = sum(dO * O) with respect to Q, K and V. The
pages print no backward formula or worked example, so each test pins the
oracle to something other than itself:
- calculus: Richardson-extrapolated central differences of the forward
  oracle (pinned on its own in test_oracle.py), on inputs whose
  perturbations are exact in binary16;
- a library routine: torch.autograd on CPU in float64;
- closed forms and invariants: sum_j dk_j = 0, sum_j dv_j = sum_i dO_i,
  uniform keys give dq = 0, a single key gives dq = dk = 0 and dv = dO, the
  last causal key sees only the last query, V shifts leave dq and dk alone,
  linearity in dO.
Between them they catch a dropped scale, a wrong sign of D, a transposed
operand, a wrong causal edge or a mixed-up head (test_oracle_mutants.py
plants such slips).
"""
import numpy as np
import pytest

import oracle


def half(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def rand4(B, H, N, d, seed, lo=-1.5, hi=1.5):
    r = np.random.default_rng(seed)
    return [half(r.uniform(lo, hi, size=(B, H, N, d))) for _ in range(4)]


def f64(x):
    return x.astype(np.float64)


def all_rows(B, H, N):
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    return np.stack([b.ravel(), h.ravel(), i.ravel()], 1)


# --- library routine ---------------------------------------------------------

@pytest.mark.parametrize("scale", [0.41, -0.41, 0.0])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd(causal, scale):
    """Gradients of sum(dO * softmax(scale Q K^T) V) by torch.autograd in
    float64, over 2 batches and 3 heads (b/h indexing) and a ragged N, for a
    positive, a negative and a zero scale."""
    torch = pytest.importorskip("torch")
    B, H, N, d = 2, 3, 23, 8
    q, k, v, do = rand4(B, H, N, d, 11 + causal)
    scale = np.float32(scale)
    dq, dk, dv = oracle.fmha_bwd_all(q, k, v, do, causal=causal, scale=scale)
    Q, K, V = (torch.tensor(f64(x), requires_grad=True) for x in (q, k, v))
    s = float(scale) * (Q @ K.transpose(-1, -2))
    if causal:
        s = s.masked_fill(~torch.tril(torch.ones(N, N, dtype=torch.bool)), float("-inf"))
    out = torch.softmax(s, dim=-1) @ V
    (out * torch.tensor(f64(do))).sum().backward()
    np.testing.assert_allclose(dq, Q.grad.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, K.grad.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, V.grad.numpy(), rtol=0, atol=1e-13)


# --- calculus ----------------------------------------------------------------

def _loss(q, k, v, do, causal, scale):
    o, _ = oracle.fmha_all(q, k, v, causal=causal, scale=scale, threads=1)
    return float((o * f64(do)).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_central_differences_of_forward_oracle(causal):
    """Every gradient entry against Richardson-extrapolated central
    differences of L = sum(dO * O), O from the forward oracle. Inputs lie on
    a 1/64 grid in (-1, 1) and steps are 1/256 and 1/128, so every perturbed
    input is exact in binary16; the extrapolated difference is accurate to
    O(h^4)."""
    B, H, N, d = 1, 2, 5, 4
    r = np.random.default_rng(21 + causal)
    q, k, v, do = (half(np.round(r.uniform(-1, 1, size=(B, H, N, d)) * 64) / 64)
                   for _ in range(4))
    scale = np.float32(0.5)
    dq, dk, dv = oracle.fmha_bwd_all(q, k, v, do, causal=causal, scale=scale)
    grads = {"q": dq, "k": dk, "v": dv}
    base = {"q": q, "k": k, "v": v}
    for name in ("q", "k", "v"):
        fd = np.zeros((B, H, N, d))
        for idx in np.ndindex(B, H, N, d):
            def central(h):
                vals = []
                for sgn in (1, -1):
                    x = dict(base)
                    t = base[name].copy()
                    t[idx] = np.float16(float(base[name][idx]) + sgn * h)
                    assert float(t[idx]) == float(base[name][idx]) + sgn * h  # exact
                    x[name] = t
                    vals.append(_loss(x["q"], x["k"], x["v"], do, causal, scale))
                return (vals[0] - vals[1]) / (2 * h)
            h = 1.0 / 256
            fd[idx] = (4 * central(h) - central(2 * h)) / 3
        np.testing.assert_allclose(grads[name], fd, rtol=0, atol=2e-8,
                                   err_msg="d%s vs finite differences" % name)


# --- closed forms and invariants ---------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(causal):
    """sum_j dS_ij = 0 for every query i (the weights sum to 1), so
    sum_j dk_j = 0 in every head."""
    q, k, v, do = rand4(2, 2, 40, 16, 31 + causal)
    _, dk, _ = oracle.fmha_bwd_all(q, k, v, do, causal=causal, scale=np.float32(0.3))
    assert np.abs(dk.sum(axis=2)).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_value_gradients_sum_to_output_gradients(causal):
    """sum_j dv_j = sum_i dO_i, because every query's weights sum to 1."""
    q, k, v, do = rand4(2, 2, 40, 16, 41 + causal)
    _, _, dv = oracle.fmha_bwd_all(q, k, v, do, causal=causal, scale=np.float32(0.3))
    np.testing.assert_allclose(dv.sum(axis=2), f64(do).sum(axis=2), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_keys_give_zero_query_gradient(causal):
    """All key rows equal: dq_i = scale * u * sum_j dS_ij = 0."""
    q, k, v, do = rand4(1, 2, 30, 8, 51)
    k[:] = k[:, :, :1]
    dq, _, _ = oracle.fmha_bwd_all(q, k, v, do, causal=causal, scale=np.float32(0.3))
    assert np.abs(dq).max() < 1e-13


def test_single_key_closed_form():
    """N = 1: P = 1 and D = dP, so dS = 0: dq = dk = 0 and dv = dO."""
    q, k, v, do = rand4(2, 3, 1, 16, 61)
    for causal in (False, True):
        dq, dk, dv = oracle.fmha_bwd_all(q, k, v, do, causal=causal, scale=np.float32(0.7))
        assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
        np.testing.assert_array_equal(dv, f64(do))


def test_last_causal_key_sees_only_last_query():
    """Causal: key N-1 is visible to query N-1 only, so dv_{N-1} = P dO_{N-1}
    and dk_{N-1} = scale * P (dP - D) q_{N-1}, with P = exp(s - lse) from the
    forward oracle and D = dO_{N-1} . o_{N-1}."""
    B, H, N, d = 1, 2, 19, 8
    q, k, v, do = rand4(B, H, N, d, 71)
    scale = np.float32(0.37)
    o, lse = oracle.fmha_all(q, k, v, causal=True, scale=scale)
    _, dk, dv = oracle.fmha_bwd_all(q, k, v, do, causal=True, scale=scale)
    for h in range(H):
        qi, kj, vj, doi = (f64(x[0, h, N - 1]) for x in (q, k, v, do))
        P = np.exp(float(scale) * qi @ kj - lse[0, h, N - 1])
        D = doi @ o[0, h, N - 1]
        np.testing.assert_allclose(dv[0, h, N - 1], P * doi, rtol=0, atol=1e-14)
        np.testing.assert_allclose(dk[0, h, N - 1], float(scale) * P * (doi @ vj - D) * qi,
                                   rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_value_shift_leaves_q_and_k_gradients(causal):
    """v_j -> v_j + c moves dP_ij and D_i by the same dO_i . c, so dS, dq and
    dk do not change; dv does not depend on V at all."""
    q, k, v, do = rand4(1, 2, 25, 8, 81 + causal)
    v = half(np.round(f64(v) * 64) / 64)  # on a 1/64 grid, so + 0.5 is exact
    v2 = half(f64(v) + 0.5)
    assert np.array_equal(f64(v2), f64(v) + 0.5)  # exact shift
    a = oracle.fmha_bwd_all(q, k, v, do, causal=causal, scale=np.float32(0.3))
    b = oracle.fmha_bwd_all(q, k, v2, do, causal=causal, scale=np.float32(0.3))
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-13)


def test_linear_in_output_gradient():
    """The gradients are linear in dO: doubling dO (exact in binary16)
    doubles every gradient bit for bit."""
    q, k, v, do = rand4(1, 2, 17, 8, 91)
    a = oracle.fmha_bwd_all(q, k, v, do, causal=False, scale=np.float32(0.3))
    b = oracle.fmha_bwd_all(q, k, v, (do.astype(np.float32) * 2).astype(np.float16),
                            causal=False, scale=np.float32(0.3))
    for x, y in zip(a, b):
        np.testing.assert_array_equal(2 * x, y)


def test_row_subsets_match_every_row():
    """Scattered (b, h, i) rows, repeated heads and thread counts give the
    same bits as computing every row."""
    B, H, N, d = 2, 3, 21, 8
    q, k, v, do = rand4(B, H, N, d, 101)
    scale = np.float32(0.3)
    full = oracle.fmha_bwd_all(q, k, v, do, causal=True, scale=scale)
    rows = all_rows(B, H, N)[np.random.default_rng(5).permutation(B * H * N)[:40]]
    qr, kr = rows[:25], rows[15:]
    dq, dk, dv = oracle.fmha_bwd_rows(q, k, v, do, qr, kr, causal=True, scale=scale, threads=3)
    np.testing.assert_array_equal(dq, full[0][qr[:, 0], qr[:, 1], qr[:, 2]])
    np.testing.assert_array_equal(dk, full[1][kr[:, 0], kr[:, 1], kr[:, 2]])
    np.testing.assert_array_equal(dv, full[2][kr[:, 0], kr[:, 1], kr[:, 2]])


def test_bad_rows_rejected():
    q, k, v, do = rand4(1, 1, 4, 4, 111)
    with pytest.raises(RuntimeError):
        oracle.fmha_bwd_rows(q, k, v, do, [[0, 0, 4]], [], causal=False, scale=0.5)
    with pytest.raises(RuntimeError):
        oracle.fmha_bwd_rows(q, k, v, do, [], [[0, 1, 0]], causal=False, scale=0.5)


# --- root-sum-square tolerance scales ----------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_rss_outputs_match_term_sums(causal):
    """The optional tolerance scales: per element sqrt(sum_t a_t^2) over the
    terms a_t of each gradient sum, and the D sensitivities
    ds_q = scale * w_i * sum_j P_ij |k_jc| and
    ds_k = scale * sqrt(sum_i (P_ij w_i q_ic)^2) with
    w_i = sum_c |dO_ic| sum_j P_ij |v_jc|, all with P and dS from torch's
    softmax (the GPU tests scale their tolerance by these). Values are
    unchanged when the scales are requested."""
    torch = pytest.importorskip("torch")
    B, H, N, d = 1, 2, 19, 8
    q, k, v, do = rand4(B, H, N, d, 121 + causal)
    scale = np.float32(0.45)
    plain = oracle.fmha_bwd_all(q, k, v, do, causal=causal, scale=scale)
    dq, dk, dv, rq, rk, rv, sq, sk = oracle.fmha_bwd_all(q, k, v, do, causal=causal, scale=scale,
                                                         rss=True)
    for x, y in zip(plain, (dq, dk, dv)):
        np.testing.assert_array_equal(x, y)
    Q, K, V, DO = (torch.tensor(f64(x)) for x in (q, k, v, do))
    s = float(scale) * (Q @ K.transpose(-1, -2))
    if causal:
        s = s.masked_fill(~torch.tril(torch.ones(N, N, dtype=torch.bool)), float("-inf"))
    P = torch.softmax(s, dim=-1)
    Dv = (DO * (P @ V)).sum(-1, keepdim=True)
    dS = P * (DO @ V.transpose(-1, -2) - Dv)
    sc = float(scale)
    np.testing.assert_allclose(rv, torch.sqrt((P ** 2).transpose(-1, -2) @ DO ** 2).numpy(),
                               rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(rk, sc * torch.sqrt((dS ** 2).transpose(-1, -2) @ Q ** 2).numpy(),
                               rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(rq, sc * torch.sqrt((dS ** 2) @ K ** 2).numpy(),
                               rtol=1e-12, atol=1e-15)
    w = (DO.abs() * (P @ V.abs())).sum(-1, keepdim=True)
    np.testing.assert_allclose(sq, (sc * w * (P @ K.abs())).numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(
        sk, sc * torch.sqrt((P ** 2).transpose(-1, -2) @ (w ** 2 * Q ** 2)).numpy(),
        rtol=1e-12, atol=1e-15)
