"""A CPU model of the backward kernels' arithmetic, held against the bar that
tests/test_gpu_bwd.py applies to the GPU results:

    |g - g_ref| <= 8u rss + 2u |g_ref| + c u ds + 2^-16,   u = 2^-11,
    c = 3 for dq, 21 for dk, 0 for dv (ds = 0 for dv).

The model rounds where the kernels round and nowhere else:
- forward: scores in fp32, weights p = 2^(s c - m) rounded to fp16, l the
  fp32 sum of those weights, O rounded once to fp16, lse in fp32;
- D_i = dO_i . O_i in fp32 from the fp16 O;
- dK/dV kernel: P = fp16(2^(s c - lse log2 e)), dV = P^T dO in fp32;
  dS = fp16(P (dP - D)) with the fp16 P, dK = scale dS^T Q in fp32;
- dQ kernel: P kept in fp32, dS = fp16(P (dP - D)), dQ = scale dS K in fp32;
- every gradient rounded once to fp16.
Matrix-core sums are modelled as the exact sum rounded to fp32.

It shows two things the GPU test cannot show by itself: that this arithmetic
stays below the bar (with margin), and that the bar has the power to fail
plausible defects: a key tile or a query step left out of a sum, the D term
dropped, lse taken in the wrong base. A sharp-softmax case shows why the ds
term is in the bar: without it the exact arithmetic exceeds the bar.
"""
import math

import numpy as np
import pytest

import oracle

U = 2.0 ** -11
LOG2E = 1.4426950408889634


def f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def exp2_f32(x):
    with np.errstate(over="ignore"):
        return f32(np.exp2(np.asarray(x, dtype=np.float32)))


def model(q, k, v, do, causal, scale, defect=None):
    """(dq, dk, dv) of one head as the kernels form them, float64 arrays
    holding fp16 values. `defect` plants one mistake."""
    N, d = q.shape
    qd, kd, vd, dod = (x.astype(np.float64) for x in (q, k, v, do))
    c2 = float(np.float32(float(scale) * LOG2E))
    vis = np.tril(np.ones((N, N), bool)) if causal else np.ones((N, N), bool)
    s = f32(qd @ kd.T)                                     # MFMA, fp32
    # forward: reference m = the row max (the exact pass)
    x = np.where(vis, f32(s * c2), -np.inf)
    m = x.max(axis=1, keepdims=True)
    p16 = f16(exp2_f32(f32(x - m)))
    lsum = f32(p16.sum(axis=1, keepdims=True))
    o16 = f16(f32(f32(p16 @ vd) / lsum))
    lse = f32((m[:, 0] + np.log2(lsum[:, 0])) * math.log(2))
    # D and -lse log2 e
    D = f32((dod * o16).sum(axis=1))
    if defect == "lse_base":
        nl = f32(-lse)
    else:
        nl = f32(-lse * LOG2E)
    expo = np.where(vis, f32(s * c2 + nl[:, None]), -np.inf)
    dp = f32(dod @ vd.T)
    Dm = 0.0 * D if defect == "no_D" else D
    # dK/dV kernel: fp16 P
    P16 = f16(exp2_f32(expo))
    dS16 = f16(f32(P16 * f32(dp - Dm[:, None])))
    keep_q = np.ones(N, bool)
    if defect == "drop_query_step":
        keep_q[64:128] = False
    dv = f16(f32(P16[keep_q].T @ dod[keep_q]))
    dk = f16(f32(f32(dS16[keep_q].T @ qd[keep_q]) * float(scale)))
    # dQ kernel: fp32 P
    P32 = exp2_f32(expo)
    dSq = f16(f32(P32 * f32(dp - Dm[:, None])))
    keep_k = np.ones(N, bool)
    if defect == "drop_key_tile":
        keep_k[64:128] = False
    dq = f16(f32(f32(dSq[:, keep_k] @ kd[keep_k]) * float(scale)))
    return dq, dk, dv


def worst_ratio(q, k, v, do, causal, scale, defect=None, c=(3, 21)):
    """Largest err / bar over every element of every gradient of every head
    (inputs [1, H, N, d])."""
    ref = oracle.fmha_bwd_all(q, k, v, do, causal=causal, scale=scale, rss=True)
    worst = {}
    for h in range(q.shape[1]):
        got = model(q[0, h], k[0, h], v[0, h], do[0, h], causal, scale, defect)
        for gi, name in enumerate(("dq", "dk", "dv")):
            r, rss = ref[gi][0, h], ref[3 + gi][0, h]
            tol = 8 * U * rss + 2 * U * np.abs(r) + 2.0 ** -16
            if gi < 2:
                tol = tol + c[gi] * U * ref[6 + gi][0, h]
            worst[name] = max(worst.get(name, 0.0), float((np.abs(got[gi] - r) / tol).max()))
    return worst


def draw(H, N, d, seed, q_gain=1.0, k_gain=1.0):
    r = np.random.default_rng(seed)
    q = (r.standard_normal((1, H, N, d)) * q_gain).astype(np.float16)
    k = (r.standard_normal((1, H, N, d)) * k_gain).astype(np.float16)
    v = r.standard_normal((1, H, N, d)).astype(np.float16)
    do = r.standard_normal((1, H, N, d)).astype(np.float16)
    return q, k, v, do


CASES = [(False, 64, 1.0), (True, 64, 1.0), (False, 128, 1.0), (True, 128, 3.0)]


@pytest.mark.parametrize("causal,d,k_gain", CASES)
def test_kernel_arithmetic_stays_below_the_bar(causal, d, k_gain):
    q, k, v, do = draw(2, 256, d, 17 + d + causal, k_gain=k_gain)
    scale = np.float32(1 / math.sqrt(d))
    w = worst_ratio(q, k, v, do, causal, scale)
    print("model err/bar:", {n: round(x, 3) for n, x in w.items()})
    assert max(w.values()) < 0.6, w


@pytest.mark.parametrize("defect,grad", [("drop_key_tile", "dq"), ("drop_query_step", "dk"),
                                         ("drop_query_step", "dv"), ("no_D", "dq"),
                                         ("no_D", "dk"), ("lse_base", "dv")])
@pytest.mark.parametrize("causal", [False, True])
def test_planted_defects_exceed_the_bar(defect, grad, causal):
    """Each defect pushes some element of the named gradient past the bar,
    by a wide margin."""
    q, k, v, do = draw(2, 256, 64, 29 + causal)
    scale = np.float32(0.125)
    w = worst_ratio(q, k, v, do, causal, scale, defect)
    print(defect, {n: round(x, 2) for n, x in w.items()})
    assert w[grad] > 1.5, (defect, w)


def test_sharp_softmax_needs_the_D_term():
    """Nearly one-hot attention (large scores): dS is tiny but D_i inherits
    the rounding of the fp16 forward output, which shifts every term of a
    dq row the same way. The exact arithmetic stays within the bar only with
    the ds term; with c = 0 it exceeds it."""
    q, k, v, do = draw(2, 256, 64, 41, q_gain=3.0, k_gain=3.0)
    scale = np.float32(0.125)
    with_term = worst_ratio(q, k, v, do, False, scale)
    without = worst_ratio(q, k, v, do, False, scale, c=(0, 0))
    print("sharp: with ds term", with_term, "without", without)
    assert max(with_term.values()) < 1.0
    assert without["dq"] > 2.0
