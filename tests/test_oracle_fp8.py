"""Pins for the oracle's FP8 path (`oracle.fmha_fp8_rows`), run on the CPU.

- library: the OCP E4M3 decode against torch.float8_e4m3fn on all 256 bytes;
- the FP16 oracle (pinned in test_oracle.py): with power-of-two descales every
  descaled E4M3 value is a binary16 value, so the FP8 path must return the
  FP16 path's results bit for bit; a wrong exponent bias, descale or
  subnormal rule breaks that;
- the tolerance scales against their definition on small cases;
- the input quantizer against the decode (|x - descale e4m3(b)| <= half an
  E4M3 step).
"""
import numpy as np
import pytest

import oracle
from software_pipelining_fmha_amd import inputs


def test_e4m3_decode_matches_torch():
    torch = pytest.importorskip("torch")
    b = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_to_double(b)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))  # signed zeros
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def random_e4m3(shape, seed):
    r = np.random.default_rng(seed)
    b = r.integers(0, 256, size=shape, dtype=np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x38  # no NaN inputs
    # keep |values| <= 8 so that descaled products stay in binary16 range
    big = np.abs(oracle.e4m3_to_double(b)) > 8
    b[big] = b[big] & 0xC7  # clear two exponent bits
    return b


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("descales", [(1.0, 1.0, 1.0), (0.25, 2.0, 0.5), (2.0 ** -3, 1.0, 4.0)])
def test_matches_fp16_oracle_on_exact_inputs(causal, descales):
    B, H, N, d = 2, 2, 37, 16
    q8, k8, v8 = (random_e4m3((B, H, N, d), s) for s in (1, 2, 3))
    scale = np.float32(0.3)
    o8, l8 = oracle.fmha_fp8_all(q8, k8, v8, descales, causal=causal, scale=scale)
    q16, k16, v16 = ((oracle.e4m3_to_double(x) * s).astype(np.float16)
                     for x, s in zip((q8, k8, v8), descales))
    for x, y, s in zip((q16, k16, v16), (q8, k8, v8), descales):
        assert np.array_equal(x.astype(np.float64), oracle.e4m3_to_double(y) * s)  # exact
    o16, l16 = oracle.fmha_all(q16, k16, v16, causal=causal, scale=scale)
    np.testing.assert_array_equal(o8, o16)
    np.testing.assert_array_equal(l8, l16)


@pytest.mark.parametrize("causal", [False, True])
def test_tolerance_scales_match_definition(causal):
    """rss_o[c] = sqrt(sum_j e_j^2 (v_jc - o_c)^2), rss_l = sqrt(sum_j e_j^2),
    e_j = max(2^-4 P_ij, 2^-10 max_j P_ij); sc_o[c] = sum_j P_ij a_ij |v_jc - o_c|,
    sc_l = sum_j P_ij a_ij, a_ij = scale sum_c |q_ic k_jc|; P from scipy's
    softmax."""
    from scipy.special import softmax
    B, H, N, d = 1, 1, 21, 8
    q8, k8, v8 = (random_e4m3((B, H, N, d), s) for s in (4, 5, 6))
    ds = (0.5, 0.25, 2.0)
    scale = np.float32(0.7)
    o, lse, ro, rl, so, sl = oracle.fmha_fp8_all(q8, k8, v8, ds, causal=causal, scale=scale,
                                                 rss=True)
    q, k, v = (oracle.e4m3_to_double(x)[0, 0] * s for x, s in zip((q8, k8, v8), ds))
    s_ = float(scale) * q @ k.T
    if causal:
        s_ = np.where(np.tril(np.ones((N, N), bool)), s_, -np.inf)
    P = softmax(s_, axis=1)
    e = np.maximum(P / 16, P.max(axis=1, keepdims=True) / 1024) * (P > 0)
    np.testing.assert_allclose(rl[0, 0], np.sqrt((e ** 2).sum(1)), rtol=1e-12)
    dev = np.abs(v[None, :, :] - o[0, 0][:, None, :])
    ref = np.sqrt(np.einsum("ij,ijc->ic", e ** 2, dev ** 2))
    np.testing.assert_allclose(ro[0, 0], ref, rtol=1e-12, atol=1e-300)
    a = float(scale) * np.einsum("ic,jc->ij", np.abs(q), np.abs(k))
    Pz = np.where(np.isfinite(s_), P, 0.0)
    np.testing.assert_allclose(sl[0, 0], (Pz * a).sum(1), rtol=1e-12)
    np.testing.assert_allclose(so[0, 0], np.einsum("ij,ijc->ic", Pz * a, dev), rtol=1e-12, atol=1e-300)


def test_quantizer_round_trip():
    x = np.random.default_rng(7).standard_normal((2, 3, 50, 16)).astype(np.float32) * 3
    b, descale = inputs.quantize_e4m3(x)
    y = oracle.e4m3_to_double(b) * float(descale)
    assert np.abs(y).max() <= 448 * float(descale) * (1 + 1e-7)
    # half an E4M3 step: 2^-4 relative in the normal range, 2^-10 absolute below it
    err = np.abs(y - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, float(descale) * 2.0 ** -10) * (1 + 1e-6)
    assert (err <= bound).all()
