"""Pins of the GEMM oracle (CPU only).

The oracle is the definition C = A x B (performance-model page for
warp-specialised kernels, section "GeMM and tiling") in fp64. It is checked
here against facts fixed by the mathematics, never against itself:
exhaustive binary16 decoding, exact integer products, identities, a
periodic closed form, the transpose identity, and numpy's float64 product as
an independent library routine. Planted slips (dropped term, transposed or
misplaced index, wrong exponent bias, lost sign, magnitude without abs) each
fail at least one pin.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "gemm_oracle.c")


def rand_half(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float16)


def test_half_decode_exhaustive():
    """A (65536 x 1) times B = [[1]] returns every binary16 value widened."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    a = bits.view(np.float16).reshape(-1, 1)
    c = oracle.gemm_all(a, np.ones((1, 1), np.float16))[:, 0]
    ref = a[:, 0].astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(c), nan)
    assert np.array_equal(c[~nan], ref[~nan])
    nz = ~nan & (ref != 0)  # the sum starts at +0, so -0 comes back as +0
    assert np.array_equal(np.signbit(c[nz]), np.signbit(ref[nz]))


@pytest.mark.parametrize("M,N,K", [(37, 45, 129), (1, 8, 8), (64, 16, 1), (5, 3, 300)])
def test_integer_inputs_exact(M, N, K):
    """Small integers are exact in binary16 and their sums exact in fp64:
    the result must equal the integer product."""
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    ai = rng.integers(-16, 17, size=(M, K))
    bi = rng.integers(-16, 17, size=(K, N))
    c = oracle.gemm_all(ai.astype(np.float16), bi.astype(np.float16))
    assert np.array_equal(c, (ai @ bi).astype(np.float64))


def test_identity_factors():
    a = rand_half((24, 40), 1)
    b = rand_half((40, 33), 2)
    assert np.array_equal(oracle.gemm_all(a, np.eye(40, dtype=np.float16)), a.astype(np.float64))
    assert np.array_equal(oracle.gemm_all(np.eye(40, dtype=np.float16), b), b.astype(np.float64))


def test_ones_times_periodic_ramp_closed_form():
    """A = ones, B[k][n] = ((k + n) mod 9) - 4: every full period of 9 terms
    sums to zero, so C[m][n] is the sum over the K mod 9 leftover terms,
    (n + j) mod 9 - 4 for j = 0 .. K mod 9 - 1."""
    M, N, K = 7, 20, 4 * 9 + 5
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    b = (((k + n) % 9) - 4).astype(np.float16)
    c = oracle.gemm_all(np.ones((M, K), np.float16), b)
    ref = np.array([sum(((nn + j) % 9) - 4 for j in range(K % 9)) for nn in range(N)], float)
    assert np.array_equal(c, np.broadcast_to(ref, (M, N)))


def test_transpose_identity_bitwise():
    """(A B)^T = B^T A^T; both sums run over the same products in the same k
    order, so they agree bit for bit."""
    a = rand_half((19, 70), 3)
    b = rand_half((70, 27), 4)
    c = oracle.gemm_all(a, b)
    ct = oracle.gemm_all(np.ascontiguousarray(b.T), np.ascontiguousarray(a.T))
    assert np.array_equal(c.T, ct)


def test_random_matches_numpy_float64():
    a = rand_half((50, 300), 5)
    b = rand_half((300, 41), 6)
    c, ca = oracle.gemm_all(a, b, magnitude=True)
    ref = a.astype(np.float64) @ b.astype(np.float64)
    assert (np.abs(c - ref) <= 1e-13 * ca).all()


def test_magnitude_sum():
    a = rand_half((30, 200), 7)
    b = rand_half((200, 25), 8)
    c, ca = oracle.gemm_all(a, b, magnitude=True)
    ref = np.abs(a.astype(np.float64)) @ np.abs(b.astype(np.float64))
    assert (np.abs(ca - ref) <= 1e-13 * ref).all()
    assert (np.abs(c) <= ca).all()
    pa, pb = np.abs(a), np.abs(b)
    c2, ca2 = oracle.gemm_all(pa, pb, magnitude=True)
    assert np.array_equal(c2, ca2)


def test_row_subset_and_degenerate_sizes():
    a = rand_half((40, 64), 9)
    b = rand_half((64, 24), 10)
    full = oracle.gemm_all(a, b)
    rows = np.array([39, 0, 17, 17, 5])
    assert np.array_equal(oracle.gemm_rows(a, b, rows), full[rows])
    z = oracle.gemm_all(np.zeros((3, 0), np.float16), np.zeros((0, 5), np.float16))
    assert z.shape == (3, 5) and not z.any()
    one = oracle.gemm_all(np.full((1, 1), 3.0, np.float16), np.full((1, 1), -0.5, np.float16))
    assert one[0, 0] == -1.5
    with pytest.raises(RuntimeError):
        oracle.gemm_rows(a, b, np.array([40]))


# ---- planted slips ---------------------------------------------------------

MUTANTS = {
    "last k term dropped": ("for (int64_t k = 0; k < K; ++k) {\n            const double am",
                            "for (int64_t k = 0; k < K - 1; ++k) {\n            const double am"),
    "B read transposed": ("jb->b + k * N", "jb->b + k"),
    "A row from the request index": ("jb->a[m * K + k]", "jb->a[r * K + k]"),
    "exponent bias 14": ("e - 25", "e - 24"),
    "subnormal scale": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "sign dropped": ("return sign ? -v : v;", "return v;"),
    "magnitude without abs": ("ca[n] += fabs(p);", "ca[n] += p;"),
}

PINS = [
    test_half_decode_exhaustive,
    lambda: test_integer_inputs_exact(37, 45, 129),
    lambda: test_integer_inputs_exact(5, 3, 300),
    test_identity_factors,
    test_ones_times_periodic_ramp_closed_form,
    test_transpose_identity_bitwise,
    test_random_matches_numpy_float64,
    test_magnitude_sum,
    test_row_subset_and_degenerate_sizes,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_slip(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site vanished: %s" % name
    cpath = tmp_path / "mut.c"
    cpath.write_text(src.replace(old, new))
    so = tmp_path / "mut.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread", str(cpath),
                    "-o", str(so), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    real = oracle._load()
    lib.oracle_gemm_rows.restype = real.oracle_gemm_rows.restype
    lib.oracle_gemm_rows.argtypes = real.oracle_gemm_rows.argtypes
    monkeypatch.setattr(oracle, "_lib", lib)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, RuntimeError):
            failed += 1
    assert failed >= 1, "no pin caught: %s" % name
