"""CPU oracle for the fused multi-head attention forward and backward passes.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench
script's CPU-baseline leg may import this package. The HIP library and its
Python binding never import it, and it imports nothing from them.

`gemm_oracle.c` holds the plain matrix product C = A x B in fp64 (the
GEMM that the performance-model page for warp-specialised kernels tiles),
pinned by `tests/test_oracle_gemm.py`.

`fmha_oracle.c` holds the attention arithmetic: the plain fp64 definition
softmax(scale * Q K^T) V, plus the natural-log logsumexp of each row, one
query row at a time; and the gradients of sum(dO * O) with respect to Q, K
and V, one row at a time, by the chain rule through that definition (the
backward kernel Twill schedules in sections 6.3 and 6.4). The pages name the
stages: QK^T, then softmax, then PV (Tawa, section III-D), and the
load/mma/softmax/rescale tasks (PipeThreader, "core method"). This module
only builds the C library and marshals arrays for it.

Every function here is pinned by `tests/test_oracle.py` (forward),
`tests/test_oracle_bwd.py` (backward) and `tests/test_oracle_fp8.py` (FP8
inputs).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fmha_oracle.c")
_GEMM_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile fmha_oracle.c and gemm_oracle.c with gcc into liboracle.so
    (next to the sources)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                        _SRC, _GEMM_SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_fmha_rows.restype = ctypes.c_int
        lib.oracle_fmha_rows.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_fmha_bwd_rows.restype = ctypes.c_int
        lib.oracle_fmha_bwd_rows.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int, ctypes.c_double,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_fmha_fp8_rows.restype = ctypes.c_int
        lib.oracle_fmha_fp8_rows.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_double, ctypes.c_double, ctypes.c_double,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_e4m3_to_double.restype = None
        lib.oracle_e4m3_to_double.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        lib.oracle_gemm_rows.restype = ctypes.c_int
        lib.oracle_gemm_rows.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_half_to_double.restype = None
        lib.oracle_half_to_double.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_int64]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def half_to_double(bits: np.ndarray) -> np.ndarray:
    """Widen binary16 values (given as float16 or uint16 arrays) to float64."""
    a = np.ascontiguousarray(bits).view(np.uint16)
    out = np.empty(a.shape, dtype=np.float64)
    _load().oracle_half_to_double(a.ctypes.data, out.ctypes.data, a.size)
    return out


def _as_half(x: np.ndarray) -> np.ndarray:
    if x.dtype != np.float16:
        raise TypeError("oracle inputs are float16 arrays, got %s" % x.dtype)
    return np.ascontiguousarray(x)


def fmha_rows(q, k, v, rows, *, causal: bool, scale, threads: int | None = None):
    """Output rows and logsumexp for the given (b, h, i) triples.

    q, k, v: float16 [B, H, N, d]. rows: int [n, 3].
    Returns (o float64 [n, d], lse float64 [n]).
    """
    q, k, v = _as_half(q), _as_half(k), _as_half(v)
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    n = rows.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    st = _load().oracle_fmha_rows(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, N, d, int(bool(causal)),
        float(scale), rows.ctypes.data, n, o.ctypes.data, lse.ctypes.data,
        int(threads or default_threads()))
    if st != 0:
        raise RuntimeError("oracle_fmha_rows failed with status %d" % st)
    return o, lse


def fmha_all(q, k, v, *, causal: bool, scale, threads: int | None = None):
    """Every row: returns (o float64 [B,H,N,d], lse float64 [B,H,N])."""
    B, H, N, d = q.shape
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    rows = np.stack([b.ravel(), h.ravel(), i.ravel()], 1)
    o, lse = fmha_rows(q, k, v, rows, causal=causal, scale=scale, threads=threads)
    return o.reshape(B, H, N, d), lse.reshape(B, H, N)


def fmha_bwd_rows(q, k, v, dout, qrows, krows, *, causal: bool, scale,
                  threads: int | None = None, rss: bool = False):
    """Gradients of sum(dout * O) for selected rows.

    q, k, v, dout: float16 [B, H, N, d]. qrows, krows: int [n, 3] triples
    (b, h, i). Returns (dq float64 [n_q, d], dk float64 [n_k, d],
    dv float64 [n_k, d]). Each distinct head among krows costs one forward
    pass over that head. With rss=True it also returns tolerance scales:
    (dq, dk, dv, rss_q, rss_k, rss_v, ds_q, ds_k), where rss_* is, per
    element, the root-sum-square of the terms summed into it, and ds_q, ds_k
    bound how dq and dk move per unit relative error in the entries of the
    forward output O through D_i = dO_i . O_i (see fmha_oracle.c).
    """
    q, k, v, dout = _as_half(q), _as_half(k), _as_half(v), _as_half(dout)
    if q.ndim != 4 or not (q.shape == k.shape == v.shape == dout.shape):
        raise ValueError("q, k, v, dout must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    qrows = np.ascontiguousarray(qrows, dtype=np.int64).reshape(-1, 3)
    krows = np.ascontiguousarray(krows, dtype=np.int64).reshape(-1, 3)
    dq = np.empty((qrows.shape[0], d), dtype=np.float64)
    dk = np.empty((krows.shape[0], d), dtype=np.float64)
    dv = np.empty((krows.shape[0], d), dtype=np.float64)
    r = [np.empty_like(x) for x in (dq, dk, dv, dq, dk)] if rss else [None] * 5
    ptr = [x.ctypes.data if x is not None else None for x in r]
    st = _load().oracle_fmha_bwd_rows(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data, B, H, N, d,
        int(bool(causal)), float(scale), qrows.ctypes.data, qrows.shape[0], dq.ctypes.data,
        krows.ctypes.data, krows.shape[0], dk.ctypes.data, dv.ctypes.data,
        *ptr, int(threads or default_threads()))
    if st != 0:
        raise RuntimeError("oracle_fmha_bwd_rows failed with status %d" % st)
    return (dq, dk, dv, *r) if rss else (dq, dk, dv)


def fmha_bwd_all(q, k, v, dout, *, causal: bool, scale, threads: int | None = None,
                 rss: bool = False):
    """Every row: returns (dq, dk, dv), each float64 [B, H, N, d] (and the
    five tolerance-scale arrays after them if rss=True)."""
    B, H, N, d = q.shape
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    rows = np.stack([b.ravel(), h.ravel(), i.ravel()], 1)
    out = fmha_bwd_rows(q, k, v, dout, rows, rows, causal=causal, scale=scale,
                        threads=threads, rss=rss)
    return tuple(x.reshape(B, H, N, d) for x in out)


def e4m3_to_double(bits: np.ndarray) -> np.ndarray:
    """Decode OCP FP8 E4M3 bytes (a uint8 array) to float64."""
    a = np.ascontiguousarray(bits, dtype=np.uint8)
    out = np.empty(a.shape, dtype=np.float64)
    _load().oracle_e4m3_to_double(a.ctypes.data, out.ctypes.data, a.size)
    return out


def fmha_fp8_rows(q8, k8, v8, descales, rows, *, causal: bool, scale,
                  threads: int | None = None, rss: bool = False):
    """Attention rows for FP8 inputs: q8, k8, v8 are uint8 [B, H, N, d] arrays
    of OCP E4M3 bytes, descales = (dq, dk, dv) per tensor. Returns
    (o float64 [n, d], lse float64 [n]), plus the tolerance scales
    (rss_o [n, d], rss_l [n], sc_o [n, d], sc_l [n]) if rss=True: rss_* for
    weights rounded to E4M3, sc_* for score errors proportional to the sum of
    the magnitudes of the products (see fmha_oracle.c)."""
    q8, k8, v8 = (np.ascontiguousarray(x, dtype=np.uint8) for x in (q8, k8, v8))
    if q8.ndim != 4 or not (q8.shape == k8.shape == v8.shape):
        raise ValueError("q8, k8, v8 must share one [B, H, N, d] shape")
    B, H, N, d = q8.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    n = rows.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    extra = [np.empty((n, d)), np.empty((n,)), np.empty((n, d)), np.empty((n,))] if rss else []
    ptrs = [x.ctypes.data for x in extra] if rss else [None] * 4
    dq, dk, dv = (float(x) for x in descales)
    st = _load().oracle_fmha_fp8_rows(
        q8.ctypes.data, k8.ctypes.data, v8.ctypes.data, dq, dk, dv, B, H, N, d,
        int(bool(causal)), float(scale), rows.ctypes.data, n, o.ctypes.data, lse.ctypes.data,
        *ptrs, int(threads or default_threads()))
    if st != 0:
        raise RuntimeError("oracle_fmha_fp8_rows failed with status %d" % st)
    return (o, lse, *extra) if rss else (o, lse)


def fmha_fp8_all(q8, k8, v8, descales, *, causal: bool, scale, threads: int | None = None,
                 rss: bool = False):
    """Every row of the FP8 attention: (o [B,H,N,d], lse [B,H,N]) (+ scales)."""
    B, H, N, d = q8.shape
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    rows = np.stack([b.ravel(), h.ravel(), i.ravel()], 1)
    out = fmha_fp8_rows(q8, k8, v8, descales, rows, causal=causal, scale=scale,
                        threads=threads, rss=rss)
    shapes = [(B, H, N, d), (B, H, N)] * 3
    return tuple(x.reshape(sh) for x, sh in zip(out, shapes))


def gemm_rows(a, b, rows, *, threads: int | None = None, magnitude: bool = False):
    """Rows of C = A x B in fp64. a: float16 [M, K], b: float16 [K, N], both
    row-major; rows: int [n]. Returns c float64 [n, N], and with
    magnitude=True also cabs = sum_k |A[m][k] B[k][n]| of the same shape."""
    a, b = _as_half(a), _as_half(b)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("a must be [M, K] and b [K, N]")
    M, K = a.shape
    N = b.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    c = np.empty((rows.size, N), dtype=np.float64)
    ca = np.empty_like(c) if magnitude else None
    st = _load().oracle_gemm_rows(a.ctypes.data, b.ctypes.data, M, N, K, rows.ctypes.data,
                                  rows.size, c.ctypes.data,
                                  ca.ctypes.data if ca is not None else None,
                                  int(threads or default_threads()))
    if st != 0:
        raise RuntimeError("oracle_gemm_rows failed with status %d" % st)
    return (c, ca) if magnitude else c


def gemm_all(a, b, *, threads: int | None = None, magnitude: bool = False):
    """Every row of C = A x B (and of cabs with magnitude=True)."""
    return gemm_rows(a, b, np.arange(a.shape[0]), threads=threads, magnitude=magnitude)
