"""Python binding of the C ABI in include/fmha.h (ctypes; argument
marshalling only). Every step of the attention forward pass runs in
libfmha.so's HIP kernels. There is no fallback: if the library is missing or
fails to load, every call here raises.

PyTorch supplies device memory and the stream.
"""
from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfmha.so")
_lib = None

FMHA_OK = 0
FMHA_ERR_INVALID_ARGUMENT = 1
FMHA_ERR_UNSUPPORTED = 2
FMHA_ERR_HIP = 3

EXPORTS = ("fmha_fwd", "fmha_status_str", "fmha_query_tile", "fmha_key_tile")


class FmhaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__("fmha_fwd failed: %s (status %d)" % (fmha_status_str(status), status))


def lib():
    """The loaded libfmha.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libfmha.so is not built (%s); run __graft_entry__.build() "
                               "or python -m software_pipelining_fmha_amd.build" % _LIB_PATH)
        l = ctypes.CDLL(_LIB_PATH)
        l.fmha_fwd.restype = ctypes.c_int
        l.fmha_fwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_float,
                                                                            ctypes.c_void_p]
        l.fmha_status_str.restype = ctypes.c_char_p
        l.fmha_status_str.argtypes = [ctypes.c_int]
        l.fmha_query_tile.restype = ctypes.c_int
        l.fmha_query_tile.argtypes = [ctypes.c_int]
        l.fmha_key_tile.restype = ctypes.c_int
        l.fmha_key_tile.argtypes = [ctypes.c_int]
        _lib = l
    return _lib


def library_path() -> str:
    return _LIB_PATH


def fmha_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, stream) -> int:
    """The C entry point, pointers as integers. Returns the status code."""
    return lib().fmha_fwd(q, k, v, o, lse, int(B), int(H), int(N), int(d), int(causal),
                          float(scale), stream)


def fmha_status_str(status: int) -> str:
    return lib().fmha_status_str(int(status)).decode()


def fmha_query_tile(d: int) -> int:
    return lib().fmha_query_tile(int(d))


def fmha_key_tile(d: int) -> int:
    return lib().fmha_key_tile(int(d))


def forward(q, k, v, *, causal: bool = False, scale: float | None = None, out=None, lse=None,
            stream=None):
    """Attention forward on torch tensors q, k, v (fp16, contiguous,
    [B, H, N, d], on one GPU). Returns (o fp16 [B,H,N,d], lse fp32 [B,H,N]).
    Launches on `stream` (default: torch's current stream) and does not
    synchronise."""
    import torch

    if q.dtype != torch.float16 or k.dtype != torch.float16 or v.dtype != torch.float16:
        raise TypeError("q, k, v must be torch.float16")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    if not (q.is_cuda and k.is_cuda and v.is_cuda) or len({q.device, k.device, v.device}) != 1:
        raise ValueError("q, k, v must be on one GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != torch.float16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp16 tensor shaped like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = fmha_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      B, H, N, d, causal, scale, handle)
    if st != FMHA_OK:
        raise FmhaError(st)
    return out, lse
