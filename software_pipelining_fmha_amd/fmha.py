"""Python binding of the C ABI in include/fmha.h (ctypes; argument
marshalling only). Every step of the attention forward and backward passes
runs in libfmha.so's HIP kernels. There is no fallback: if the library is missing or
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
FMHA_ERR_TOO_LARGE = 4
FMHA_BWD_NOALLOC_MAX_ROWS = 1 << 21

EXPORTS = ("fmha_fwd", "fmha_fwd_fp8", "fmha_bwd", "fmha_bwd_workspace_bytes",
           "fmha_status_str", "fmha_query_tile", "fmha_key_tile", "fmha_bwd_noalloc")


class FmhaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__("fmha call failed: %s (status %d)" % (fmha_status_str(status), status))


def lib():
    """The loaded libfmha.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libfmha.so is not built (%s); run __graft_entry__.build() "
                               "or python -m software_pipelining_fmha_amd.build" % _LIB_PATH)
        # torch sets up the HIP runtime first: if the library's kernels are
        # registered before torch initialises HIP, their launches fail with
        # hipErrorOutOfMemory on the MI355X image this targets.
        try:
            import torch
            if torch.cuda.is_available():
                torch.cuda.init()
        except ImportError:  # pragma: no cover
            pass
        l = ctypes.CDLL(_LIB_PATH)
        l.fmha_fwd.restype = ctypes.c_int
        l.fmha_fwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_float,
                                                                            ctypes.c_void_p]
        l.fmha_fwd_fp8.restype = ctypes.c_int
        l.fmha_fwd_fp8.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_float] * 3 + [
            ctypes.c_void_p] * 2 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_void_p]
        l.fmha_bwd.restype = ctypes.c_int
        l.fmha_bwd.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 5 + [ctypes.c_float,
                                                                             ctypes.c_void_p]
        l.fmha_bwd_noalloc.restype = ctypes.c_int
        l.fmha_bwd_noalloc.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 5 + [
            ctypes.c_float, ctypes.c_void_p]
        l.fmha_bwd_workspace_bytes.restype = ctypes.c_size_t
        l.fmha_bwd_workspace_bytes.argtypes = [ctypes.c_int] * 3
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


def fmha_fwd_fp8(q, k, v, dq, dk, dv, o, lse, B, H, N, d, causal, scale, stream) -> int:
    """The C entry point, pointers as integers. Returns the status code."""
    return lib().fmha_fwd_fp8(q, k, v, float(dq), float(dk), float(dv), o, lse, int(B), int(H),
                              int(N), int(d), int(causal), float(scale), stream)


def fmha_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, N, d, causal, scale, stream) -> int:
    """The C entry point, pointers as integers. Returns the status code."""
    return lib().fmha_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, int(B), int(H), int(N), int(d),
                          int(causal), float(scale), stream)


def fmha_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal, scale,
                     stream) -> int:
    """The C entry point, pointers as integers. Returns the status code."""
    return lib().fmha_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, int(B), int(H), int(N),
                                  int(d), int(causal), float(scale), stream)


def fmha_bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(lib().fmha_bwd_workspace_bytes(int(B), int(H), int(N)))


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


def forward_fp8(q8, k8, v8, descales, *, causal: bool = False, scale: float | None = None,
                out=None, lse=None, stream=None):
    """Attention forward with FP8 inputs: q8, k8, v8 are uint8 (or
    float8_e4m3fn) contiguous [B, H, N, 128] torch tensors of OCP E4M3 bytes
    on one GPU, descales = (dq, dk, dv). Returns (o fp16, lse fp32).
    Launches on `stream` (default: torch's current stream) and does not
    synchronise."""
    import torch

    ok = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))
    for t in (q8, k8, v8):
        if t.dtype not in ok or t.dim() != 4 or t.shape != q8.shape:
            raise ValueError("q8, k8, v8 must be uint8 / float8_e4m3fn tensors of one shape")
        if not t.is_contiguous() or not t.is_cuda or t.device != q8.device:
            raise ValueError("q8, k8, v8 must be contiguous and on one GPU")
    B, H, N, d = q8.shape
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.float16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    if out.shape != q8.shape or out.dtype != torch.float16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp16 tensor shaped like q8")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q8.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    dq, dk, dv = (float(x) for x in descales)
    with torch.cuda.device(q8.device):
        st = fmha_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), dq, dk, dv, out.data_ptr(),
                          lse.data_ptr(), B, H, N, d, causal, scale, handle)
    if st != FMHA_OK:
        raise FmhaError(st)
    return out, lse


def backward(q, k, v, o, lse, dout, *, causal: bool = False, scale: float | None = None,
             dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Attention backward on torch tensors: q, k, v, o, dout fp16 contiguous
    [B, H, N, d] and lse fp32 [B, H, N] from the forward pass with the same
    causal and scale. Returns (dq, dk, dv), fp16 [B, H, N, d]. The workspace
    (fp32, at least 2*B*H*N elements) is allocated here unless given.
    Launches on `stream` (default: torch's current stream) and does not
    synchronise."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.dtype != torch.float16 or t.dim() != 4 or t.shape != q.shape:
            raise ValueError("%s must be fp16 shaped like q" % name)
        if not t.is_contiguous() or not t.is_cuda or t.device != q.device:
            raise ValueError("%s must be contiguous and on q's GPU" % name)
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t in (dq, dk, dv):
        if t.shape != q.shape or t.dtype != torch.float16 or not t.is_contiguous():
            raise ValueError("gradient outputs must be contiguous fp16 tensors shaped like q")
    if workspace is None:
        workspace = torch.empty((2 * B * H * N,), dtype=torch.float32, device=q.device)
    if (workspace.dtype != torch.float32 or not workspace.is_contiguous()
            or workspace.numel() < 2 * B * H * N):
        raise ValueError("workspace must be contiguous fp32 with at least 2*B*H*N elements")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = fmha_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                      lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                      workspace.data_ptr(), B, H, N, d, causal, scale, handle)
    if st != FMHA_OK:
        raise FmhaError(st)
    return dq, dk, dv


def backward_noalloc(q, k, v, o, lse, dout, *, causal: bool = False, scale: float | None = None,
                     dq=None, dk=None, dv=None, stream=None):
    """backward() through fmha_bwd_noalloc: the library's fixed workspace
    instead of a caller buffer (B*H*N <= FMHA_BWD_NOALLOC_MAX_ROWS). Calls
    that overlap in time on one GPU race on that workspace. Output tensors
    are allocated here unless given."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.dtype != torch.float16 or t.dim() != 4 or t.shape != q.shape:
            raise ValueError("%s must be fp16 shaped like q" % name)
        if not t.is_contiguous() or not t.is_cuda or t.device != q.device:
            raise ValueError("%s must be contiguous and on q's GPU" % name)
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t in (dq, dk, dv):
        if t.shape != q.shape or t.dtype != torch.float16 or not t.is_contiguous():
            raise ValueError("gradient outputs must be contiguous fp16 tensors shaped like q")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = fmha_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), B, H, N, d, causal, scale, handle)
    if st != FMHA_OK:
        raise FmhaError(st)
    return dq, dk, dv
