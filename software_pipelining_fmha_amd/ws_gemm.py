"""Python binding of include/ws_gemm.h (ctypes; argument marshalling only).

The GEMM runs in libfmha.so's HIP kernels and the model's recurrences in
its host code. There is no fallback: if the library is missing or fails to
load, every call here raises.
"""
from __future__ import annotations

import ctypes

from software_pipelining_fmha_amd import fmha

EXPORTS = ("ws_gemm", "ws_gemm_trace_words", "ws_gemm_config_count", "ws_gemm_config",
           "ws_model_stage_times", "ws_model_launch_time", "ws_model_two_point",
           "ws_model_default", "ws_gemm_choose")


class ModelParams(ctypes.Structure):
    """ws_model_params: times in microseconds, sizes in elements."""
    _fields_ = [("load_throughput", ctypes.c_double), ("load_latency", ctypes.c_double),
                ("compute_throughput", ctypes.c_double), ("compute_latency", ctypes.c_double),
                ("t_epilogue", ctypes.c_double), ("t_init", ctypes.c_double),
                ("n_units", ctypes.c_int)]


_ready = False


def lib():
    global _ready
    l = fmha.lib()
    if not _ready:
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        l.ws_gemm.restype = I
        l.ws_gemm.argtypes = [P, P, P, I, I, I, I, I, I, I, P, P, P]
        l.ws_gemm_trace_words.restype = ctypes.c_size_t
        l.ws_gemm_trace_words.argtypes = [I] * 6
        l.ws_gemm_config_count.restype = I
        l.ws_gemm_config_count.argtypes = []
        l.ws_gemm_config.restype = I
        l.ws_gemm_config.argtypes = [I, P, P, P, P]
        l.ws_model_stage_times.restype = D
        l.ws_model_stage_times.argtypes = [I, I, D, D, D, P, P, P, P]
        l.ws_model_launch_time.restype = D
        l.ws_model_launch_time.argtypes = [ctypes.POINTER(ModelParams)] + [I] * 7
        l.ws_model_two_point.restype = I
        l.ws_model_two_point.argtypes = [D, D, D, D, P, P]
        l.ws_model_default.restype = None
        l.ws_model_default.argtypes = [ctypes.POINTER(ModelParams), I]
        l.ws_gemm_choose.restype = I
        l.ws_gemm_choose.argtypes = [ctypes.POINTER(ModelParams), I, I, I, P, P, P, P]
        _ready = True
    return l


def configs() -> list[tuple[int, int, int, int]]:
    """The compiled variants as (T_M, T_N, T_K, ring)."""
    out = []
    for i in range(lib().ws_gemm_config_count()):
        v = [ctypes.c_int() for _ in range(4)]
        lib().ws_gemm_config(i, *(ctypes.byref(x) for x in v))
        out.append(tuple(x.value for x in v))
    return out


def trace_words(M, N, K, tile_m, tile_n, tile_k) -> int:
    return int(lib().ws_gemm_trace_words(M, N, K, tile_m, tile_n, tile_k))


def stage_times(S: int, ring: int, t_load_a: float, t_load_b: float, t_math: float):
    """The model's recurrences: (s_a, s_b, s_m lists, math_end, math_wait)."""
    arr = ctypes.c_double * max(S, 1)
    sa, sb, sm = arr(), arr(), arr()
    wait = ctypes.c_double()
    end = lib().ws_model_stage_times(S, ring, t_load_a, t_load_b, t_math, sa, sb, sm,
                                     ctypes.byref(wait))
    if end < 0:
        raise ValueError("invalid stage count or ring depth")
    return list(sa)[:S], list(sb)[:S], list(sm)[:S], end, wait.value


def default_params(cus: int = 256) -> ModelParams:
    p = ModelParams()
    lib().ws_model_default(ctypes.byref(p), cus)
    return p


def launch_time(p: ModelParams, M, N, K, tile_m, tile_n, tile_k, ring) -> float:
    t = lib().ws_model_launch_time(ctypes.byref(p), M, N, K, tile_m, tile_n, tile_k, ring)
    if t < 0:
        raise ValueError("invalid model arguments")
    return t


def two_point(size1, time1, size2, time2):
    thr, lat = ctypes.c_double(), ctypes.c_double()
    if lib().ws_model_two_point(size1, time1, size2, time2, ctypes.byref(thr), ctypes.byref(lat)):
        raise ValueError("the two points coincide")
    return thr.value, lat.value


def choose(M, N, K, p: ModelParams | None = None):
    v = [ctypes.c_int() for _ in range(4)]
    st = lib().ws_gemm_choose(ctypes.byref(p) if p is not None else None, M, N, K,
                              *(ctypes.byref(x) for x in v))
    if st != 0:
        raise fmha.FmhaError(st)
    return tuple(x.value for x in v)


def gemm(a, b, *, out=None, config=(0, 0, 0, 0), trace=None, status=None, stream=None):
    """C = A B on torch tensors: a fp16 [M, K], b fp16 [K, N], contiguous, on
    one GPU. config = (T_M, T_N, T_K, ring), or zeros for the model's pick.
    trace: optional int64 device tensor of trace_words(...) elements; status:
    optional int32 device tensor of one element. Launches on `stream`
    (default: torch's current stream) and does not synchronise."""
    import torch

    if a.dtype != torch.float16 or b.dtype != torch.float16:
        raise TypeError("a and b must be torch.float16")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("a must be [M, K] and b [K, N]")
    if not (a.is_cuda and b.is_cuda) or a.device != b.device:
        raise ValueError("a and b must be on one GPU")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous")
    M, K = a.shape
    N = b.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=a.device)
    if out.shape != (M, N) or out.dtype != torch.float16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp16 [M, N] tensor")
    tr = 0
    if trace is not None:
        need = trace_words(M, N, K, *config[:3])
        if trace.dtype != torch.int64 or trace.numel() < need or not trace.is_contiguous():
            raise ValueError("trace must be a contiguous int64 tensor of >= %d elements" % need)
        tr = trace.data_ptr()
    stp = status.data_ptr() if status is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(a.device):
        st = lib().ws_gemm(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, *config,
                           tr or None, stp or None, handle)
    if st != 0:
        raise fmha.FmhaError(st)
    return out
