"""The C ABI on the CPU: the library loads, exports every function that
include/fmha.h declares, and rejects bad arguments before any HIP call (so
no GPU is needed here)."""
import math
import os
import re

import pytest

from software_pipelining_fmha_amd import fmha

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fmha.h")

A = 1 << 20  # a fake, 16-byte aligned "device address" (never dereferenced)


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fmha_\w+)\s*\(", text, re.M)))


def test_header_declares_the_exports():
    assert declared_functions() == sorted(fmha.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = fmha.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def call(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=1, N=128, d=128, causal=0,
         scale=0.125):
    return fmha.fmha_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_null_pointer_is_invalid(which):
    assert call(**{which: 0}) == fmha.FMHA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("field", ["B", "H", "N"])
def test_negative_size_is_invalid(field):
    assert call(**{field: -1}) == fmha.FMHA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("scale", [math.inf, -math.inf, math.nan])
def test_non_finite_scale_is_invalid(scale):
    assert call(scale=scale) == fmha.FMHA_ERR_INVALID_ARGUMENT


def no_gpu():
    """True when no GPU is visible: then a call that passes every argument
    check fails at its first HIP call (status 3) instead of launching on
    the fake addresses these tests pass."""
    try:
        import torch
        return not torch.cuda.is_available()
    except ImportError:  # pragma: no cover
        return True


@pytest.mark.skipif(not no_gpu(), reason="would launch on fake device addresses")
@pytest.mark.parametrize("scale", [0.0, -0.0, -0.125, -3.0])
def test_any_finite_scale_passes_the_checks(scale):
    assert call(scale=scale) == fmha.FMHA_ERR_HIP
    assert call_fp8(scale=scale) == fmha.FMHA_ERR_HIP
    assert call_bwd(scale=scale) == fmha.FMHA_ERR_HIP


@pytest.mark.parametrize("d", [0, 32, 96, 256, -64])
def test_head_dim_outside_64_128_is_unsupported(d):
    assert call(d=d) == fmha.FMHA_ERR_UNSUPPORTED


@pytest.mark.parametrize("which,off", [("q", 8), ("k", 2), ("v", 4), ("o", 8), ("lse", 2)])
def test_misaligned_pointer_is_unsupported(which, off):
    base = {"q": A, "k": 2 * A, "v": 3 * A, "o": 4 * A, "lse": 5 * A}[which]
    assert call(**{which: base + off}) == fmha.FMHA_ERR_UNSUPPORTED


def test_head_too_long_is_unsupported():
    # (N + 256) * d * 2 bytes per head must stay below 2^31
    assert call(N=(1 << 23), d=128) == fmha.FMHA_ERR_UNSUPPORTED


def test_grid_too_large_is_unsupported():
    assert call(B=1 << 20, H=1 << 10, N=1 << 14, q=1 << 50, k=2 << 50, v=3 << 50, o=4 << 50,
                lse=5 << 50) == fmha.FMHA_ERR_UNSUPPORTED


@pytest.mark.parametrize("which", ["q", "k", "v"])
def test_output_aliasing_input_is_invalid(which):
    kw = {which: 4 * A}  # same address as o
    assert call(**kw) == fmha.FMHA_ERR_INVALID_ARGUMENT
    kw = {which: 5 * A}  # same address as lse
    assert call(**kw) == fmha.FMHA_ERR_INVALID_ARGUMENT


def test_lse_overlapping_o_is_invalid():
    assert call(lse=4 * A + 64) == fmha.FMHA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("field", ["B", "H", "N"])
def test_empty_problem_is_ok_and_launches_nothing(field):
    # returns before any HIP call, so it runs without a GPU
    assert call(**{field: 0}) == fmha.FMHA_OK


def test_status_strings():
    for s in range(5):
        assert fmha.fmha_status_str(s) and fmha.fmha_status_str(s) != "unknown status"
    assert fmha.fmha_status_str(99) == "unknown status"


def test_tiles_reported():
    for d in (64, 128):
        assert fmha.fmha_query_tile(d) > 0 and fmha.fmha_key_tile(d) > 0
    assert fmha.fmha_query_tile(96) == 0 and fmha.fmha_key_tile(96) == 0


def test_row_sampler_uses_the_kernel_tiles():
    """The causal workloads' edge rows (inputs.boundary_rows) are taken at the
    forward kernels' real tile sizes."""
    from software_pipelining_fmha_amd import inputs
    assert fmha.fmha_query_tile(128) == inputs.FWD_QUERY_TILE
    assert fmha.fmha_key_tile(128) == inputs.FWD_KEY_TILE
    assert {inputs.FWD_QUERY_TILE, inputs.FWD_KEY_TILE} <= set(inputs.TILE_EDGES)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(fmha, "_lib", None)
    monkeypatch.setattr(fmha, "_LIB_PATH", "/nonexistent/libfmha.so")
    with pytest.raises(RuntimeError, match="not built"):
        fmha.lib()


def call_fp8(q=A, k=2 * A, v=3 * A, dq=0.01, dk=0.01, dv=0.01, o=4 * A, lse=5 * A, B=1, H=1,
             N=128, d=128, causal=0, scale=0.088):
    return fmha.fmha_fwd_fp8(q, k, v, dq, dk, dv, o, lse, B, H, N, d, causal, scale, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_fp8_null_pointer_is_invalid(which):
    assert call_fp8(**{which: 0}) == fmha.FMHA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("which", ["dq", "dk", "dv", "scale"])
def test_fp8_non_finite_factor_is_invalid(which):
    assert call_fp8(**{which: math.nan}) == fmha.FMHA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("which", ["dq", "dk", "dv"])
def test_fp8_non_positive_descale_is_unsupported(which):
    assert call_fp8(**{which: 0.0}) == fmha.FMHA_ERR_UNSUPPORTED


@pytest.mark.parametrize("d", [64, 96, 256])
def test_fp8_head_dim_other_than_128_is_unsupported(d):
    assert call_fp8(d=d) == fmha.FMHA_ERR_UNSUPPORTED


def test_fp8_output_aliasing_input_is_invalid():
    assert call_fp8(q=4 * A) == fmha.FMHA_ERR_INVALID_ARGUMENT
    assert call_fp8(lse=4 * A + 64) == fmha.FMHA_ERR_INVALID_ARGUMENT


def test_fp8_empty_problem_is_ok():
    assert call_fp8(B=0) == fmha.FMHA_OK


BWD = dict(q=A, k=2 * A, v=3 * A, o=4 * A, dout=5 * A, lse=6 * A, dq=7 * A, dk=8 * A, dv=9 * A,
           ws=10 * A)


def call_bwd(B=1, H=1, N=128, d=128, causal=0, scale=0.088, **ptrs):
    p = dict(BWD, **ptrs)
    return fmha.fmha_bwd(p["q"], p["k"], p["v"], p["o"], p["dout"], p["lse"], p["dq"], p["dk"],
                         p["dv"], p["ws"], B, H, N, d, causal, scale, None)


def call_noalloc(B=1, H=1, N=128, d=128, causal=0, scale=0.088, **ptrs):
    p = dict(BWD, **ptrs)
    return fmha.fmha_bwd_noalloc(p["q"], p["k"], p["v"], p["o"], p["dout"], p["lse"], p["dq"],
                                 p["dk"], p["dv"], B, H, N, d, causal, scale, None)


@pytest.mark.parametrize("which", sorted(BWD))
def test_bwd_null_pointer_is_invalid(which):
    assert call_bwd(**{which: 0}) == fmha.FMHA_ERR_INVALID_ARGUMENT
    if which != "ws":
        assert call_noalloc(**{which: 0}) == fmha.FMHA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("which", ["dq", "dk", "dv", "ws"])
def test_bwd_output_aliasing_input_is_invalid(which):
    assert call_bwd(**{which: A}) == fmha.FMHA_ERR_INVALID_ARGUMENT
    if which != "ws":
        assert call_noalloc(**{which: 2 * A}) == fmha.FMHA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("scale", [math.nan, math.inf])
def test_bwd_non_finite_scale_is_invalid(scale):
    assert call_bwd(scale=scale) == fmha.FMHA_ERR_INVALID_ARGUMENT
    assert call_noalloc(scale=scale) == fmha.FMHA_ERR_INVALID_ARGUMENT


def test_bwd_empty_problem_is_ok():
    assert call_bwd(N=0) == fmha.FMHA_OK and call_noalloc(B=0) == fmha.FMHA_OK


def test_noalloc_rejects_problems_beyond_its_workspace():
    # B*H*N one row past the fixed workspace: refused before any HIP call
    big = dict(q=1 << 40, k=2 << 40, v=3 << 40, o=4 << 40, dout=5 << 40, lse=6 << 40, dq=7 << 40,
               dk=8 << 40, dv=9 << 40)
    rows = fmha.FMHA_BWD_NOALLOC_MAX_ROWS
    assert call_noalloc(B=1, H=1, N=rows + 1, d=64, **big) == fmha.FMHA_ERR_TOO_LARGE
    assert call_noalloc(B=4, H=32, N=16385, d=128, **big) == fmha.FMHA_ERR_TOO_LARGE
    assert "workspace" in fmha.fmha_status_str(fmha.FMHA_ERR_TOO_LARGE)


def test_noalloc_limit_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define FMHA_BWD_NOALLOC_MAX_ROWS \(1 << (\d+)\)", text)
    assert m and (1 << int(m.group(1))) == fmha.FMHA_BWD_NOALLOC_MAX_ROWS
    assert re.search(r"#define FMHA_ERR_TOO_LARGE %d\b" % fmha.FMHA_ERR_TOO_LARGE, text)
