"""Compiles the HIP library (libfmha.so) for gfx950, in-tree, with hipcc.

    python -m software_pipelining_fmha_amd.build
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfmha.so")
SOURCES = [os.path.join(CSRC, "fmha_api.hip"), os.path.join(CSRC, "ws_gemm_api.hip"),
           os.path.join(CSRC, "fmha_noalloc.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # No packed-fp32 VALU forms (v_pk_fma_f32 and kin) in device code. The
    # host pass does not know this gfx950 feature and warns that it ignores
    # it; the device pass applies it (device_asm() below shows the result).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def command(out: str = LIB, extra: list[str] | None = None) -> list[str]:
    """One hipcc line that compiles and links every source."""
    return [HIPCC, *FLAGS, *(extra or []), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *SOURCES, "-o", out]


def build(extra: list[str] | None = None, out: str = LIB) -> str:
    """Compile each source to an object in parallel, then link the library."""
    tmp = out + ".tmp%d" % os.getpid()
    objs = ["%s.%d.o" % (tmp, i) for i in range(len(SOURCES))]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    procs = [subprocess.Popen([HIPCC, *compile_flags, *(extra or []), "-c", "-I",
                               os.path.join(ROOT, "include"), "-I", CSRC, src, "-o", obj])
             for src, obj in zip(SOURCES, objs)]
    codes = [p.wait() for p in procs]
    try:
        if any(codes):
            raise subprocess.CalledProcessError(max(codes), "hipcc -c")
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       check=True)
        os.replace(tmp, out)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return out


def device_asm(src: str, out: str, extra: list[str] | None = None) -> str:
    """The gfx950 assembly of one source's device code, built with the
    library's flags (no host pass, no link)."""
    flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([HIPCC, *flags, *(extra or []), "--cuda-device-only", "-S", "-I",
                    os.path.join(ROOT, "include"), "-I", CSRC, src, "-o", out], check=True)
    return out


if __name__ == "__main__":
    print(build())
