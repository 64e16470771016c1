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
SOURCES = [os.path.join(CSRC, "fmha_api.hip")]
HEADERS = [os.path.join(CSRC, "fmha_fwd_kernel.hpp"), os.path.join(ROOT, "include", "fmha.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU forms in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def command(out: str = LIB, extra: list[str] | None = None) -> list[str]:
    return [HIPCC, *FLAGS, *(extra or []), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *SOURCES, "-o", out]


def build(extra: list[str] | None = None, out: str = LIB) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(command(tmp, extra), check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
