"""The library's gfx950 device code, compiled here on the CPU with the
library's own flags, holds no packed-fp32 VALU instruction (v_pk_fma_f32,
v_pk_mul_f32, v_pk_add_f32 and kin): the build turns the feature off, and
this test checks that it took effect on every kernel. A control build of a
tiny kernel without that flag shows the check can see such instructions."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from software_pipelining_fmha_amd import build

PK_F32 = re.compile(r"^\s*v_pk_\w+_f32\b", re.M)

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="no hipcc")


def test_no_packed_fp32_in_device_code(tmp_path):
    outs = [str(tmp_path / (os.path.basename(s) + ".s")) for s in build.SOURCES]
    with ThreadPoolExecutor(len(outs)) as ex:
        list(ex.map(build.device_asm, build.SOURCES, outs))
    for out in outs:
        text = open(out).read()
        assert "mfma" in text or "ws_gemm" not in out, out  # real kernels were built
        found = PK_F32.findall(text)
        assert not found, "%s: %s" % (os.path.basename(out), sorted(set(found)))


def test_control_build_shows_packed_fp32(tmp_path):
    """float2 a*x+b compiles to v_pk_fma_f32 unless the feature is off."""
    src = tmp_path / "pk.hip"
    src.write_text(
        "#include <hip/hip_runtime.h>\n"
        "__global__ void k(float2* x, float a, float b) {\n"
        "  float2 v = x[threadIdx.x]; v.x = v.x * a + b; v.y = v.y * a + b;\n"
        "  x[threadIdx.x] = v;\n}\n")
    off = tmp_path / "off.s"
    build.device_asm(str(src), str(off))
    assert not PK_F32.findall(off.read_text())
    # the same kernel without the four tokens that turn the feature off
    feature = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    i = next(i for i in range(len(flags)) if flags[i:i + 4] == feature)
    on = tmp_path / "on.s"
    subprocess.run([build.HIPCC, *flags[:i], *flags[i + 4:], "--cuda-device-only", "-S",
                    str(src), "-o", str(on)], check=True)
    assert PK_F32.findall(on.read_text()), "control build has no packed fp32"
