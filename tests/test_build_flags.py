"""The device code is built without packed fp32 VALU instructions.

hipcc pairs ordinary float operations into v_pk_add_f32 / v_pk_mul_f32 /
v_pk_fma_f32 by itself unless the target feature is switched off; the build
switches it off.  This compiles every source of the library for the gfx950
device (assembly text, no GPU needed) and checks that none of those three
instructions appears, and that the flag is what keeps them out: a small
float2 kernel compiled with and without it.
"""

import os
import re
import subprocess
import tempfile

import pytest

from exact_tiled_attention_14_amd import build

PACKED = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")

PROBE = """
#include <hip/hip_runtime.h>
__global__ void k(float2* a, const float2* b, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) { float2 x = a[i], y = b[i]; x.x = x.x * y.x + 1.5f; x.y = x.y * y.y + 1.5f; a[i] = x; }
}
"""


def _hipcc_available():
    return os.path.exists(build._hipcc())


pytestmark = pytest.mark.skipif(not _hipcc_available(), reason="hipcc not installed")


@pytest.mark.parametrize("src", build.SOURCES)
def test_sources_have_no_packed_fp32(src):
    with tempfile.TemporaryDirectory() as d:
        asm = open(build.device_asm(src, os.path.join(d, src + ".s"))).read()
    found = sorted({m.group(0) for m in PACKED.finditer(asm)})
    assert not found, f"{src}: packed fp32 instructions in the device code: {found}"


def test_flag_is_what_keeps_them_out():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "probe.hip")
        open(src, "w").write(PROBE)
        counts = []
        for flags in ([], ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]):
            out = os.path.join(d, "probe.s")
            r = subprocess.run([build._hipcc(), "--offload-arch=gfx950", "-O3", *flags, "--cuda-device-only", "-S",
                                src, "-o", out], capture_output=True, text=True)
            assert r.returncode == 0, r.stderr
            counts.append(len(PACKED.findall(open(out).read())))
    assert counts[0] > 0, "the probe no longer produces packed fp32 code without the flag"
    assert counts[1] == 0, "the flag did not remove the packed fp32 instructions"
    assert "-packed-fp32-ops" in " ".join(build.HIP_FLAGS)
