"""Build step: compile the HIP sources into the in-tree shared library
``libattn.so`` for gfx950 with hipcc (cross-compiles without a GPU)."""

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
SOURCES = ["attn_api.hip", "attn_fwd_bf16.hip", "attn_fwd_f32.hip", "attn_bwd_bf16.hip", "attn_merge.hip", "attn_fwd_fp8.hip",
           "attn_fp8_prep.hip"]

# Packed fp32 VALU forms (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32) are
# turned off for the device code: without the feature flag the compiler pairs
# ordinary float operations into them by itself.  The flag acts in the gfx950
# device pass; the host pass, which has no such feature, prints a warning that
# it ignores it.  tests/test_build_flags.py compiles every source for the
# device and checks that no packed fp32 instruction is left.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def device_asm(src, out_s):
    """Compile one source file for the gfx950 device only, to assembly text."""
    cmd = [_hipcc(), *HIP_FLAGS, "-I" + INCLUDE, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out_s]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stderr}")
    return out_s


def _hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose=False):
    """Compile every source to an object and link libattn.so (always rebuilds)."""
    out = tempfile.mkdtemp(prefix="attn_build_")
    objs = []

    def compile_one(src):
        obj = os.path.join(out, src + ".o")
        cmd = [_hipcc(), *HIP_FLAGS, "-I" + INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        if verbose and r.stderr:
            sys.stderr.write(r.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
