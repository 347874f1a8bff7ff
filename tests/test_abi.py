"""The C ABI without a GPU: the library loads, exports every entry point that
include/*.h declares, and rejects invalid arguments on the host (these calls
return before any HIP call, so they run on a machine with no GPU)."""

import ctypes
import glob
import math
import os
import re
import subprocess
import sys

import pytest

import exact_tiled_attention_14_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(attn.ENTRY_POINTS)


def test_library_exports_every_declared_symbol():
    lib = attn.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    assert attn.attn_status_str(0) == "ok"
    for s in range(1, 7):
        assert attn.attn_status_str(s) and attn.attn_status_str(s) != "ok"
    assert "unknown" in attn.attn_status_str(99)


# fake, 16-byte aligned, never dereferenced device addresses
P = 0x10000
GOOD = dict(q=P, k=P * 2, v=P * 3, o=P * 4, lse=P * 5, B=1, H=4, Hkv=2, N=64, d=64,
            scale=0.125, causal=0, key_lens=None, stream=None)


def call(fn, **over):
    a = dict(GOOD, **over)
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["N"], a["d"],
              a["scale"], a["causal"], a["key_lens"], a["stream"])


ENTRY = [attn.attn_fwd_bf16, attn.attn_fwd_f32, attn.attn_fwd]


@pytest.mark.parametrize("fn", ENTRY, ids=lambda f: f.__name__)
@pytest.mark.parametrize("over,status", [
    (dict(d=96), attn.ATTN_ERR_HEAD_DIM),
    (dict(d=0), attn.ATTN_ERR_HEAD_DIM),
    (dict(d=256), attn.ATTN_ERR_HEAD_DIM),
    (dict(H=3, Hkv=2), attn.ATTN_ERR_SHAPE),
    (dict(H=0), attn.ATTN_ERR_SHAPE),
    (dict(Hkv=0), attn.ATTN_ERR_SHAPE),
    (dict(B=-1), attn.ATTN_ERR_SHAPE),
    (dict(N=-5), attn.ATTN_ERR_SHAPE),
    (dict(causal=2), attn.ATTN_ERR_SHAPE),
    (dict(B=65536, H=256, Hkv=256, N=2**20), attn.ATTN_ERR_SHAPE),
    (dict(scale=math.nan), attn.ATTN_ERR_SCALE),
    (dict(scale=math.inf), attn.ATTN_ERR_SCALE),
    (dict(q=None), attn.ATTN_ERR_NULL),
    (dict(k=None), attn.ATTN_ERR_NULL),
    (dict(v=None), attn.ATTN_ERR_NULL),
    (dict(o=None), attn.ATTN_ERR_NULL),
    (dict(lse=None), attn.ATTN_ERR_NULL),
    (dict(q=P + 8), attn.ATTN_ERR_ALIGN),
    (dict(o=P + 2), attn.ATTN_ERR_ALIGN),
    (dict(lse=P + 4), attn.ATTN_ERR_ALIGN),
    (dict(key_lens=P + 4), attn.ATTN_ERR_ALIGN),
    # empty problems are a no-op and may pass NULL data pointers
    (dict(B=0, q=None, k=None, v=None, o=None, lse=None), attn.ATTN_OK),
    (dict(N=0, q=None, k=None, v=None, o=None, lse=None), attn.ATTN_OK),
])
def test_host_validation(fn, over, status):
    assert call(fn, **over) == status


def test_python_forward_rejects_bad_tensors():
    import torch
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.forward(q, q, q)            # CPU tensors
    with pytest.raises(ValueError):
        attn.forward(q[0], q, q)         # wrong rank
    with pytest.raises(TypeError):
        attn.forward(q, q.float(), q)    # mixed dtypes


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(attn, "_LIB", None)
    monkeypatch.setattr(attn, "library_path", lambda: str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        attn.load_library()


def test_one_hip_runtime_whatever_the_import_order():
    """Loading the library before torch must not bring a second HIP runtime
    into the process (torch ships its own under the same soname; a second
    one sees no device).  Checked in a fresh interpreter."""
    code = ("import exact_tiled_attention_14_amd as a; a.load_library(); import torch; "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    runtimes = eval(out.stdout.strip().splitlines()[-1])
    assert len(runtimes) == 1, runtimes


BWD_GOOD = dict(q=P, k=P * 2, v=P * 3, o=P * 4, dout=P * 5, lse=P * 6, dq=P * 7, dk=P * 8, dv=P * 9,
                delta=P * 10, B=1, H=4, Hkv=2, N=64, d=128, scale=0.125, causal=1, key_lens=None, stream=None)


def call_bwd(**over):
    a = dict(BWD_GOOD, **over)
    return attn.attn_bwd_bf16(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                              a["delta"], a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"],
                              a["key_lens"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(d=96), attn.ATTN_ERR_HEAD_DIM),
    (dict(H=3, Hkv=2), attn.ATTN_ERR_SHAPE),
    (dict(causal=-1), attn.ATTN_ERR_SHAPE),
    (dict(scale=math.inf), attn.ATTN_ERR_SCALE),
    (dict(q=None), attn.ATTN_ERR_NULL),
    (dict(dq=None), attn.ATTN_ERR_NULL),
    (dict(lse=None), attn.ATTN_ERR_NULL),
    (dict(o=None), attn.ATTN_ERR_NULL),
    (dict(dout=None), attn.ATTN_ERR_NULL),
    (dict(dk=None), attn.ATTN_ERR_NULL),
    (dict(dv=None), attn.ATTN_ERR_NULL),
    (dict(delta=None), attn.ATTN_ERR_NULL),
    (dict(dout=P + 8), attn.ATTN_ERR_ALIGN),
    (dict(dv=P + 2), attn.ATTN_ERR_ALIGN),
    (dict(delta=P + 4), attn.ATTN_ERR_ALIGN),
    (dict(B=0, q=None, k=None, v=None, o=None, dout=None, lse=None, dq=None, dk=None, dv=None, delta=None),
     attn.ATTN_OK),
])
def test_backward_host_validation(over, status):
    assert call_bwd(**over) == status


VAR_GOOD = dict(q=P, k=P * 2, v=P * 3, o=P * 4, lse=P * 5, cu=P * 6, B=3, H=4, Hkv=2, total=300,
                max_seqlen=200, d=128, scale=0.125, causal=1, stream=None)


def call_varlen(**over):
    a = dict(VAR_GOOD, **over)
    return attn.attn_fwd_varlen_bf16(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["B"], a["H"], a["Hkv"],
                                     a["total"], a["max_seqlen"], a["d"], a["scale"], a["causal"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(d=96), attn.ATTN_ERR_HEAD_DIM),
    (dict(H=3, Hkv=2), attn.ATTN_ERR_SHAPE),
    (dict(B=-1), attn.ATTN_ERR_SHAPE),
    (dict(total=-1), attn.ATTN_ERR_SHAPE),
    (dict(max_seqlen=-1), attn.ATTN_ERR_SHAPE),
    (dict(causal=2), attn.ATTN_ERR_SHAPE),
    # one sequence's query rows must be addressable with 32-bit byte offsets
    (dict(H=64, Hkv=64, max_seqlen=2**17 - 128), attn.ATTN_ERR_SHAPE),
    (dict(scale=math.nan), attn.ATTN_ERR_SCALE),
    (dict(q=None), attn.ATTN_ERR_NULL),
    (dict(lse=None), attn.ATTN_ERR_NULL),
    (dict(cu=None), attn.ATTN_ERR_NULL),
    (dict(k=P + 8), attn.ATTN_ERR_ALIGN),
    (dict(cu=P + 2), attn.ATTN_ERR_ALIGN),
    # int32 offsets only need their natural alignment
    (dict(B=0, cu=P + 4, q=None, k=None, v=None, o=None, lse=None), attn.ATTN_OK),
    # empty problems are a no-op and may pass NULL pointers
    (dict(B=0, q=None, k=None, v=None, o=None, lse=None, cu=None), attn.ATTN_OK),
    (dict(total=0, q=None, k=None, v=None, o=None, lse=None, cu=None), attn.ATTN_OK),
    (dict(max_seqlen=0, q=None, k=None, v=None, o=None, lse=None, cu=None), attn.ATTN_OK),
])
def test_varlen_host_validation(over, status):
    assert call_varlen(**over) == status


def test_python_forward_varlen_rejects_bad_tensors():
    import torch
    q = torch.zeros(8, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    with pytest.raises(ValueError):
        attn.forward_varlen(q, q, q, cu, 8)              # CPU tensors
    with pytest.raises(ValueError):
        attn.forward_varlen(q[None], q, q, cu, 8)        # wrong rank


PART_GOOD = dict(q=P, k=P * 2, v=P * 3, o=P * 4, lse=P * 5, B=2, H=4, Hkv=2, Nq=100, Nk=300, d=64, scale=0.125,
                 causal=1, q_offset=200, k_offset=0, stream=None)


def call_partial(**over):
    a = dict(PART_GOOD, **over)
    return attn.attn_fwd_partial_bf16(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["Nq"],
                                      a["Nk"], a["d"], a["scale"], a["causal"], a["q_offset"], a["k_offset"],
                                      a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(d=32), attn.ATTN_ERR_HEAD_DIM),
    (dict(Nk=-1), attn.ATTN_ERR_SHAPE),
    (dict(Nq=-1), attn.ATTN_ERR_SHAPE),
    (dict(Nk=2**23), attn.ATTN_ERR_SHAPE),
    (dict(H=4, Hkv=3), attn.ATTN_ERR_SHAPE),
    (dict(scale=math.inf), attn.ATTN_ERR_SCALE),
    (dict(k=None), attn.ATTN_ERR_NULL),
    (dict(o=None), attn.ATTN_ERR_NULL),
    (dict(v=P + 8), attn.ATTN_ERR_ALIGN),
    (dict(B=0, q=None, k=None, v=None, o=None, lse=None), attn.ATTN_OK),
    (dict(Nq=0, q=None, k=None, v=None, o=None, lse=None), attn.ATTN_OK),
])
def test_partial_host_validation(over, status):
    assert call_partial(**over) == status


MERGE_GOOD = dict(op=P, lp=P * 2, S=3, B=2, H=4, N=100, d=128, o=P * 3, o_bf16=1, lse=P * 4, stream=None)


def call_merge(**over):
    a = dict(MERGE_GOOD, **over)
    return attn.attn_merge(a["op"], a["lp"], a["S"], a["B"], a["H"], a["N"], a["d"], a["o"], a["o_bf16"], a["lse"],
                           a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(S=0), attn.ATTN_ERR_SHAPE),
    (dict(o_bf16=2), attn.ATTN_ERR_SHAPE),
    (dict(H=0), attn.ATTN_ERR_SHAPE),
    (dict(d=96), attn.ATTN_ERR_HEAD_DIM),
    (dict(op=None), attn.ATTN_ERR_NULL),
    (dict(lse=None), attn.ATTN_ERR_NULL),
    (dict(lp=P + 4), attn.ATTN_ERR_ALIGN),
    (dict(N=0, op=None, lp=None, o=None, lse=None), attn.ATTN_OK),
])
def test_merge_host_validation(over, status):
    assert call_merge(**over) == status


def test_splitkv_workspace_bytes():
    # bf16 partial O (d values) and an fp32 partial LSE per row and range
    assert attn.attn_splitkv_workspace_bytes(2, 4, 1000, 64, 3) == 3 * 2 * 4 * 1000 * (64 * 2 + 4)
    assert attn.attn_splitkv_workspace_bytes(2, 4, 1000, 64, 0) == 0
    assert attn.attn_splitkv_workspace_bytes(2, 4, 1000, 64, attn.ATTN_MAX_SPLITS + 1) == 0
    assert attn.attn_splitkv_workspace_bytes(2, 4, 1000, 96, 2) == 0


SPLIT_GOOD = dict(GOOD, Nq=200, Nk=1000, q_offset=800, k_offset=0, ns=4, ws=P * 8,
                  wsb=attn.attn_splitkv_workspace_bytes(1, 4, 200, 64, 4))


def call_split(**over):
    a = dict(SPLIT_GOOD, **over)
    return attn.attn_fwd_splitkv_bf16(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["Nq"],
                                      a["Nk"], a["d"], a["scale"], a["causal"], a["q_offset"], a["k_offset"],
                                      a["key_lens"], a["ns"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(ns=0), attn.ATTN_ERR_SHAPE),
    (dict(ns=attn.ATTN_MAX_SPLITS + 1), attn.ATTN_ERR_SHAPE),
    (dict(d=80), attn.ATTN_ERR_HEAD_DIM),
    (dict(q=None), attn.ATTN_ERR_NULL),
    (dict(ws=None), attn.ATTN_ERR_WORKSPACE),
    (dict(wsb=100), attn.ATTN_ERR_WORKSPACE),
    (dict(ws=P * 8 + 4), attn.ATTN_ERR_ALIGN),
    (dict(Nk=-3), attn.ATTN_ERR_SHAPE),
    (dict(B=0, q=None, k=None, v=None, o=None, lse=None, ws=None), attn.ATTN_OK),
    # one range (Nk <= 128): the plain forward pass, no workspace needed
    (dict(Nk=100, ws=None, wsb=0, q=None), attn.ATTN_ERR_NULL),
])
def test_splitkv_host_validation(over, status):
    assert call_split(**over) == status


FP8_GOOD = dict(GOOD, N=64, qd=0.01, kd=0.02, vd=0.03)


def call_fp8(**over):
    a = dict(FP8_GOOD, **over)
    return attn.attn_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["qd"], a["kd"], a["vd"], a["B"], a["H"],
                             a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], a["key_lens"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(N=-1), attn.ATTN_ERR_SHAPE),
    (dict(d=96), attn.ATTN_ERR_HEAD_DIM),
    (dict(qd=math.nan), attn.ATTN_ERR_SCALE),
    (dict(vd=math.inf), attn.ATTN_ERR_SCALE),
    (dict(scale=1e30, qd=1e30), attn.ATTN_ERR_SCALE),  # the combined score scale overflows
    (dict(H=3, Hkv=2), attn.ATTN_ERR_SHAPE),
    (dict(v=None), attn.ATTN_ERR_NULL),
    (dict(k=P + 4), attn.ATTN_ERR_ALIGN),
    (dict(B=0, q=None, k=None, v=None, o=None, lse=None), attn.ATTN_OK),
    (dict(N=0, q=None, k=None, v=None, o=None, lse=None), attn.ATTN_OK),
])
def test_fp8_host_validation(over, status):
    assert call_fp8(**over) == status


@pytest.mark.parametrize("call,status", [
    # attn_fp8_amax(x, signs, rows, d, amax, stream)
    (lambda: attn.attn_fp8_amax(P, None, -1, 64, P, None), attn.ATTN_ERR_SHAPE),
    (lambda: attn.attn_fp8_amax(P, None, 1 << 47, 64, P, None), attn.ATTN_ERR_SHAPE),
    (lambda: attn.attn_fp8_amax(P, None, 4, 96, P, None), attn.ATTN_ERR_HEAD_DIM),
    (lambda: attn.attn_fp8_amax(P, None, 4, 64, None, None), attn.ATTN_ERR_NULL),
    (lambda: attn.attn_fp8_amax(None, None, 4, 64, P, None), attn.ATTN_ERR_NULL),
    (lambda: attn.attn_fp8_amax(P + 8, None, 4, 64, P, None), attn.ATTN_ERR_ALIGN),
    (lambda: attn.attn_fp8_amax(P, P + 4, 4, 64, P, None), attn.ATTN_ERR_ALIGN),
    (lambda: attn.attn_fp8_amax(P, None, 4, 64, P + 2, None), attn.ATTN_ERR_ALIGN),
    # attn_fp8_quantize(x, signs, rows, d, amax, x8, descale, stream)
    (lambda: attn.attn_fp8_quantize(P, None, -5, 128, P, P, P, None), attn.ATTN_ERR_SHAPE),
    (lambda: attn.attn_fp8_quantize(P, None, 4, 32, P, P, P, None), attn.ATTN_ERR_HEAD_DIM),
    (lambda: attn.attn_fp8_quantize(P, None, 4, 128, P, None, P, None), attn.ATTN_ERR_NULL),
    (lambda: attn.attn_fp8_quantize(P, None, 4, 128, P, P, None, None), attn.ATTN_ERR_NULL),
    (lambda: attn.attn_fp8_quantize(P, None, 4, 128, P, P + 8, P, None), attn.ATTN_ERR_ALIGN),
    # attn_fp8_quantize_vt(v, heads, N, d, amax, vt8, descale, stream)
    (lambda: attn.attn_fp8_quantize_vt(P, -1, 64, 64, P, P, P, None), attn.ATTN_ERR_SHAPE),
    (lambda: attn.attn_fp8_quantize_vt(P, 2, -1, 64, P, P, P, None), attn.ATTN_ERR_SHAPE),
    (lambda: attn.attn_fp8_quantize_vt(P, 2, 64, 100, P, P, P, None), attn.ATTN_ERR_HEAD_DIM),
    (lambda: attn.attn_fp8_quantize_vt(None, 2, 64, 64, P, P, P, None), attn.ATTN_ERR_NULL),
    (lambda: attn.attn_fp8_quantize_vt(P, 2, 64, 64, P, P + 4, P, None), attn.ATTN_ERR_ALIGN),
])
def test_fp8_prep_host_validation(call, status):
    assert call() == status


def test_noalloc_backward_host_validation():
    """attn_bwd_bf16_noalloc: the checks of attn_bwd_bf16, then the size of
    the built-in scratch (2·B·H·N floats), all before any HIP call."""
    f = attn.attn_bwd_bf16_noalloc
    args = [P] * 9 + [1, 2, 1, 64, 64, 0.125, 0, None, None]

    def call(**kw):
        a = list(args)
        names = ["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "B", "H", "Hkv", "N", "d"]
        for key, val in kw.items():
            a[names.index(key)] = val
        return f(*a)

    assert call(d=96) == attn.ATTN_ERR_HEAD_DIM
    assert call(H=3, Hkv=2) == attn.ATTN_ERR_SHAPE
    assert call(dout=None) == attn.ATTN_ERR_NULL
    assert call(dv=P + 4) == attn.ATTN_ERR_ALIGN
    assert call(B=0) == attn.ATTN_OK
    limit = attn.ATTN_NOALLOC_SCRATCH_FLOATS
    assert call(B=1, H=1, N=limit // 2 + 1) == attn.ATTN_ERR_SCRATCH
    assert call(B=4, H=32, N=limit // 256 + 1) == attn.ATTN_ERR_SCRATCH
    assert attn.ATTN_ERR_SCRATCH == 8 and "scratch" in attn.attn_status_str(attn.ATTN_ERR_SCRATCH)


def test_fp8_quantisation_recipe():
    """The test-input quantiser: values within half an e4m3 step, no NaN
    from out-of-range magnitudes, max maps to 448."""
    import torch

    from workloads import quantize_fp8
    x = torch.tensor([0.0, 1.0, -3.0, 7.5, 1e-6])
    s, d = quantize_fp8(x)
    back = s.float() * d
    assert not torch.isnan(back).any()
    assert abs(float(s.float().abs().max()) - 448.0) == 0.0
    assert torch.all((back - x).abs() <= x.abs() * 2.0 ** -4 + d * 2.0 ** -10)
