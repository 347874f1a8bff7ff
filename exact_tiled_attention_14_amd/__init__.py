"""Python binding of the MI355X exact tiled attention library.

Thin ctypes layer over ``libattn.so`` (see ``include/attn.h``): the functions
``attn_fwd_bf16``, ``attn_fwd_f32``, ``attn_fwd``, ``attn_fwd_varlen_bf16``,
``attn_fwd_partial_bf16``, ``attn_merge``, ``attn_fwd_splitkv_bf16``,
``attn_splitkv_workspace_bytes``, ``attn_bwd_bf16``, ``attn_fwd_fp8``,
``attn_fp8_amax``, ``attn_fp8_quantize``, ``attn_fp8_quantize_vt`` and
``attn_status_str``
take the same arguments as the C entry points (device pointers as Python
ints) and return what they return.  ``forward``, ``forward_varlen``,
``forward_partial``, ``merge``, ``forward_splitkv``, ``forward_fp8``,
``quantize_fp8``, ``quantize_fp8_vt`` and ``backward`` marshal
torch tensors onto them; every step of the computation
runs in the HIP kernels.  There is no fallback: if the library is missing,
every call raises.
"""

import ctypes
import math
import os

__all__ = [
    "AttnError", "attn_fwd", "attn_fwd_bf16", "attn_fwd_f32", "attn_fwd_varlen_bf16", "attn_bwd_bf16",
    "attn_fwd_fp8", "forward_fp8", "attn_fp8_amax", "attn_fp8_quantize", "attn_fp8_quantize_vt",
    "quantize_fp8", "quantize_fp8_vt", "hadamard_signs", "attn_fwd_partial_bf16", "attn_merge", "attn_fwd_splitkv_bf16", "attn_splitkv_workspace_bytes",
    "attn_status_str", "forward", "forward_varlen", "forward_partial", "merge", "forward_splitkv", "backward",
    "library_path", "load_library", "ATTN_ERR_WORKSPACE", "ATTN_MAX_SPLITS",
    "ATTN_OK", "ATTN_ERR_NULL", "ATTN_ERR_SHAPE", "ATTN_ERR_HEAD_DIM", "ATTN_ERR_ALIGN",
    "ATTN_ERR_SCALE", "ATTN_ERR_HIP", "ATTN_ERR_SCRATCH", "ATTN_NOALLOC_SCRATCH_FLOATS", "attn_bwd_bf16_noalloc",
]

ATTN_OK, ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_HEAD_DIM = 0, 1, 2, 3
ATTN_ERR_ALIGN, ATTN_ERR_SCALE, ATTN_ERR_HIP, ATTN_ERR_WORKSPACE, ATTN_ERR_SCRATCH = 4, 5, 6, 7, 8
ATTN_NOALLOC_SCRATCH_FLOATS = 4 * 1024 * 1024
ATTN_MAX_SPLITS = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

# (name, argtypes) of every exported entry point, matching include/attn.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_FWD_ARGS = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P]
ENTRY_POINTS = {
    "attn_fwd_bf16": (_FWD_ARGS, ctypes.c_int),
    "attn_fwd_f32": (_FWD_ARGS, ctypes.c_int),
    "attn_fwd": (_FWD_ARGS, ctypes.c_int),
    "attn_fwd_varlen_bf16": ([_P] * 6 + [_I] * 6 + [ctypes.c_float, _I, _P], ctypes.c_int),
    "attn_fwd_partial_bf16": ([_P] * 5 + [_I] * 6 + [ctypes.c_float, _I, _I, _I, _P], ctypes.c_int),
    "attn_merge": ([_P, _P] + [_I] * 5 + [_P, _I, _P, _P], ctypes.c_int),
    "attn_fwd_splitkv_bf16": ([_P] * 5 + [_I] * 6 + [ctypes.c_float, _I, _I, _I, _P, _I, _P, ctypes.c_size_t, _P],
                              ctypes.c_int),
    "attn_splitkv_workspace_bytes": ([_I] * 5, ctypes.c_size_t),
    "attn_fwd_fp8": ([_P] * 5 + [ctypes.c_float] * 3 + [_I] * 5 + [ctypes.c_float, _I, _P, _P], ctypes.c_int),
    "attn_bwd_bf16": ([_P] * 10 + [_I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P], ctypes.c_int),
    "attn_bwd_bf16_noalloc": ([_P] * 9 + [_I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P], ctypes.c_int),
    "attn_fp8_amax": ([_P, _P, ctypes.c_int64, _I, _P, _P], ctypes.c_int),
    "attn_fp8_quantize": ([_P, _P, ctypes.c_int64, _I, _P, _P, _P, _P], ctypes.c_int),
    "attn_fp8_quantize_vt": ([_P, ctypes.c_int64, _I, _I, _P, _P, _P, _P], ctypes.c_int),
    "attn_status_str": ([_I], ctypes.c_char_p),
    "attn_last_hip_error": ([], ctypes.c_char_p),
}


class AttnError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status, where):
        self.status = status
        text = f"{where}: status {status} ({attn_status_str(status)})"
        if status == ATTN_ERR_HIP:
            text += ": " + load_library().attn_last_hip_error().decode()
        super().__init__(text)


def library_path():
    return os.path.join(_HERE, "libattn.so")


def load_library():
    """Load libattn.so (built by ``exact_tiled_attention_14_amd.build``)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it first (python -m exact_tiled_attention_14_amd.build); "
                "there is no fallback implementation")
        # PyTorch-ROCm carries its own HIP and HSA runtimes under the same
        # sonames as /opt/rocm's.  Loaded first, they satisfy the library's
        # libamdhip64.so.7 dependency and the process has one runtime; loaded
        # after the library, a second pair comes in beside it, and the
        # library's runtime then finds no device (hipErrorNoDevice).
        import torch  # noqa: F401

        lib = ctypes.CDLL(path)
        for name, (argtypes, restype) in ENTRY_POINTS.items():
            fn = getattr(lib, name)
            fn.argtypes = argtypes
            fn.restype = restype
        _LIB = lib
    return _LIB


def attn_fwd_bf16(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, key_lens, stream):
    return load_library().attn_fwd_bf16(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, key_lens, stream)


def attn_fwd_f32(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, key_lens, stream):
    return load_library().attn_fwd_f32(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, key_lens, stream)


def attn_fwd(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, key_lens, stream):
    return load_library().attn_fwd(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, key_lens, stream)


def attn_fwd_varlen_bf16(q, k, v, o, lse, cu_seqlens, B, H, Hkv, total, max_seqlen, d, scale, causal, stream):
    return load_library().attn_fwd_varlen_bf16(q, k, v, o, lse, cu_seqlens, B, H, Hkv, total, max_seqlen,
                                               d, scale, causal, stream)


def attn_fwd_partial_bf16(q, k, v, o_part, lse_part, B, H, Hkv, Nq, Nk, d, scale, causal, q_offset, k_offset,
                          stream):
    return load_library().attn_fwd_partial_bf16(q, k, v, o_part, lse_part, B, H, Hkv, Nq, Nk, d, scale, causal,
                                                q_offset, k_offset, stream)


def attn_fwd_fp8(q, k, vt, o, lse, q_descale, k_descale, v_descale, B, H, Hkv, N, d, scale, causal, key_lens,
                 stream):
    return load_library().attn_fwd_fp8(q, k, vt, o, lse, q_descale, k_descale, v_descale, B, H, Hkv, N, d, scale,
                                       causal, key_lens, stream)


def attn_fp8_amax(x, signs, rows, d, amax, stream):
    return load_library().attn_fp8_amax(x, signs, rows, d, amax, stream)


def attn_fp8_quantize(x, signs, rows, d, amax, x8, descale, stream):
    return load_library().attn_fp8_quantize(x, signs, rows, d, amax, x8, descale, stream)


def attn_fp8_quantize_vt(v, heads, N, d, amax, vt8, descale, stream):
    return load_library().attn_fp8_quantize_vt(v, heads, N, d, amax, vt8, descale, stream)


def attn_merge(o_parts, lse_parts, S, B, H, N, d, o, o_bf16, lse, stream):
    return load_library().attn_merge(o_parts, lse_parts, S, B, H, N, d, o, o_bf16, lse, stream)


def attn_fwd_splitkv_bf16(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, q_offset, k_offset, key_lens,
                          num_splits, workspace, workspace_bytes, stream):
    return load_library().attn_fwd_splitkv_bf16(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, q_offset,
                                                k_offset, key_lens, num_splits, workspace, workspace_bytes, stream)


def attn_splitkv_workspace_bytes(B, H, N, d, num_splits):
    return load_library().attn_splitkv_workspace_bytes(B, H, N, d, num_splits)


def attn_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Hkv, N, d, scale, causal, key_lens, stream):
    return load_library().attn_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, delta,
                                        B, H, Hkv, N, d, scale, causal, key_lens, stream)


def attn_bwd_bf16_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, key_lens, stream):
    return load_library().attn_bwd_bf16_noalloc(q, k, v, o, dout, lse, dq, dk, dv,
                                                B, H, Hkv, N, d, scale, causal, key_lens, stream)


def attn_status_str(status):
    return load_library().attn_status_str(int(status)).decode()


def forward(q, k, v, *, scale=None, causal=False, key_lens=None, out=None, lse=None, stream=None):
    """Run the forward pass on torch tensors already on the GPU.

    q: [B, H, N, d]; k, v: [B, Hkv, N, d]; all bf16 or all fp32, contiguous.
    key_lens: None or an int32 CUDA tensor [B].  scale defaults to 1/sqrt(d).
    Returns (o, lse): o like q, lse fp32 [B, H, N].  The launch is enqueued on
    ``stream`` (default: torch's current stream of q's device) and not waited on.
    """
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D: [B, H, N, d] and [B, Hkv, N, d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q, k, v must all be bfloat16 or all float32")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if key_lens is not None:
        if key_lens.dtype != torch.int32 or not key_lens.is_cuda or key_lens.numel() != B:
            raise ValueError("key_lens must be an int32 GPU tensor with B entries")
        key_lens = key_lens.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    fn = attn_fwd_bf16 if q.dtype == torch.bfloat16 else attn_fwd_f32
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            B, H, Hkv, N, d, float(scale), int(bool(causal)),
            key_lens.data_ptr() if key_lens is not None else None, stream)
    if st != ATTN_OK:
        raise AttnError(st, fn.__name__)
    return out, lse


def forward_varlen(q, k, v, cu_seqlens, max_seqlen, *, scale=None, causal=False, out=None, lse=None,
                   stream=None):
    """Forward pass over packed sequences (bf16 GPU tensors).

    q: [total, H, d]; k, v: [total, Hkv, d]; cu_seqlens: int32 GPU tensor [B + 1]
    of sequence offsets (0 = cu[0] <= cu[1] <= ... <= cu[B] = total); every
    sequence length at most ``max_seqlen`` (an int: the device offsets are not
    read on the host).  Returns (o, lse): o [total, H, d] bf16, lse fp32
    [H, total].  Enqueued on ``stream`` (default: torch's current stream).
    """
    import torch

    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D: [total, H, d] and [total, Hkv, d]")
    total, H, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (total, Hkv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 GPU tensor")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 GPU tensor [B + 1]")
    cu_seqlens = cu_seqlens.contiguous()
    B = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_fwd_varlen_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                              cu_seqlens.data_ptr(), B, H, Hkv, total, int(max_seqlen), d, float(scale),
                              int(bool(causal)), stream)
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_varlen_bf16")
    return out, lse


def _check_bf16(**tensors):
    import torch

    for name, t in tensors.items():
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 GPU tensor")


def forward_fp8(q, k, vt, q_descale, k_descale, v_descale, *, scale=None, causal=False, key_lens=None,
                stream=None):
    """FP8 forward: q [B, H, N, d], k [B, Hkv, N, d], vt [B, Hkv, d, N16] (V
    transposed, N16 = N rounded up to a multiple of 16) as
    torch.float8_e4m3fn GPU tensors standing for descale · stored value.
    Returns (o bf16 [B, H, N, d], lse fp32 [B, H, N])."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or vt.dim() != 4:
        raise ValueError("q, k, vt must be 4-D")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    n16 = (N + 15) // 16 * 16
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(vt.shape) != (B, Hkv, d, n16):
        raise ValueError("shape mismatch: k must be [B, Hkv, N, d] and vt [B, Hkv, d, N16] (N16 = N rounded up "
                         "to a multiple of 16)")
    for name, t in (("q", q), ("k", k), ("vt", vt)):
        if t.dtype != torch.float8_e4m3fn or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float8_e4m3fn GPU tensor")
    if key_lens is not None:
        if key_lens.dtype != torch.int32 or not key_lens.is_cuda or key_lens.numel() != B:
            raise ValueError("key_lens must be an int32 GPU tensor with B entries")
        key_lens = key_lens.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_fwd_fp8(q.data_ptr(), k.data_ptr(), vt.data_ptr(), o.data_ptr(), lse.data_ptr(), float(q_descale),
                      float(k_descale), float(v_descale), B, H, Hkv, N, d, float(scale), int(bool(causal)),
                      key_lens.data_ptr() if key_lens is not None else None, stream)
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_fp8")
    return o, lse


def hadamard_signs(d, seed, device):
    """d random signs (+1 / -1, fp32) for the incoherent-processing rotation,
    drawn on the CPU by a torch.Generator seeded with ``seed`` and copied to
    ``device``."""
    import torch

    g = torch.Generator("cpu").manual_seed(int(seed))
    s = torch.randint(0, 2, (d,), generator=g, dtype=torch.int32).float() * 2.0 - 1.0
    return s.to(device)


def quantize_fp8(x, signs=None, *, stream=None):
    """Per-tensor fp8 e4m3 quantisation of a bf16 GPU tensor [..., d] on the
    GPU (attn_fp8_amax, then attn_fp8_quantize), each row first rotated by
    R = H_d · diag(signs) / sqrt(d) when ``signs`` (fp32 GPU tensor [d]) is
    given.  Returns (x8 float8_e4m3fn like x, descale float).  Reading the
    descale back waits for the two kernels."""
    import torch

    _check_bf16(x=x)
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if signs is not None and (signs.dtype != torch.float32 or not signs.is_cuda or signs.numel() != d
                              or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous float32 GPU tensor with d entries")
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    scal = torch.empty(8, dtype=torch.float32, device=x.device)  # [0] amax, [4] descale (16-byte apart)
    x8 = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    sp = signs.data_ptr() if signs is not None else None
    st = attn_fp8_amax(x.data_ptr(), sp, rows, d, scal.data_ptr(), stream)
    if st != ATTN_OK:
        raise AttnError(st, "attn_fp8_amax")
    st = attn_fp8_quantize(x.data_ptr(), sp, rows, d, scal.data_ptr(), x8.data_ptr(), scal[4:].data_ptr(), stream)
    if st != ATTN_OK:
        raise AttnError(st, "attn_fp8_quantize")
    return x8, float(scal[4].item())


def quantize_fp8_vt(v, *, stream=None):
    """V [B, Hkv, N, d] bf16 (GPU) to its transposed fp8 form for forward_fp8:
    (vt8 float8_e4m3fn [B, Hkv, d, N16], descale float), per-tensor scale,
    on the GPU (attn_fp8_amax, then attn_fp8_quantize_vt)."""
    import torch

    _check_bf16(v=v)
    if v.dim() != 4:
        raise ValueError("v must be [B, Hkv, N, d]")
    B, Hkv, N, d = v.shape
    n16 = (N + 15) // 16 * 16
    if stream is None:
        stream = torch.cuda.current_stream(v.device).cuda_stream
    scal = torch.empty(8, dtype=torch.float32, device=v.device)
    vt8 = torch.empty((B, Hkv, d, n16), dtype=torch.float8_e4m3fn, device=v.device)
    st = attn_fp8_amax(v.data_ptr(), None, B * Hkv * N, d, scal.data_ptr(), stream)
    if st != ATTN_OK:
        raise AttnError(st, "attn_fp8_amax")
    st = attn_fp8_quantize_vt(v.data_ptr(), B * Hkv, N, d, scal.data_ptr(), vt8.data_ptr(), scal[4:].data_ptr(),
                              stream)
    if st != ATTN_OK:
        raise AttnError(st, "attn_fp8_quantize_vt")
    return vt8, float(scal[4].item())


def forward_partial(q, k, v, *, q_offset=0, k_offset=0, scale=None, causal=False, stream=None):
    """Attention of q [B, H, Nq, d] over one key block k, v [B, Hkv, Nk, d]
    (bf16 GPU tensors) whose first query / key sit at positions q_offset /
    k_offset.  Returns (o_part fp32 [B, H, Nq, d], lse_part fp32 [B, H, Nq])."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch")
    _check_bf16(q=q, k=k, v=v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, H, Nq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_fwd_partial_bf16(q.data_ptr(), k.data_ptr() if Nk else None, v.data_ptr() if Nk else None,
                               o.data_ptr(), lse.data_ptr(), B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                               int(q_offset), int(k_offset), stream)
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_partial_bf16")
    return o, lse


def merge(o_parts, lse_parts, *, out_dtype=None, stream=None):
    """Combine partials o_parts fp32 [S, B, H, N, d], lse_parts fp32
    [S, B, H, N] into (o [B, H, N, d] of out_dtype (bf16 default), lse fp32)."""
    import torch

    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    S, B, H, N, d = o_parts.shape
    for name, t in (("o_parts", o_parts), ("lse_parts", lse_parts)):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor")
    if tuple(lse_parts.shape) != (S, B, H, N):
        raise ValueError("lse_parts shape mismatch")
    o = torch.empty((B, H, N, d), dtype=out_dtype, device=o_parts.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=o_parts.device)
    if stream is None:
        stream = torch.cuda.current_stream(o_parts.device).cuda_stream
    st = attn_merge(o_parts.data_ptr(), lse_parts.data_ptr(), S, B, H, N, d, o.data_ptr(),
                    int(out_dtype == torch.bfloat16), lse.data_ptr(), stream)
    if st != ATTN_OK:
        raise AttnError(st, "attn_merge")
    return o, lse


def forward_splitkv(q, k, v, num_splits, *, q_offset=0, k_offset=0, scale=None, causal=False, key_lens=None):
    """Attention of q [B, H, Nq, d] over k, v [B, Hkv, Nk, d] (bf16 GPU
    tensors; positions as in forward_partial) computed over ``num_splits``
    key ranges and merged.  Returns (o bf16 [B, H, Nq, d], lse fp32
    [B, H, Nq]).  The workspace is a torch allocation released when this
    returns; the launches go to torch's current stream, which orders them
    before any later reuse of that memory."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch")
    _check_bf16(q=q, k=k, v=v)
    if key_lens is not None:
        if key_lens.dtype != torch.int32 or not key_lens.is_cuda or key_lens.numel() != B:
            raise ValueError("key_lens must be an int32 GPU tensor with B entries")
        key_lens = key_lens.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = attn_splitkv_workspace_bytes(B, H, Nq, d, int(num_splits))
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_fwd_splitkv_bf16(q.data_ptr(), k.data_ptr() if Nk else None, v.data_ptr() if Nk else None,
                               o.data_ptr(), lse.data_ptr(), B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                               int(q_offset), int(k_offset), key_lens.data_ptr() if key_lens is not None else None,
                               int(num_splits), ws.data_ptr(), nbytes, stream)
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_splitkv_bf16")
    return o, lse


def backward(q, k, v, o, lse, dout, *, scale=None, causal=False, key_lens=None, stream=None, out=None,
             builtin_scratch=False):
    """Gradients (dq, dk, dv) of sum(o * dout) for bf16 GPU tensors, where
    (o, lse) = forward(q, k, v, ...) with the same arguments.  Allocates the
    outputs (unless ``out`` = (dq, dk, dv) is given) and the fp32 [2, B, H, N]
    scratch; with ``builtin_scratch`` it calls attn_bwd_bf16_noalloc instead,
    whose scratch is built into the library, so that with ``out`` given
    nothing is allocated.  The two kernels are enqueued on ``stream``
    (default: torch's current stream) and not waited on."""
    import torch

    B, H, N, d = q.shape
    Hkv = k.shape[1]
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 GPU tensor")
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != tuple(k.shape) or o.shape != q.shape \
            or dout.shape != q.shape or tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("shape or dtype mismatch")
    if key_lens is not None:
        if key_lens.dtype != torch.int32 or not key_lens.is_cuda or key_lens.numel() != B:
            raise ValueError("key_lens must be an int32 GPU tensor with B entries")
        key_lens = key_lens.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
            if t.shape != like.shape or t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous bfloat16 GPU tensor shaped like its input")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    kl = key_lens.data_ptr() if key_lens is not None else None
    if builtin_scratch:
        st = attn_bwd_bf16_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                   lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                   B, H, Hkv, N, d, float(scale), int(bool(causal)), kl, stream)
        if st != ATTN_OK:
            raise AttnError(st, "attn_bwd_bf16_noalloc")
        return dq, dk, dv
    delta = torch.empty((2, B, H, N), dtype=torch.float32, device=q.device)
    st = attn_bwd_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                       B, H, Hkv, N, d, float(scale), int(bool(causal)), kl, stream)
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd_bf16")
    return dq, dk, dv
