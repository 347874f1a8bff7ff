"""Seeded synthetic inputs for the attention forward pass.

This module is shared by the tests, ``bench.py`` and ``smoke()``: it feeds the
same tensors to the GPU path and to the fp64 oracle.  It holds shapes and random
draws only — no attention arithmetic — and imports neither the oracle nor the
GPU package.

Recipe (stated once, used everywhere): a ``torch.Generator('cpu')`` seeded with
the workload's seed draws Q, K and V, in that order, as i.i.d. N(0, 1) float32
with ``torch.randn``; bf16 workloads then round them to bfloat16 (round to
nearest even).  A padded workload draws its per-sequence key lengths last from
the same generator, uniform on the integers N/2 .. N inclusive.  The softmax
scale is 1/sqrt(head_dim) rounded to float32, the value the GPU receives.
"""

import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    dtype: str          # "f32" or "bf16": storage type of q, k, v, o
    causal: bool
    padded: bool        # per-sequence key lengths with a key padding mask
    seed: int

    @property
    def scale(self):
        return float(np.float32(1.0 / math.sqrt(self.d)))


# The five workloads the attention pages' examples are sized like: a small
# fp32 single-head case, multi-head at N=1024, d_model=512 split 8x64 at
# N=4096 (the memory-wall analysis size), a long causal sequence, and a
# grouped-query padded batch.
WORKLOADS = {
    1: Workload("fp32 single-head B1 H1 N256 d64", 1, 1, 1, 256, 64, "f32", False, False, 1),
    2: Workload("mha B4 H8 N1024 d64 bf16", 4, 8, 8, 1024, 64, "bf16", False, False, 2),
    3: Workload("causal B2 H8 N4096 d64 bf16", 2, 8, 8, 4096, 64, "bf16", True, False, 3),
    4: Workload("causal long B1 H16 N16384 d128 bf16", 1, 16, 16, 16384, 128, "bf16", True, False, 4),
    5: Workload("gqa padded B2 Hq32 Hkv8 N8192 d128 bf16", 2, 32, 8, 8192, 128, "bf16", False, True, 5),
}


def make_qkv(B, H, Hkv, N, d, dtype="bf16", seed=0, padded=False):
    """Draw (q, k, v, key_lens) on the CPU following the recipe above.

    q: [B, H, N, d], k and v: [B, Hkv, N, d] as torch CPU tensors of the
    storage dtype; key_lens: int32 [B] or None."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    if dtype == "bf16":
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    key_lens = None
    if padded:
        key_lens = torch.randint(N // 2, N + 1, (B,), generator=g, dtype=torch.int32)
    return q, k, v, key_lens


def make_inputs(w: Workload):
    """Inputs of a named workload: (q, k, v, key_lens) on the CPU."""
    return make_qkv(w.B, w.H, w.Hkv, w.N, w.d, w.dtype, w.seed, w.padded)


# Packed variable-length batch (the aifi page's dynamic-sequence case, with
# the key-length mix of the padded workload: lengths uniform on N/2 .. N):
# sequences laid end to end, token-major [total, H, d], causal.
VARLEN = dict(name="packed varlen B8 lengths U[4096,8192] Hq32 Hkv8 d128 causal bf16",
              B=8, N=8192, H=32, Hkv=8, d=128, causal=True, seed=6)


# Split-KV: the last 512 positions of a 32768-token sequence (a chunk of
# queries) over its whole key cache, causal, GQA, in 16 key ranges: only
# 32 heads x 4 query tiles of work without the split.
SPLITKV = dict(name="split-KV chunk Nq512 over Nk32768 Hq32 Hkv8 d128 causal, 16 ranges, bf16",
               B=1, H=32, Hkv=8, Nq=512, Nk=32768, d=128, causal=True, splits=16, seed=7)


def make_splitkv(spec):
    """Inputs of the split-KV shape: a torch.Generator('cpu') seeded with the
    spec's seed draws q [B, H, Nq, d], then k and v [B, Hkv, Nk, d], as
    N(0, 1) float32 rounded to bf16 (the recipe above)."""
    g = torch.Generator("cpu").manual_seed(int(spec["seed"]))
    q = torch.randn((spec["B"], spec["H"], spec["Nq"], spec["d"]), generator=g).to(torch.bfloat16)
    k = torch.randn((spec["B"], spec["Hkv"], spec["Nk"], spec["d"]), generator=g).to(torch.bfloat16)
    v = torch.randn((spec["B"], spec["Hkv"], spec["Nk"], spec["d"]), generator=g).to(torch.bfloat16)
    return q, k, v


def varlen_lengths(B, lo, hi, seed):
    """B sequence lengths drawn uniformly from the integers lo .. hi inclusive
    (a torch.Generator('cpu') seeded with ``seed``)."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).tolist()


def make_varlen(lengths, H, Hkv, d, seed=0):
    """Packed bf16 inputs for the given sequence lengths, following the recipe
    above (Q, K, V drawn in that order as N(0, 1) float32, rounded to bf16):
    q [total, H, d], k and v [total, Hkv, d], and cu_seqlens int32 [B + 1]."""
    total = int(sum(lengths))
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn((total, H, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((total, Hkv, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((total, Hkv, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    cu = torch.tensor([0] + list(np.cumsum(lengths, dtype=np.int64)), dtype=torch.int32)
    return q, k, v, cu


def as_f64(t):
    """Exact fp64 numpy copy of a CPU tensor (bf16 and fp32 both embed exactly)."""
    return t.detach().to("cpu", torch.float64).numpy()


def quantize_fp8(x):
    """Per-tensor fp8 (OCP e4m3) quantisation of a float tensor for the fp8
    path: descale = max|x| / 448 (e4m3's largest finite value), stored =
    round-to-nearest-even of x / descale after clamping to ±448 (torch's cast
    does not saturate).  Returns (stored float8_e4m3fn tensor, descale float);
    the value a stored byte stands for is descale · stored."""
    amax = float(x.abs().max())
    descale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
    stored = (x.float() / descale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return stored, descale


def make_fp8(B, H, Hkv, N, d, seed=0, padded=False):
    """fp8 inputs following the recipe above: q, k, v drawn as for
    ``make_qkv`` (fp32 N(0, 1)), each quantised per tensor with
    ``quantize_fp8``; V is also returned transposed ([B, Hkv, d, N16], see
    ``transpose_fp8_v``) as the fp8 path takes it.  Returns (q8, k8, v8, vt8, (qd, kd, vd), key_lens)."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    key_lens = None
    if padded:
        key_lens = torch.randint(N // 2, N + 1, (B,), generator=g, dtype=torch.int32)
    q8, qd = quantize_fp8(q)
    k8, kd = quantize_fp8(k)
    v8, vd = quantize_fp8(v)
    return q8, k8, v8, transpose_fp8_v(v8), (qd, kd, vd), key_lens


def transpose_fp8_v(v8):
    """V [B, Hkv, N, d] (fp8) in the fp8 path's transposed layout
    [B, Hkv, d, N16], N16 = N rounded up to a multiple of 16, the extra columns
    zero."""
    B, Hkv, N, d = v8.shape
    n16 = (N + 15) // 16 * 16
    vt = torch.zeros((B, Hkv, d, n16), dtype=torch.uint8)
    vt[..., :N] = v8.view(torch.uint8).transpose(-1, -2)
    return vt.view(torch.float8_e4m3fn)
