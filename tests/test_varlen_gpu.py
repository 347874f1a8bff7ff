"""GPU parity of the packed variable-length forward (attn_fwd_varlen_bf16,
through the C ABI) against the fp64 packed-sequence oracle.

Same tolerances as the dense bf16 path: max |O_gpu − O_oracle| ≤ 1.5e-2,
max |LSE_gpu − LSE_oracle| ≤ 1e-3 over finite entries, −∞ entries equal, no NaN.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_14_amd as attn
import oracle
from tests.fullsize import parallel_heads
from workloads import VARLEN, as_f64, make_qkv, make_varlen, varlen_lengths

pytestmark = pytest.mark.gpu

TOL_O = 1.5e-2
TOL_LSE = 1e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    attn.load_library()
    return torch.device("cuda:0")


def check(o, lse, O, L, what):
    o, lse = as_f64(o), as_f64(lse)
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    assert not np.isnan(lse).any(), f"{what}: NaN in LSE"
    assert np.array_equal(np.isneginf(lse), np.isneginf(L)), f"{what}: -inf pattern of LSE differs"
    eo = float(np.max(np.abs(o - O))) if o.size else 0.0
    fin = np.isfinite(L)
    el = float(np.max(np.abs(lse[fin] - L[fin]))) if fin.any() else 0.0
    print(f"  {what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O, f"{what}: max|dO| {eo:.3e} > {TOL_O}"
    assert el <= TOL_LSE, f"{what}: max|dLSE| {el:.3e} > {TOL_LSE}"


def run(dev, q, k, v, cu, max_seqlen, scale, causal):
    o, lse = attn.forward_varlen(q.to(dev), k.to(dev), v.to(dev), cu.to(dev), max_seqlen, scale=scale,
                                 causal=causal)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


MIXES = [  # sequence lengths: ragged tails, empty sequences, one-token sequences, tile edges
    [1],
    [5, 0, 130, 1, 257],
    [128, 128, 127, 129],
    [300, 64, 0, 999],
    [0, 0, 700],
]


@pytest.mark.parametrize("lengths", MIXES, ids=lambda m: "L" + "-".join(map(str, m)))
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_mixes(dev, lengths, d, causal):
    H, Hkv = 4, 2
    what = f"varlen {lengths} d={d} causal={causal}"
    print(what, flush=True)
    q, k, v, cu = make_varlen(lengths, H, Hkv, d, seed=sum(lengths) + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = run(dev, q, k, v, cu, max(lengths), scale, causal)
    O, L = oracle.attention_varlen(as_f64(q), as_f64(k), as_f64(v), cu.tolist(), scale, causal=causal)
    check(o, lse, O, L, what)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_many_heads_and_sequences(dev, d, causal):
    """Enough (sequence, head, tile) items for the one-tile-per-workgroup
    schedule, with a long sequence next to many short ones."""
    lengths = [1000] + [37, 250, 129] * 5
    H, Hkv = 32, 8
    what = f"varlen many d={d} causal={causal}"
    print(what, flush=True)
    q, k, v, cu = make_varlen(lengths, H, Hkv, d, seed=77 + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = run(dev, q, k, v, cu, max(lengths), scale, causal)
    O, L = oracle.attention_varlen(as_f64(q), as_f64(k), as_f64(v), cu.tolist(), scale, causal=causal)
    check(o, lse, O, L, what)


@pytest.mark.parametrize("shape", [(3, 4, 2, 333), (4, 32, 8, 1100)], ids=["small", "large"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_dense_entry_bitwise(dev, shape, d, causal):
    """B sequences of one length packed end to end give bit for bit the dense
    entry point's results on the [B, H, N, d] layout (same kernels, other
    strides; the large shape has enough tiles for the one-tile-per-workgroup
    launch, at d = 128 the eight-wave form)."""
    B, H, Hkv, N = shape
    q, k, v, _ = make_qkv(B, H, Hkv, N, d, "bf16", seed=5)
    scale = float(np.float32(1 / math.sqrt(d)))
    od, lsed = attn.forward(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=causal)
    pack = lambda x: x.transpose(1, 2).reshape(B * N, x.shape[1], d).contiguous()  # noqa: E731
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32)
    o, lse = run(dev, pack(q), pack(k), pack(v), cu, N, scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(o, pack(od.cpu())), "packed O differs from the dense entry point"
    assert torch.equal(lse, lsed.cpu().transpose(0, 1).reshape(H, B * N)), "packed LSE differs"


def test_uncovered_tokens_untouched_and_poison_contained(dev):
    """Tokens past cu_seqlens[B] belong to no sequence: their NaN q/k/v must
    not reach any output and their o / lse entries must not be written."""
    lengths = [200, 77]
    H, Hkv, d = 4, 1, 128
    q, k, v, cu = make_varlen(lengths + [50], H, Hkv, d, seed=9)
    cu = cu[:-1].contiguous()           # the last 50 tokens are outside every sequence
    total = q.shape[0]
    for t in (q, k, v):
        t[277:] = float("nan")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.full_like(qd, 7.0)
    lse = torch.full((H, total), 3.0, dtype=torch.float32, device=dev)
    attn.forward_varlen(qd, kd, vd, cu.to(dev), max(lengths), scale=0.1, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    assert torch.all(o[277:] == 7.0) and torch.all(lse[:, 277:] == 3.0), "uncovered tokens were written"
    O, L = oracle.attention_varlen(as_f64(q[:277]), as_f64(k[:277]), as_f64(v[:277]), cu.tolist(), 0.1, causal=True)
    check(o[:277], lse[:, :277], O, L, "covered tokens")


def test_lengths_clamped_to_max_seqlen(dev):
    """A sequence longer than max_seqlen is cut to its first max_seqlen tokens
    (queries and keys); the rest of it is not written."""
    lengths = [150, 400]
    H, Hkv, d = 2, 2, 64
    q, k, v, cu = make_varlen(lengths, H, Hkv, d, seed=4)
    qd = q.to(dev)
    o = torch.full_like(qd, 5.0)
    lse = torch.full((H, 550), 2.0, dtype=torch.float32, device=dev)
    attn.forward_varlen(qd, k.to(dev), v.to(dev), cu.to(dev), 256, scale=0.125, causal=False, out=o, lse=lse)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    keep = torch.cat([torch.arange(0, 150), torch.arange(150, 406)])
    O, L = oracle.attention_varlen(as_f64(q[keep]), as_f64(k[keep]), as_f64(v[keep]), [0, 150, 406], 0.125)
    check(o[keep], lse[:, keep], O, L, "clamped")
    assert torch.all(o[406:] == 5.0) and torch.all(lse[:, 406:] == 2.0), "tokens past max_seqlen were written"


def test_empty_pack_is_a_noop(dev):
    q = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device=dev)
    cu = torch.zeros(4, dtype=torch.int32, device=dev)
    o, lse = attn.forward_varlen(q, q, q, cu, 0)
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 64) and lse.shape == (2, 0)


def test_varlen_workload_all_heads(dev):
    """The benchmarked packed batch at full size: every token of every
    sequence and head against the packed-sequence oracle (each (sequence,
    head) pair as a one-sequence pack; the pairs run side by side on the
    host's cores)."""
    w = VARLEN
    lengths = varlen_lengths(w["B"], w["N"] // 2, w["N"], w["seed"])
    q, k, v, cu = make_varlen(lengths, w["H"], w["Hkv"], w["d"], seed=w["seed"])
    scale = float(np.float32(1 / math.sqrt(w["d"])))
    o, lse = run(dev, q, k, v, cu, w["N"], scale, w["causal"])
    q64, k64, v64 = as_f64(q), as_f64(k), as_f64(v)
    group = w["H"] // w["Hkv"]
    items = [(b, h) for b in range(len(lengths)) for h in range(w["H"])]

    def one(bh):
        b, h = bh
        s0, s1 = int(cu[b]), int(cu[b + 1])
        g = h // group
        return oracle.attention_varlen(q64[s0:s1, h:h + 1], k64[s0:s1, g:g + 1], v64[s0:s1, g:g + 1], [0, s1 - s0],
                                       scale, causal=w["causal"])

    O = np.zeros(q.shape)
    L = np.zeros((w["H"], q.shape[0]))
    for (b, h), (ob, lb) in zip(items, parallel_heads(one, items)):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        O[s0:s1, h] = ob[:, 0]
        L[h, s0:s1] = lb[0]
    check(o, lse, O, L, f"packed batch, all {len(lengths)} sequences x {w['H']} heads, every token")
