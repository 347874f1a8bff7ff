"""GPU parity of the split-KV pieces (through the C ABI) against the fp64
oracle: the key-block partial (attn_fwd_partial_bf16), the S-way merge
(attn_merge) and the split-KV forward (attn_fwd_splitkv_bf16).

Tolerances: O of a bf16-input attention ≤ 1.5e-2 and LSE ≤ 1e-3 (as for the
dense path; the split-KV forward keeps its partial O in bf16, which adds one
rounding of up to 2^-8 relative before the merge, far inside that bound, and its
partial LSE in fp32);
the merge of given fp32 partials ≤ 1e-5 (fp32 output) or half a bf16 unit of
the output magnitude (bf16 output), LSE ≤ 1e-5.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_14_amd as attn
import oracle
from tests.fullsize import parallel_heads
from workloads import SPLITKV, as_f64, make_qkv, make_splitkv

pytestmark = pytest.mark.gpu

TOL_O = 1.5e-2
TOL_LSE = 1e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    attn.load_library()
    return torch.device("cuda:0")


def check(o, lse, O, L, what, tol_o=TOL_O, tol_l=TOL_LSE):
    o, lse = as_f64(o), as_f64(lse)
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    assert not np.isnan(lse).any(), f"{what}: NaN in LSE"
    assert np.array_equal(np.isneginf(lse), np.isneginf(L)), f"{what}: -inf pattern of LSE differs"
    eo = float(np.max(np.abs(o - O))) if o.size else 0.0
    fin = np.isfinite(L)
    el = float(np.max(np.abs(lse[fin] - L[fin]))) if fin.any() else 0.0
    print(f"  {what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= tol_o, f"{what}: max|dO| {eo:.3e} > {tol_o}"
    assert el <= tol_l, f"{what}: max|dLSE| {el:.3e} > {tol_l}"


def qkv(B, H, Hkv, Nq, Nk, d, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, H, Nq, d), generator=g).to(torch.bfloat16)
    k = torch.randn((B, Hkv, Nk, d), generator=g).to(torch.bfloat16)
    v = torch.randn((B, Hkv, Nk, d), generator=g).to(torch.bfloat16)
    return q, k, v


PART_CASES = [  # (B, H, Hkv, Nq, Nk, d, q_offset, k_offset)
    (1, 2, 1, 100, 300, 64, 250, 0),      # the queries' block follows most of the keys
    (2, 4, 2, 129, 77, 128, 0, 50),       # keys start after the first 50 queries: those rows are empty
    (1, 2, 2, 64, 0, 64, 0, 0),           # no keys at all
    (1, 3, 1, 300, 300, 128, 0, 0),       # the whole self-attention problem
    (2, 2, 1, 40, 1000, 64, 960, 0),      # a chunk of the last 40 queries over the whole cache
    (1, 4, 4, 257, 130, 128, 1000, 2000),  # keys entirely after the queries: every row empty under causal
]


@pytest.mark.parametrize("case", PART_CASES, ids=lambda c: "B%dH%dKV%dNq%dNk%dd%d_q%d_k%d" % c)
@pytest.mark.parametrize("causal", [False, True])
def test_partial_block(dev, case, causal):
    B, H, Hkv, Nq, Nk, d, qo, ko = case
    q, k, v = qkv(B, H, Hkv, Nq, Nk, d, seed=Nq + Nk)
    o, lse = attn.forward_partial(q.to(dev), k.to(dev), v.to(dev), q_offset=qo, k_offset=ko, scale=0.1,
                                  causal=causal)
    torch.cuda.synchronize()
    O, L = oracle.attention_partial(as_f64(q), as_f64(k), as_f64(v), 0.1, causal=causal, q_offset=qo, k_offset=ko)
    check(o.cpu(), lse.cpu(), O, L, f"partial {case} causal={causal}")


@pytest.mark.parametrize("S", [1, 3, 5])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_merge(dev, S, out):
    B, H, N, d = 2, 3, 70, 128
    g = torch.Generator("cpu").manual_seed(S)
    o_parts = torch.randn((S, B, H, N, d), generator=g)
    lse_parts = torch.randn((S, B, H, N), generator=g) * 20.0
    lse_parts[0, 0, 0, :] = -math.inf            # an empty part
    lse_parts[:, 1, 2, 5] = -math.inf            # a row empty in every part
    o_parts[:, 1, 2, 5, :] = 0.0
    o_parts[0, 0, 0, :, :] = 0.0
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    o, lse = attn.merge(o_parts.to(dev), lse_parts.to(dev), out_dtype=dt)
    torch.cuda.synchronize()
    O, L = oracle.merge_many(as_f64(o_parts), as_f64(lse_parts))
    tol = float(np.max(np.abs(O))) * 2.0 ** -8 if out == "bf16" else 1e-5
    check(o.cpu(), lse.cpu(), O, L, f"merge S={S} {out}", tol_o=tol, tol_l=1e-5)


SPLIT_CASES = [  # (B, H, Hkv, N, d)
    (1, 2, 1, 300, 64), (2, 4, 2, 777, 128), (1, 8, 2, 1030, 64),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "B%dH%dKV%dN%dd%d" % c)
@pytest.mark.parametrize("splits", [2, 3, 8])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_splitkv_self_attention(dev, case, splits, causal, padded):
    B, H, Hkv, N, d = case
    q, k, v, kl = make_qkv(B, H, Hkv, N, d, "bf16", seed=N + splits, padded=padded)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = attn.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), splits, scale=scale, causal=causal,
                                  key_lens=None if kl is None else kl.to(dev))
    torch.cuda.synchronize()
    O, L = oracle.attention(as_f64(q), as_f64(k), as_f64(v), scale, causal=causal,
                            key_lens=None if kl is None else kl.tolist())
    check(o.cpu(), lse.cpu(), O, L, f"splitkv {case} S={splits} causal={causal} padded={padded}")


@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_query_chunk_over_cache(dev, causal):
    """The last Nq positions of a sequence over its whole key cache (the
    chunked-prefill shape), split 7 ways."""
    B, H, Hkv, Nq, Nk, d = 2, 4, 2, 150, 2000, 128
    q, k, v = qkv(B, H, Hkv, Nq, Nk, d, seed=3)
    o, lse = attn.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), 7, q_offset=Nk - Nq, scale=0.09, causal=causal)
    torch.cuda.synchronize()
    O, L = oracle.attention_partial(as_f64(q), as_f64(k), as_f64(v), 0.09, causal=causal, q_offset=Nk - Nq)
    check(o.cpu(), lse.cpu(), O, L, f"chunk over cache causal={causal}")


def test_partials_then_merge_equal_dense(dev):
    """Key blocks [0, 333) and [333, 900) as separate partial calls, merged by
    attn_merge, against the dense entry point and the oracle."""
    B, H, Hkv, N, d = 1, 4, 2, 900, 64
    q, k, v, _ = make_qkv(B, H, Hkv, N, d, "bf16", seed=11)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    parts = [attn.forward_partial(qd, kd[:, :, a:b].contiguous(), vd[:, :, a:b].contiguous(), k_offset=a,
                                  scale=0.125, causal=True) for a, b in ((0, 333), (333, 900))]
    o, lse = attn.merge(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]))
    torch.cuda.synchronize()
    O, L = oracle.attention(as_f64(q), as_f64(k), as_f64(v), 0.125, causal=True)
    check(o.cpu(), lse.cpu(), O, L, "two partials merged")


def test_splitkv_workload_all_heads(dev):
    """The benchmarked split-KV shape at full size (512 queries at the end of a
    32768-key sequence, 16 key ranges): every row of every head against the
    oracle (the heads run side by side on the host's cores)."""
    w = SPLITKV
    q, k, v = make_splitkv(w)
    scale = float(np.float32(1 / math.sqrt(w["d"])))
    o, lse = attn.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), w["splits"], q_offset=w["Nk"] - w["Nq"],
                                  scale=scale, causal=w["causal"])
    torch.cuda.synchronize()
    q64, k64, v64 = as_f64(q), as_f64(k), as_f64(v)
    group = w["H"] // w["Hkv"]
    heads = [(b, h) for b in range(w["B"]) for h in range(w["H"])]

    def one(bh):
        b, h = bh
        g = h // group
        return oracle.attention_partial(q64[b:b + 1, h:h + 1], k64[b:b + 1, g:g + 1], v64[b:b + 1, g:g + 1], scale,
                                        causal=w["causal"], q_offset=w["Nk"] - w["Nq"])

    O = np.zeros(q.shape)
    L = np.zeros(q.shape[:3])
    for (b, h), (ob, lb) in zip(heads, parallel_heads(one, heads)):
        O[b, h], L[b, h] = ob[0, 0], lb[0, 0]
    check(o.cpu(), lse.cpu(), O, L, f"split-KV workload, all {len(heads)} heads x {w['Nq']} rows")
