"""GPU parity of the backward pass (attn_bwd_bf16 through the C ABI) against
the fp64 backward oracle, on bf16 inputs.

Tolerance: max |grad_gpu − grad_oracle| ≤ 2e-2 · max |grad_oracle| per tensor
(dQ, dK, dV).  The gradients are stored in bf16 (relative rounding up to
2^-8: 8 significant bits, nearest), and
inside the kernels P and dS are rounded to bf16 as matrix-core operands and D
is formed from the bf16 forward output; each of these is a relative
perturbation of order 2^-8 of terms that are summed over up to N keys or
queries with mixed signs, so the bound leaves a margin of about 5× over
2^-8 on the largest gradient entry.  No NaN may appear.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_14_amd as attn
import oracle
from tests.fullsize import parallel_heads
from workloads import as_f64

pytestmark = pytest.mark.gpu

TOL_REL = 2e-2


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    attn.load_library()
    return torch.device("cuda:0")


def _inputs(B, H, Hkv, N, d, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16)
    do = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16)
    return q, k, v, do


def run_case(dev, B, H, Hkv, N, d, causal, key_lens, seed, scale=None, poison=False, inputs=None):
    what = f"bwd B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} key_lens={key_lens} scale={scale}"
    print(what, flush=True)
    q, k, v, do = _inputs(B, H, Hkv, N, d, seed) if inputs is None else inputs
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    scale = float(np.float32(scale))
    kl = None if key_lens is None else torch.tensor(key_lens, dtype=torch.int32)
    kg, vg = k.clone(), v.clone()
    if poison and key_lens is not None:
        for b, n in enumerate(key_lens):
            kg[b, :, max(n, 0):] = float("nan")
            vg[b, :, max(n, 0):] = float("nan")
    qd, kd, vd, dod = (t.to(dev).contiguous() for t in (q, kg, vg, do))
    kld = None if kl is None else kl.to(dev)
    o, lse = attn.forward(qd, kd, vd, scale=scale, causal=causal, key_lens=kld)
    dq, dk, dv = attn.backward(qd, kd, vd, o, lse, dod, scale=scale, causal=causal, key_lens=kld)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(as_f64(q), as_f64(k), as_f64(v), as_f64(do), scale, causal=causal,
                                    key_lens=key_lens)
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        g64 = as_f64(got.cpu())
        assert not np.isnan(g64).any(), f"{what}: NaN in {name}"
        err = float(np.max(np.abs(g64 - want))) if want.size else 0.0
        mag = float(np.max(np.abs(want))) if want.size else 0.0
        print(f"  {name}: max err {err:.3e}  max |ref| {mag:.3e}", flush=True)
        assert err <= TOL_REL * mag + 1e-6, f"{what}: {name} max err {err:.3e} > {TOL_REL} x {mag:.3e}"
    return dq, dk, dv


SMALL = [  # (B, H, Hkv, N, d): ragged tails, several tiles, grouped heads
    (1, 1, 1, 1, 64), (2, 2, 1, 17, 64), (1, 4, 2, 100, 128), (2, 2, 2, 129, 64),
    (1, 2, 1, 255, 128), (1, 3, 3, 300, 64), (2, 4, 2, 200, 128),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}H{}Hkv{}N{}d{}".format(*s))
@pytest.mark.parametrize("causal", [False, True])
def test_backward_small(dev, shape, causal):
    B, H, Hkv, N, d = shape
    run_case(dev, B, H, Hkv, N, d, causal, None, seed=7 + N)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_padded_with_poison(dev, causal, d):
    # padded K/V hold NaN: they must not reach any gradient; padded keys get 0
    N = 190
    key_lens = [150, 0, 190, 1]
    dq, dk, dv = run_case(dev, 4, 2, 1, N, d, causal, key_lens, seed=11, poison=True)
    dk, dv = as_f64(dk.cpu()), as_f64(dv.cpu())
    for b, n in enumerate(key_lens):
        assert np.all(dk[b, :, n:] == 0) and np.all(dv[b, :, n:] == 0), "padded keys"
    assert np.all(as_f64(dq.cpu())[1] == 0), "sequence without keys"


@pytest.mark.parametrize("causal", [False, True])
def test_backward_padded_very_negative_scores(dev, causal):
    """Every admissible score below -100 (so LSE is too): a padded key's zero
    score would give exp(0 - LSE) > exp(100), beyond fp32.  Its K row is zero,
    so it may only contribute 0 to dQ, and to nothing else.  (q and k share an
    opposite offset of the size of their spread, so that dQ, whose component
    along the offset cancels, stays well conditioned in bf16.)"""
    B, H, Hkv, N, d = 2, 2, 1, 200, 64
    g = torch.Generator().manual_seed(21)
    q = (0.5 + 0.5 * torch.randn(B, H, N, d, generator=g)).to(torch.bfloat16)
    k = -(0.5 + 0.5 * torch.randn(B, Hkv, N, d, generator=g).abs()).to(torch.bfloat16)
    v = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16)
    do = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16)
    s = (q.double()[:, :, :, None, :] * k.double()[:, :1, None, :, :]).sum(-1) * 8.0
    assert s.max().item() < -100.0
    dq, dk, dv = run_case(dev, B, H, Hkv, N, d, causal, [150, 77], seed=0, scale=8.0, inputs=(q, k, v, do))
    for b, n in enumerate([150, 77]):
        assert np.all(as_f64(dk.cpu())[b, :, n:] == 0) and np.all(as_f64(dv.cpu())[b, :, n:] == 0), "padded keys"


@pytest.mark.parametrize("scale", [0.0, -0.2])
def test_backward_scale_edge_cases(dev, scale):
    run_case(dev, 1, 2, 1, 70, 64, True, None, seed=13, scale=scale)


def test_backward_medium(dev):
    # several query and key tiles in both kernels, grouped heads, causal
    run_case(dev, 1, 4, 2, 700, 128, True, None, seed=17)


def _workload_backward(dev, wid):
    """Forward + backward of a named workload at full size, in the launch
    configuration bench.py times (same inputs and seeded dout)."""
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[wid]
    q, k, v, kl = make_inputs(w)
    g = torch.Generator().manual_seed(1000 + w.seed)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    kld = None if kl is None else kl.to(dev)
    o, lse = attn.forward(qd, kd, vd, scale=w.scale, causal=w.causal, key_lens=kld)
    dq, dk, dv = attn.backward(qd, kd, vd, o, lse, dod, scale=w.scale, causal=w.causal, key_lens=kld)
    torch.cuda.synchronize()
    return w, (q, k, v, do, kl), (dq.cpu(), dk.cpu(), dv.cpu())


def _compare(what, got, want):
    g64 = as_f64(got)
    assert not np.isnan(g64).any(), f"{what}: NaN"
    err = float(np.max(np.abs(g64 - want)))
    mag = float(np.max(np.abs(want)))
    print(f"  {what}: max err {err:.3e}  max |ref| {mag:.3e}", flush=True)
    assert err <= TOL_REL * mag + 1e-6, f"{what}: max err {err:.3e} > {TOL_REL} x {mag:.3e}"


def test_backward_workload2_full(dev):
    """Workload 2 (B4 H8 N1024 d64) at full size: every gradient element."""
    w, (q, k, v, do, kl), grads = _workload_backward(dev, 2)
    ref = oracle.attention_backward(as_f64(q), as_f64(k), as_f64(v), as_f64(do), w.scale, causal=w.causal)
    for name, got, want in zip(("dQ", "dK", "dV"), grads, ref):
        _compare(f"workload 2 {name}", got, want)


def test_backward_workload3_all_heads(dev):
    """Workload 3 (causal B2 H8 N4096 d64) at full size: dQ, dK and dV of all
    16 heads, every element, against the oracle (each head is its own kv head
    there; the heads run side by side on the host's cores)."""
    w, (q, k, v, do, kl), (dq, dk, dv) = _workload_backward(dev, 3)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(bh):
        b, h = bh
        return oracle.attention_backward(as_f64(q[b:b + 1, h:h + 1]), as_f64(k[b:b + 1, h:h + 1]),
                                         as_f64(v[b:b + 1, h:h + 1]), as_f64(do[b:b + 1, h:h + 1]), w.scale,
                                         causal=True)

    refs = parallel_heads(one, heads)
    for name, i, got in (("dQ", 0, dq), ("dK", 1, dk), ("dV", 2, dv)):
        want = np.zeros(got.shape)
        for (b, h), r in zip(heads, refs):
            want[b, h] = r[i][0, 0]
        _compare(f"workload 3 all 16 heads {name}", got, want)


def _groups_against_oracle(wid, w, inputs, grads, groups):
    """Whole kv groups (b, g) of a workload: dQ of the group's query heads and
    dK, dV of the kv head, every element, against the oracle."""
    q, k, v, do, kl = inputs
    dq, dk, dv = grads
    group = w.H // w.Hkv
    for b, g in groups:
        hs = slice(g * group, (g + 1) * group)
        ref = oracle.attention_backward(as_f64(q[b:b + 1, hs]), as_f64(k[b:b + 1, g:g + 1]),
                                        as_f64(v[b:b + 1, g:g + 1]), as_f64(do[b:b + 1, hs]), w.scale,
                                        causal=w.causal, key_lens=None if kl is None else [int(kl[b])])
        for name, got, want in zip(("dQ", "dK", "dV"), (dq[b:b + 1, hs], dk[b:b + 1, g:g + 1],
                                                        dv[b:b + 1, g:g + 1]), ref):
            _compare(f"workload {wid} b={b} kv head {g} ({group} query heads) {name}", got, want)


def _column_sums(wid, w, inputs, grads):
    """A property of the definition at any size, over every kv group: each
    admissible row's weights sum to one, so for every kv head the dV rows
    summed over the keys equal the dO rows summed over that head's query
    heads; padded keys get exactly zero gradients.  Tolerance: the weights
    are bf16 operands (relative rounding up to 2^-8 each) and dV is stored in
    bf16."""
    q, k, v, do, kl = inputs
    dq, dk, dv = grads
    group = w.H // w.Hkv
    do64, dv64 = as_f64(do), as_f64(dv)
    assert not np.isnan(as_f64(dq)).any() and not np.isnan(as_f64(dk)).any() and not np.isnan(dv64).any()
    for b in range(w.B):
        n = w.N if kl is None else int(kl[b])
        if kl is not None:
            assert np.all(as_f64(dk)[b, :, n:] == 0) and np.all(dv64[b, :, n:] == 0), "padded keys"
        for g in range(w.Hkv):
            got = dv64[b, g, :n].sum(axis=0)
            want = do64[b, g * group:(g + 1) * group].sum(axis=(0, 1))
            tol = 2.0 ** -8 * np.abs(do64[b, g * group:(g + 1) * group]).sum(axis=(0, 1)) \
                + 2.0 ** -8 * np.abs(dv64[b, g, :n]).sum(axis=0)
            worst = float(np.max(np.abs(got - want) / tol))
            assert worst <= 1.0, f"workload {wid} b={b} g={g}: column sums of dV off by {worst:.2f}x the bound"
    print(f"  workload {wid}: dV column sums of every kv group within bounds", flush=True)


def test_backward_workload4_heads(dev):
    """Workload 4 (causal B1 H16 N16384 d128) at full size, in the launch
    configuration bench.py times: the first and the last head compared
    element by element with the oracle (each N x N oracle head holds about
    9 GiB of fp64 matrices), and the column-sum property over every head."""
    w, inputs, grads = _workload_backward(dev, 4)
    _groups_against_oracle(4, w, inputs, grads, [(0, 0), (0, w.Hkv - 1)])
    _column_sums(4, w, inputs, grads)


def test_backward_workload5_groups(dev):
    """Workload 5 (GQA padded B2 Hq32 Hkv8 N8192 d128) at full size: two whole
    kv groups (4 query heads each; the two sequences have different key
    lengths) element by element against the oracle, and the column-sum
    property over every group."""
    w, inputs, grads = _workload_backward(dev, 5)
    _groups_against_oracle(5, w, inputs, grads, [(0, 0), (w.B - 1, w.Hkv - 1)])
    _column_sums(5, w, inputs, grads)
