"""GPU parity of the fp8 forward (attn_fwd_fp8, through the C ABI) against the
fp64 oracle evaluated on the values the fp8 inputs stand for (descale ·
stored byte, exact in fp64).

Tolerance (the pages give none for fp8): the kernel's only rounding beyond
fp32 is that of the softmax weights to fp8 e4m3 before P·V.  A weight p_j
(normalised) is off by at most 2^-4·p_j (3 mantissa bits, nearest) or, in
e4m3's subnormal range, by at most 2^-17 (half a subnormal step, 2^-10, over
a row sum that is at least 2^7).  Taking those errors as independent and
uniform, an output element O_id has standard deviation
σ_id = sqrt(Σ_j (4^-4·p_j² + 4^-17)·v_jd² / 3); the test allows 7σ plus the
bf16 rounding of the output (2^-8·|O|) plus 1e-5.  LSE comes from the fp32
weights: ≤ 1e-3 as for bf16.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_14_amd as attn
import oracle
from workloads import WORKLOADS, as_f64, make_fp8

pytestmark = pytest.mark.gpu

TOL_LSE = 1e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    attn.load_library()
    return torch.device("cuda:0")


def oracle_scale(scale, qd, kd):
    """The score scale the oracle applies to the dequantised q and k: the
    kernel multiplies the raw fp8 products by scale·q_descale·k_descale
    evaluated in fp32, left to right."""
    s_eff = np.float32(np.float32(np.float32(scale) * np.float32(qd)) * np.float32(kd))
    return float(s_eff) / (float(qd) * float(kd))


def deq(x8, descale):
    return as_f64(x8.float()) * float(descale)


def reference(q, k, v, scale, causal, key_lens, rows=None):
    """Oracle O, LSE and the per-element tolerance of the rounding model."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    O, L = oracle.attention(q, k, v, scale, causal=causal, key_lens=key_lens, rows=rows)
    tol = np.zeros_like(O)
    for b in range(B):
        kl = N if key_lens is None else int(min(max(int(key_lens[b]), 0), N))
        for h in range(H):
            g = oracle.kv_head_of(h, H, Hkv)
            s = oracle.scores(q[b, h, rows], k[b, g, :kl], scale)
            s = np.where(oracle.admissible(rows, kl, causal), s, -np.inf)
            p, _, _ = oracle.softmax_rows(s)
            v2 = v[b, g, :kl] ** 2
            var = ((4.0 ** -4) * (p ** 2) + 4.0 ** -17 * (p > 0)) @ v2 / 3.0
            tol[b, h] = 7.0 * np.sqrt(var) + 2.0 ** -8 * np.abs(O[b, h]) + 1e-5
    return O, L, tol


def check(o, lse, O, L, tol, what):
    o, lse = as_f64(o), as_f64(lse)
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    assert not np.isnan(lse).any(), f"{what}: NaN in LSE"
    assert np.array_equal(np.isneginf(lse), np.isneginf(L)), f"{what}: -inf pattern of LSE differs"
    err = np.abs(o - O)
    fin = np.isfinite(L)
    el = float(np.max(np.abs(lse[fin] - L[fin]))) if fin.any() else 0.0
    worst = float(np.max(err / tol)) if err.size else 0.0
    print(f"  {what}: max|dO|={float(err.max()) if err.size else 0:.3e} max(|dO|/tol)={worst:.3f} "
          f"max|dLSE|={el:.3e}", flush=True)
    assert worst <= 1.0, f"{what}: error exceeds the fp8 rounding model by {worst:.2f}x"
    assert el <= TOL_LSE, f"{what}: max|dLSE| {el:.3e} > {TOL_LSE}"


def run(dev, q8, k8, vt8, ds, scale, causal, kl):
    o, lse = attn.forward_fp8(q8.to(dev), k8.to(dev), vt8.to(dev), ds[0], ds[1], ds[2], scale=scale, causal=causal,
                              key_lens=None if kl is None else kl.to(dev))
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


SHAPES = [  # (B, H, Hkv, N, d): several tiles, ragged tails (N a multiple of 16), GQA
    (1, 1, 1, 16, 64), (1, 2, 1, 64, 64), (2, 4, 2, 208, 128), (1, 2, 2, 512, 64), (2, 8, 2, 384, 128),
    (1, 3, 1, 1008, 128),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dKV%dN%dd%d" % s)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_fp8_shapes(dev, shape, causal, padded):
    B, H, Hkv, N, d = shape
    q8, k8, v8, vt8, ds, kl = make_fp8(B, H, Hkv, N, d, seed=N + d, padded=padded)
    scale = float(np.float32(1 / math.sqrt(d)))
    if kl is not None:
        # poison the padded keys: NaN bytes (0x7F) in K rows and Vᵀ columns past the key length
        k8 = k8.clone()
        vt8 = vt8.clone()
        for b in range(B):
            k8.view(torch.uint8)[b, :, int(kl[b]):] = 0x7F
            vt8.view(torch.uint8)[b, :, :, int(kl[b]):] = 0x7F
    o, lse = run(dev, q8, k8, vt8, ds, scale, causal, kl)
    O, L, tol = reference(deq(q8, ds[0]), np.nan_to_num(deq(k8, ds[1])), deq(v8, ds[2]),
                          oracle_scale(scale, ds[0], ds[1]), causal, None if kl is None else kl.tolist())
    check(o, lse, O, L, tol, f"fp8 {shape} causal={causal} padded={padded}")


@pytest.mark.parametrize("scale", [0.0, -0.3])
def test_fp8_scale_edge_cases(dev, scale):
    B, H, Hkv, N, d = 1, 2, 1, 96, 128
    q8, k8, v8, vt8, ds, _ = make_fp8(B, H, Hkv, N, d, seed=9)
    o, lse = run(dev, q8, k8, vt8, ds, scale, False, None)
    O, L, tol = reference(deq(q8, ds[0]), deq(k8, ds[1]), deq(v8, ds[2]), oracle_scale(scale, ds[0], ds[1]), False,
                          None)
    check(o, lse, O, L, tol, f"fp8 scale={scale}")


def test_fp8_key_length_zero(dev):
    B, H, Hkv, N, d = 2, 2, 2, 64, 64
    q8, k8, v8, vt8, ds, _ = make_fp8(B, H, Hkv, N, d, seed=2)
    kl = torch.tensor([0, 33], dtype=torch.int32)
    o, lse = run(dev, q8, k8, vt8, ds, 0.125, False, kl)
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0])), "a sequence without keys must give O=0, -inf"
    O, L, tol = reference(deq(q8, ds[0])[1:], deq(k8, ds[1])[1:], deq(v8, ds[2])[1:],
                          oracle_scale(0.125, ds[0], ds[1]), False, [33])
    check(o[1:], lse[1:], O, L, tol, "fp8 key length 33")


@pytest.mark.parametrize("wid", [4, 5])
def test_fp8_workload_sampled_rows(dev, wid):
    """The fp8 forms of the long workloads at full size (the benchmarked
    shapes): sampled query rows of a few heads against the oracle."""
    w = WORKLOADS[wid]
    q8, k8, v8, vt8, ds, kl = make_fp8(w.B, w.H, w.Hkv, w.N, w.d, seed=100 + w.seed, padded=w.padded)
    o, lse = run(dev, q8, k8, vt8, ds, w.scale, w.causal, kl)
    rows = np.array([0, 1, 127, 128, 4095, w.N // 2 + 17, w.N - 1])
    for b in range(w.B):
        for h in (0, w.H - 1):
            g = h // (w.H // w.Hkv)
            O, L, tol = reference(deq(q8[b:b + 1, h:h + 1], ds[0]), deq(k8[b:b + 1, g:g + 1], ds[1]),
                                  deq(v8[b:b + 1, g:g + 1], ds[2]), oracle_scale(w.scale, ds[0], ds[1]), w.causal,
                                  None if kl is None else [int(kl[b])], rows=rows)
            check(o[b:b + 1, h:h + 1, rows], lse[b:b + 1, h:h + 1, rows], O, L, tol, f"fp8 W{wid} b={b} h={h}")
