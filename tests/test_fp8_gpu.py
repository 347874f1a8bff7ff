"""GPU parity of the fp8 path (through the C ABI) against the fp64 oracle.

The forward pass (attn_fwd_fp8) is compared with the oracle evaluated on the
values the fp8 inputs stand for (descale · stored byte, exact in fp64).  The
pages give no tolerance for fp8; the kernel's only rounding beyond fp32 is that
of the softmax weights to fp8 e4m3 before P·V.  A normalised weight p_j is off
by at most b_j = 2^-4·p_j (3 mantissa bits, nearest) or, in e4m3's subnormal
range, 2^-17 (half a subnormal step, 2^-10, over a row sum of at least 2^7:
the weights are scaled so that the row's largest is between 2^7 and 2^8).
Per output element O_id the checks are

* a hard bound, which holds whatever the rounding errors are:
  |ΔO_id| ≤ Σ_j (2^-4·p_j + 2^-17)·|v_jd| + 2^-8·|O_id| + 1e-5
  (the last two terms: the bf16 output rounding and fp32 arithmetic);
* a tighter bound from Hoeffding's inequality, reading the rounding errors of
  different weights as independent and zero-mean (nearest rounding of values
  spread over many binade positions): with e_j the error of weight j,
  P(|Σ_j e_j v_jd| > t) ≤ 2·exp(−t² / (2 Σ_j b_j² v_jd²)), so
  t = 8.5·sqrt(Σ_j b_j² v_jd²) is exceeded with probability below 1e-15 per
  element; the test allows t + 2^-8·|O_id| + 1e-5.

Both products run on the fp8 matrix-core instruction, which sums each block of
64 products with an error of up to about 2^-12 of the block's largest product
(measured on gfx950 with an in-bounds probe against exact products: 2^-12.0
to 2^-13.8 over six operand patterns; the bf16 instruction shows nothing
similar).  With a 2x margin, a score s_ij = scale·q_i·k_j is off by at most
δ_i = (d/64)·2^-11·|scale|·max_c|q_ic|·max_{j admissible} max_c|k_jc|, so
LSE_i is off by at most δ_i, and the weights by a factor within e^(±2δ_i),
which adds (e^(2δ_i) − 1)·Σ_j p_j|v_jd − O_id| ≤ (e^(2δ_i) − 1)·(Σ_j p_j|v_jd| +
|O_id|) to both bounds above; the P·V
sums add 2^-11·Σ_j p_j·|v_jd|.  LSE: ≤ 1e-3 + δ_i (the 1e-3 of the bf16
path covers the fp32 sums).  On N(0,1) inputs δ is ~1e-3 as a bound while the
measured LSE errors stay near 3e-5; with outlier features it dominates,
which is what the incoherent processing (rotation) reduces.

The preparation kernels (attn_fp8_amax, attn_fp8_quantize,
attn_fp8_quantize_vt) are compared with oracle/fp8.py: the amax to fp32
rounding, the descale bit for bit from that amax, and every stored byte
against the e4m3 rounding of the fp64 value, allowing the neighbouring code
only where the value lies within fp32 rounding of a rounding boundary.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_14_amd as attn
import oracle
from oracle import fp8 as ofp8
from tests.fullsize import parallel_heads
from workloads import WORKLOADS, as_f64, make_fp8, make_qkv, transpose_fp8_v

pytestmark = pytest.mark.gpu

TOL_LSE = 1e-3
HOEFFDING = 8.5


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


def reference_head(q, k, v, scale, causal, kl, rows=None, chunk=1024):
    """One head (q [N, d], k and v [N, d] fp64): oracle O [R, d] and LSE [R],
    the hard and Hoeffding bounds of every O element and the LSE bound of
    every row (rows in chunks)."""
    N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    O, L = oracle.attention(q[None, None], k[None, None], v[None, None], scale, causal=causal,
                            key_lens=None if kl is None else [kl], rows=rows)
    O, L = O[0, 0], L[0, 0]
    n = N if kl is None else int(min(max(kl, 0), N))
    hard = np.zeros_like(O)
    hoef = np.zeros_like(O)
    tol_l = np.full(L.shape, TOL_LSE)
    av, v2 = np.abs(v[:n]), v[:n] ** 2
    qmax = np.abs(q).max(axis=1)                      # per query row
    kmax = np.abs(k[:n]).max(axis=1) if n else np.zeros(0)
    for c0 in range(0, len(rows), chunk):
        r = rows[c0:c0 + chunk]
        ok = oracle.admissible(r, n, causal)
        s = np.where(ok, oracle.scores(q[r], k[:n], scale), -np.inf)
        p, _, _ = oracle.softmax_rows(s)
        live = (p > 0) | ok
        b = 2.0 ** -4 * p + 2.0 ** -17 * live
        o = O[c0:c0 + len(r)]
        # score error bound of the fp8 matrix-core sums, per row
        kmx = np.where(ok, kmax[None, :], 0.0).max(axis=1) if n else np.zeros(len(r))
        delta = (d / 64) * 2.0 ** -11 * abs(scale) * qmax[r] * kmx
        pav = p @ av
        # Σ_j p_j |v_jd − O_id| ≤ Σ_j p_j |v_jd| + |O_id|
        extra = np.expm1(2 * delta)[:, None] * (pav + np.abs(o)) + 2.0 ** -11 * pav
        hard[c0:c0 + len(r)] = b @ av + extra
        hoef[c0:c0 + len(r)] = HOEFFDING * np.sqrt((b ** 2) @ v2) + extra
        tol_l[c0:c0 + len(r)] = TOL_LSE + delta
    out = 2.0 ** -8 * np.abs(O) + 1e-5
    return O, L, hard + out, hoef + out, tol_l


def reference(q, k, v, scale, causal, key_lens, rows=None):
    """Every (b, h) head of q [B, H, N, d] (k, v [B, Hkv, N, d]), side by side
    on the host's cores: (O, LSE, hard bound, Hoeffding bound, LSE bound)."""
    B, H, N, d = q.shape
    group = H // k.shape[1]
    heads = [(b, h) for b in range(B) for h in range(H)]

    def one(bh):
        b, h = bh
        return reference_head(q[b, h], k[b, h // group], v[b, h // group], scale, causal,
                              None if key_lens is None else int(key_lens[b]), rows)

    res = parallel_heads(one, heads)
    R = N if rows is None else len(rows)
    O, L, hard, hoef = np.zeros((B, H, R, d)), np.zeros((B, H, R)), np.zeros((B, H, R, d)), np.zeros((B, H, R, d))
    tol_l = np.zeros((B, H, R))
    for (b, h), (o, l_, t1, t2, t3) in zip(heads, res):
        O[b, h], L[b, h], hard[b, h], hoef[b, h], tol_l[b, h] = o, l_, t1, t2, t3
    return O, L, hard, hoef, tol_l


def check(o, lse, O, L, hard, hoef, tol_l, what):
    o, lse = as_f64(o), as_f64(lse)
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    assert not np.isnan(lse).any(), f"{what}: NaN in LSE"
    assert np.array_equal(np.isneginf(lse), np.isneginf(L)), f"{what}: -inf pattern of LSE differs"
    err = np.abs(o - O)
    fin = np.isfinite(L)
    el = np.abs(lse[fin] - L[fin])
    w_l = float(np.max(el / tol_l[fin])) if fin.any() else 0.0
    w_hard = float(np.max(err / hard)) if err.size else 0.0
    w_hoef = float(np.max(err / hoef)) if err.size else 0.0
    print(f"  {what}: max|dO|={float(err.max()) if err.size else 0:.3e} max(|dO|/hard bound)={w_hard:.3f} "
          f"max(|dO|/Hoeffding bound)={w_hoef:.3f} max|dLSE|={float(el.max()) if el.size else 0:.3e} "
          f"max(|dLSE|/bound)={w_l:.3f}", flush=True)
    assert w_hard <= 1.0, f"{what}: error exceeds the hard fp8 bound by {w_hard:.2f}x"
    assert w_hoef <= 1.0, f"{what}: error exceeds the Hoeffding bound by {w_hoef:.2f}x"
    assert w_l <= 1.0, f"{what}: LSE error exceeds its bound by {w_l:.2f}x"


def run(dev, q8, k8, vt8, ds, scale, causal, kl):
    o, lse = attn.forward_fp8(q8.to(dev), k8.to(dev), vt8.to(dev), ds[0], ds[1], ds[2], scale=scale, causal=causal,
                              key_lens=None if kl is None else kl.to(dev))
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


SHAPES = [  # (B, H, Hkv, N, d): several tiles, ragged tails (any N), GQA
    (1, 1, 1, 16, 64), (1, 2, 1, 64, 64), (2, 4, 2, 208, 128), (1, 2, 2, 512, 64), (2, 8, 2, 384, 128),
    (1, 3, 1, 1008, 128), (1, 1, 1, 1, 64), (2, 2, 1, 17, 128), (1, 2, 2, 100, 64), (2, 4, 2, 250, 128),
    (1, 2, 1, 1001, 64),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dKV%dN%dd%d" % s)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_fp8_shapes(dev, shape, causal, padded):
    B, H, Hkv, N, d = shape
    q8, k8, v8, vt8, ds, kl = make_fp8(B, H, Hkv, N, d, seed=N + d, padded=padded)
    scale = float(np.float32(1 / math.sqrt(d)))
    # poison: NaN bytes (0x7F) in the unused Vᵀ columns past N, and, when
    # padded, in K rows and Vᵀ columns past the key length
    k8, vt8 = k8.clone(), vt8.clone()
    vt8.view(torch.uint8)[..., N:] = 0x7F
    if kl is not None:
        for b in range(B):
            k8.view(torch.uint8)[b, :, int(kl[b]):] = 0x7F
            vt8.view(torch.uint8)[b, :, :, int(kl[b]):] = 0x7F
    o, lse = run(dev, q8, k8, vt8, ds, scale, causal, kl)
    O, L, hard, hoef, tol_l = reference(deq(q8, ds[0]), np.nan_to_num(deq(k8, ds[1])), deq(v8, ds[2]),
                                 oracle_scale(scale, ds[0], ds[1]), causal, None if kl is None else kl.tolist())
    check(o, lse, O, L, hard, hoef, tol_l, f"fp8 {shape} causal={causal} padded={padded}")


@pytest.mark.parametrize("scale", [0.0, -0.3])
def test_fp8_scale_edge_cases(dev, scale):
    B, H, Hkv, N, d = 1, 2, 1, 96, 128
    q8, k8, v8, vt8, ds, _ = make_fp8(B, H, Hkv, N, d, seed=9)
    o, lse = run(dev, q8, k8, vt8, ds, scale, False, None)
    O, L, hard, hoef, tol_l = reference(deq(q8, ds[0]), deq(k8, ds[1]), deq(v8, ds[2]), oracle_scale(scale, ds[0], ds[1]),
                                 False, None)
    check(o, lse, O, L, hard, hoef, tol_l, f"fp8 scale={scale}")


def test_fp8_key_length_zero(dev):
    B, H, Hkv, N, d = 2, 2, 2, 64, 64
    q8, k8, v8, vt8, ds, _ = make_fp8(B, H, Hkv, N, d, seed=2)
    kl = torch.tensor([0, 33], dtype=torch.int32)
    o, lse = run(dev, q8, k8, vt8, ds, 0.125, False, kl)
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0])), "a sequence without keys must give O=0, -inf"
    O, L, hard, hoef, tol_l = reference(deq(q8, ds[0])[1:], deq(k8, ds[1])[1:], deq(v8, ds[2])[1:],
                                 oracle_scale(0.125, ds[0], ds[1]), False, [33])
    check(o[1:], lse[1:], O, L, hard, hoef, tol_l, "fp8 key length 33")


@pytest.mark.parametrize("wid", [4, 5])
def test_fp8_workload_whole_heads(dev, wid):
    """The fp8 forms of the long workloads at full size (the benchmarked
    shapes): every row of the first and last head of each sequence against the
    oracle."""
    w = WORKLOADS[wid]
    q8, k8, v8, vt8, ds, kl = make_fp8(w.B, w.H, w.Hkv, w.N, w.d, seed=100 + w.seed, padded=w.padded)
    o, lse = run(dev, q8, k8, vt8, ds, w.scale, w.causal, kl)
    group = w.H // w.Hkv
    heads = [(b, h) for b in range(w.B) for h in (0, w.H - 1)]
    qd, kd, vd = deq(q8, ds[0]), deq(k8, ds[1]), deq(v8, ds[2])
    sc = oracle_scale(w.scale, ds[0], ds[1])

    def one(bh):
        b, h = bh
        return reference_head(qd[b, h], kd[b, h // group], vd[b, h // group], sc, w.causal,
                              None if kl is None else int(kl[b]))

    for (b, h), (O, L, hard, hoef, tol_l) in zip(heads, parallel_heads(one, heads)):
        check(o[b, h], lse[b, h], O, L, hard, hoef, tol_l, f"fp8 workload {wid} b={b} h={h}, all {w.N} rows")


# ------------------------------------------------------------------ preparation kernels


def signs_of(d, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randint(0, 2, (d,), generator=g, dtype=torch.int32).float() * 2.0 - 1.0


def check_bytes(x8_gpu, y64, descale, eps, what, slack=0.0):
    """Stored bytes against the oracle: the code of e4m3(y / descale), or a
    neighbour where y / descale lies within fp32 rounding of the GPU's
    rotation and scaling (relative eps, plus an absolute slack on y) of a
    rounding boundary."""
    got = as_f64(x8_gpu.cpu().float())
    z = y64 / descale
    dz = eps * np.abs(z) + np.asarray(slack) / descale
    lo = ofp8.e4m3_round(z - dz)
    hi = ofp8.e4m3_round(z + dz)
    exact = ofp8.e4m3_round(z)
    ok = (got >= lo) & (got <= hi)
    n_exact = int(np.sum(got == exact))
    print(f"  {what}: {got.size} bytes, {n_exact} equal to the nearest-even code, "
          f"{int(np.sum(ok)) - n_exact} at a boundary within fp32 rounding", flush=True)
    assert ok.all(), f"{what}: {int((~ok).sum())} bytes off the e4m3 rounding of the oracle's value"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rows", [0, 1, 7, 1000, 4099])
@pytest.mark.parametrize("rotate", [False, True])
def test_fp8_quantize_matches_oracle(dev, d, rows, rotate):
    """attn_fp8_amax then attn_fp8_quantize through the C ABI: the amax against
    the oracle's (fp32 rounding of the rotation), the descale bit for bit from
    the GPU's amax, and every byte against the e4m3 rounding of the oracle's
    rotated value."""
    g = torch.Generator("cpu").manual_seed(rows + d)
    x = (torch.randn((rows, d), generator=g) * 2.0).to(torch.bfloat16)
    if rows:
        x[:, 5] *= 40.0  # an outlier channel
    s = signs_of(d, 77) if rotate else None
    xd = x.to(dev)
    sd = None if s is None else s.to(dev)
    scal = torch.full((8,), -1.0, dtype=torch.float32, device=dev)  # [0] amax, [4] descale
    x8 = torch.empty((rows, d), dtype=torch.float8_e4m3fn, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    sp = None if sd is None else sd.data_ptr()
    assert attn.attn_fp8_amax(xd.data_ptr(), sp, rows, d, scal.data_ptr(), stream) == attn.ATTN_OK
    assert attn.attn_fp8_quantize(xd.data_ptr(), sp, rows, d, scal.data_ptr(), x8.data_ptr(), scal[4:].data_ptr(),
                                  stream) == attn.ATTN_OK
    torch.cuda.synchronize()
    gpu_amax, descale = float(scal[0].item()), float(scal[4].item())
    y = ofp8.rotate(as_f64(x), as_f64(s)) if rotate else as_f64(x)
    amax = float(np.abs(y).max()) if rows else 0.0
    assert abs(gpu_amax - amax) <= 1e-5 * amax, f"amax {gpu_amax} vs the oracle's {amax}"
    assert descale == ofp8.descale_of(gpu_amax), f"descale {descale} vs {ofp8.descale_of(gpu_amax)}"
    # the GPU rotates in fp32: each rotated value may be off by a few units of
    # 2^-24 of its row's absolute sum (seven butterfly stages), then scaled
    slack = 10 * 2.0 ** -24 * np.abs(as_f64(x)).sum(axis=1, keepdims=True) / math.sqrt(d) if rotate else 0.0
    check_bytes(x8, y, descale, 2.0 ** -22, f"quantize d={d} rows={rows} rotate={rotate}", slack=slack)


@pytest.mark.parametrize("N", [1, 16, 100, 130, 1000])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_quantize_vt_matches_oracle(dev, N, d):
    B, Hkv = 2, 3
    _, _, v, _ = make_qkv(B, 1, Hkv, N, d, "bf16", seed=N + 3 * d)
    vt8, descale = attn.quantize_fp8_vt(v.to(dev))
    torch.cuda.synchronize()
    n16 = (N + 15) // 16 * 16
    assert tuple(vt8.shape) == (B, Hkv, d, n16)
    raw = vt8.cpu().view(torch.uint8)
    assert torch.all(raw[..., N:] == 0), "columns past N must be zero"
    amax = float(np.abs(as_f64(v)).max())
    assert descale == ofp8.descale_of(amax), f"descale {descale} vs {ofp8.descale_of(amax)}"
    check_bytes(vt8[..., :N], as_f64(v).transpose(0, 1, 3, 2), descale, 2.0 ** -22, f"quantize_vt N={N} d={d}")


def test_fp8_prep_host_errors(dev):
    x = torch.zeros((4, 96), dtype=torch.bfloat16, device=dev)
    with pytest.raises(attn.AttnError) as e:
        attn.quantize_fp8(x)
    assert e.value.status == attn.ATTN_ERR_HEAD_DIM
    lib = attn.load_library()
    assert lib.attn_fp8_amax(None, None, 4, 64, None, None) == attn.ATTN_ERR_NULL
    assert lib.attn_fp8_quantize(None, None, -1, 64, None, None, None, None) == attn.ATTN_ERR_SHAPE


@pytest.mark.parametrize("causal", [False, True])
def test_incoherent_processing_lowers_the_error(dev, causal):
    """Queries and keys with outlier features (a few channels 30-60x the
    rest): the fp8 forward with the rotation applied to q and k (the same
    random signs) is closer to the exact attention of the bf16 inputs than
    without it, and in both cases the forward meets its bounds on the values
    the fp8 bytes stand for (the rotated ones when rotated)."""
    B, H, Hkv, N, d = 1, 4, 2, 777, 128
    q, k, v, _ = make_qkv(B, H, Hkv, N, d, "bf16", seed=31)
    q, k = q.float(), k.float()
    q[..., 3] *= 60.0
    q[..., 90] *= 30.0
    k[..., 3] *= 40.0
    k[..., 17] *= 30.0
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    scale = float(np.float32(0.002))
    O, L = oracle.attention(as_f64(q), as_f64(k), as_f64(v), scale, causal=causal)
    vt8, vds = attn.quantize_fp8_vt(v.to(dev))
    s = signs_of(d, 5)
    errs = {}
    for rotate in (False, True):
        sd = s.to(dev) if rotate else None
        q8, qds = attn.quantize_fp8(q.to(dev), sd)
        k8, kds = attn.quantize_fp8(k.to(dev), sd)
        o, lse = attn.forward_fp8(q8, k8, vt8, qds, kds, vds, scale=scale, causal=causal)
        torch.cuda.synchronize()
        o, lse = o.cpu(), lse.cpu()
        errs[rotate] = (float(np.max(np.abs(as_f64(o) - O))), float(np.max(np.abs(as_f64(lse) - L))))
        # the forward itself against the values its bytes stand for
        qv, kv = deq(q8.cpu(), qds), deq(k8.cpu(), kds)
        vv = deq(vt8.cpu()[..., :N].transpose(-1, -2), vds)
        Or, Lr, hard, hoef, tol_l = reference(qv, kv, vv, oracle_scale(scale, qds, kds), causal, None)
        check(o, lse, Or, Lr, hard, hoef, tol_l, f"fp8 with outliers rotate={rotate} causal={causal}")
    print(f"  error against the exact bf16 attention: O {errs[False][0]:.3e} -> {errs[True][0]:.3e}, "
          f"LSE {errs[False][1]:.3e} -> {errs[True][1]:.3e} with the rotation", flush=True)
    assert errs[True][0] < 0.5 * errs[False][0], "the rotation did not lower the output error"
    assert errs[True][1] < 0.5 * errs[False][1], "the rotation did not lower the LSE error"


def test_transpose_helper_layout():
    """workloads.transpose_fp8_v (test input layout) pads to whole 16-byte pieces."""
    v8 = torch.arange(2 * 3 * 5 * 4, dtype=torch.uint8).reshape(2, 3, 5, 4).view(torch.float8_e4m3fn)
    vt = transpose_fp8_v(v8).view(torch.uint8)
    assert tuple(vt.shape) == (2, 3, 4, 16)
    assert torch.equal(vt[..., :5], v8.view(torch.uint8).transpose(-1, -2)) and torch.all(vt[..., 5:] == 0)
