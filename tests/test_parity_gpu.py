"""GPU parity: the HIP kernels (called through the C ABI) against the fp64 oracle.

Tolerances (stated for exact attention on bf16/fp32 storage with fp32
accumulation): max |O_gpu − O_oracle| ≤ 1.5e-2 for bf16 inputs and ≤ 1e-5 for
fp32 inputs; max |LSE_gpu − LSE_oracle| ≤ 1e-3 over finite entries; −∞
entries must coincide and no NaN may appear.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_14_amd as attn
import oracle
from tests.fullsize import oracle_all_heads
from workloads import WORKLOADS, as_f64, make_inputs, make_qkv

pytestmark = pytest.mark.gpu

TOL_O = {"bf16": 1.5e-2, "f32": 1e-5}
TOL_LSE = 1e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    attn.load_library()
    return torch.device("cuda:0")


def run_gpu(dev, q, k, v, scale, causal, key_lens):
    o, lse = attn.forward(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=causal,
                          key_lens=None if key_lens is None else key_lens.to(dev))
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(o, lse, O, L, tol_o, what):
    o, lse = as_f64(o), as_f64(lse)
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    assert not np.isnan(lse).any(), f"{what}: NaN in LSE"
    assert np.array_equal(np.isneginf(lse), np.isneginf(L)), f"{what}: -inf pattern of LSE differs"
    eo = float(np.max(np.abs(o - O))) if o.size else 0.0
    fin = np.isfinite(L)
    el = float(np.max(np.abs(lse[fin] - L[fin]))) if fin.any() else 0.0
    print(f"  {what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= tol_o, f"{what}: max|dO| {eo:.3e} > {tol_o}"
    assert el <= TOL_LSE, f"{what}: max|dLSE| {el:.3e} > {TOL_LSE}"


def oracle_of(q, k, v, scale, causal, key_lens, rows=None):
    return oracle.attention(as_f64(q), as_f64(k), as_f64(v), scale, causal=causal,
                            key_lens=None if key_lens is None else key_lens.tolist(), rows=rows)


SMALL = [  # (B, H, Hkv, N, d): several tiles, ragged tails, grouped heads
    (1, 1, 1, 1, 64), (2, 2, 1, 17, 64), (1, 4, 2, 100, 128), (2, 2, 2, 129, 64),
    (1, 2, 1, 255, 128), (1, 3, 3, 300, 64), (2, 4, 1, 520, 128),
    # enough (b, h, query tile) work items that each workgroup keeps its whole
    # key range (small grids split the key range over two wave groups)
    (4, 64, 16, 260, 64), (2, 128, 32, 300, 128),
    # enough causal query tiles per CU for the non-persistent causal schedule
    (8, 64, 16, 300, 64),
    # d = 128 on a large grid: the eight-wave (256-row) workgroups, ragged
    # in the last query tile, causal and not
    (8, 64, 16, 300, 128),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dH%dKV%dN%dd%d" % s)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_small_shapes(dev, dtype, shape, causal, padded):
    B, H, Hkv, N, d = shape
    what = f"{dtype} {shape} causal={causal} padded={padded}"
    print(what, flush=True)
    q, k, v, kl = make_qkv(B, H, Hkv, N, d, dtype, seed=hash(shape) % 1000, padded=padded)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = run_gpu(dev, q, k, v, scale, causal, kl)
    O, L = oracle_of(q, k, v, scale, causal, kl)
    check(o, lse, O, L, TOL_O[dtype], what)


def _sample_rows(N, n=192, seed=0):
    """Row sample: both ends, every 128-row tile edge region, plus random rows."""
    fixed = {0, 1, 2, 31, 32, 63, 64, 127, 128, N - 1, N - 2, N - 128, N // 2}
    rng = np.random.default_rng(seed)
    rnd = set(rng.choice(N, size=min(n, N), replace=False).tolist())
    return np.array(sorted(r for r in fixed | rnd if 0 <= r < N))


@pytest.mark.parametrize("wid", sorted(WORKLOADS))
def test_workload_full_size(dev, wid):
    """Each named workload at its full size, in the launch configuration the
    benchmark times: every row of every head against the oracle (the heads run
    side by side on the host's cores)."""
    w = WORKLOADS[wid]
    print(f"workload {wid}: {w.name}", flush=True)
    q, k, v, kl = make_inputs(w)
    o, lse = run_gpu(dev, q, k, v, w.scale, w.causal, kl)
    O, L = oracle_all_heads(q, k, v, w.scale, w.causal, None if kl is None else kl.tolist())
    check(o, lse, O, L, TOL_O[w.dtype], f"{w.name}, all {w.B * w.H} heads x {w.N} rows")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_key_len_edge_values(dev, dtype):
    """key_len 0 (empty rows: O = 0, LSE = −∞), 1, N, and values outside
    [0, N] (clamped)."""
    B, H, Hkv, N, d = 6, 2, 1, 150, 64
    q, k, v, _ = make_qkv(B, H, Hkv, N, d, dtype, seed=11)
    kl = torch.tensor([0, 1, N, N + 77, -4, 129], dtype=torch.int32)
    for causal in (False, True):
        o, lse = run_gpu(dev, q, k, v, 0.125, causal, kl)
        O, L = oracle_of(q, k, v, 0.125, causal, kl)
        check(o, lse, O, L, TOL_O[dtype], f"{dtype} key_len edges causal={causal}")
        assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_padding_content_is_ignored(dev, dtype):
    """Padded K/V filled with 1e4 and with NaN give bitwise the same output."""
    B, H, Hkv, N, d = 2, 4, 2, 333, 128
    q, k, v, _ = make_qkv(B, H, Hkv, N, d, dtype, seed=12)
    kl = torch.tensor([200, 65], dtype=torch.int32)
    o0, l0 = run_gpu(dev, q, k, v, 0.09, False, kl)
    for fill in (1e4, float("nan")):
        k2, v2 = k.clone(), v.clone()
        for b in range(B):
            k2[b, :, kl[b]:] = fill
            v2[b, :, kl[b]:] = fill
        o1, l1 = run_gpu(dev, q, k2, v2, 0.09, False, kl)
        assert torch.equal(o1, o0) and torch.equal(l1, l0), f"padding fill {fill} leaked"
    O, L = oracle_of(q, k, v, 0.09, False, kl)
    check(o0, l0, O, L, TOL_O[dtype], f"{dtype} padded")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_constant_scores_give_mean_of_v(dev, dtype):
    """scale = 0 makes every admissible score equal: O_i is the mean of the
    admissible V rows and LSE_i = ln(count) (closed form, not the oracle)."""
    B, H, Hkv, N, d = 1, 2, 1, 260, 64
    q, k, v, _ = make_qkv(B, H, Hkv, N, d, dtype, seed=13)
    kl = torch.tensor([250], dtype=torch.int32)
    vv = as_f64(v)
    for causal in (False, True):
        o, lse = run_gpu(dev, q, k, v, 0.0, causal, kl)
        O = np.zeros((B, H, N, d))
        L = np.zeros((B, H, N))
        for i in range(N):
            n = min(250, i + 1) if causal else 250
            O[0, :, i] = vv[0, 0, :n].mean(axis=0)
            L[0, :, i] = math.log(n)
        check(o, lse, O, L, TOL_O[dtype], f"{dtype} mean-of-V causal={causal}")


def test_one_hot_dominant_key(dev):
    """One key scoring ~60 above the rest: O is that key's V row, exactly in
    bf16 (the output rounding of a bf16 value is exact)."""
    B, H, Hkv, N, d = 1, 2, 2, 200, 128
    _, k, v, _ = make_qkv(B, H, Hkv, N, d, "bf16", seed=14)
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    q[..., 0] = 1.0
    k[..., 0] = 0.0
    k[0, :, 77, 0] = 60.0
    o, lse = run_gpu(dev, q, k, v, 1.0, False, None)
    want = v[0, :, 77].unsqueeze(1).expand(H, N, d)
    assert torch.equal(o[0], want)
    assert float((lse - 60.0).abs().max()) <= 1e-3


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_late_dominant_key(dev, causal, d):
    """A key far past the first tiles scores 150 above the rest (about 216 in
    base-2 units, beyond the fp32 exponent range relative to the first tiles'
    max).  O must be that key's V row and LSE its score; rows before it (under
    the causal mask) must match the oracle."""
    B, H, Hkv, N = 1, 2, 1, 700
    _, k, v, _ = make_qkv(B, H, Hkv, N, d, "bf16", seed=18)
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    q[..., 0] = 1.0
    k[..., 0] = 0.0
    k[0, 0, 600, 0] = 150.0
    o, lse = run_gpu(dev, q, k, v, 1.0, causal, None)
    O, L = oracle_of(q, k, v, 1.0, causal, None)
    check(o, lse, O, L, TOL_O["bf16"], f"late dominant key d={d} causal={causal}")
    rows = slice(600, N)
    assert torch.equal(o[0, :, rows], v[0, 0, 600].expand(H, N - 600, d))
    assert float((lse[0, :, rows] - 150.0).abs().max()) <= 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_negative_scale(dev, dtype):
    B, H, Hkv, N, d = 1, 2, 1, 190, 128
    q, k, v, _ = make_qkv(B, H, Hkv, N, d, dtype, seed=15)
    for causal in (False, True):
        o, lse = run_gpu(dev, q, k, v, -0.2, causal, None)
        O, L = oracle_of(q, k, v, -0.2, causal, None)
        check(o, lse, O, L, TOL_O[dtype], f"{dtype} negative scale causal={causal}")


def test_repeat_runs_bitwise_identical_and_no_allocation(dev):
    """No atomics: three runs are bitwise equal.  The call allocates no device
    memory beyond the caller's O and LSE (the N×N matrix never exists)."""
    w = WORKLOADS[3]
    q, k, v, _ = make_inputs(w)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    outs = []
    for _ in range(3):
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats(dev)
        before = torch.cuda.memory_allocated(dev)
        attn.forward(q, k, v, scale=w.scale, causal=True, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.cuda.max_memory_allocated(dev) == before
        outs.append((o.clone(), lse.clone()))
    for oo, ll in outs[1:]:
        assert torch.equal(oo, outs[0][0]) and torch.equal(ll, outs[0][1])


def test_empty_problem_is_noop(dev):
    for B, N in ((0, 64), (2, 0)):
        q = torch.empty((B, 2, N, 64), dtype=torch.bfloat16, device=dev)
        o, lse = attn.forward(q, q, q)
        torch.cuda.synchronize()
        assert o.shape == q.shape and lse.shape == (B, 2, N)


def test_side_stream(dev):
    """The launch goes on the caller's stream."""
    q, k, v, _ = make_qkv(1, 2, 2, 300, 64, "bf16", seed=16)
    s = torch.cuda.Stream(dev)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, lse = attn.forward(qd, kd, vd, scale=0.125)
    s.synchronize()
    O, L = oracle_of(q, k, v, 0.125, False, None)
    check(o.cpu(), lse.cpu(), O, L, TOL_O["bf16"], "side stream")


def test_host_errors_through_binding(dev):
    q = torch.zeros((1, 3, 64, 64), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(attn.AttnError) as e:
        attn.forward(q, kv, kv)
    assert e.value.status == attn.ATTN_ERR_SHAPE
    q96 = torch.zeros((1, 1, 64, 96), dtype=torch.bfloat16, device=dev)
    with pytest.raises(attn.AttnError) as e:
        attn.forward(q96, q96, q96)
    assert e.value.status == attn.ATTN_ERR_HEAD_DIM


def test_long_single_head(dev):
    """A long sequence (N = 65536, causal) on one head: many key tiles per
    query tile; a row sample is checked."""
    B, H, Hkv, N, d = 1, 1, 1, 65536, 64
    q, k, v, _ = make_qkv(B, H, Hkv, N, d, "bf16", seed=17)
    o, lse = run_gpu(dev, q, k, v, 0.125, True, None)
    rows = _sample_rows(N, n=64, seed=17)
    O, L = oracle_of(q, k, v, 0.125, True, None, rows=rows)
    check(o[:, :, rows], lse[:, :, rows], O, L, TOL_O["bf16"], "N=65536 causal")
