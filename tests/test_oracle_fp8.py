"""Pins of the fp8 oracle (oracle/fp8.py): e4m3 rounding, per-tensor
quantisation and the incoherent-processing rotation, each against something
other than the oracle itself: the e4m3 bit layout decoded by hand, torch's
float8_e4m3fn cast, closed forms of the Hadamard matrix, and the invariance of
attention under a common orthogonal rotation of queries and keys.  Planted
mistakes in copies of the functions must be caught.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8


def decode_e4m3(code):
    """Value of an OCP e4m3 (E4M3FN) byte from its bit layout: sign bit 7,
    exponent bits 6..3 (bias 7), mantissa bits 2..0; exponent 0 is subnormal
    (m/8 · 2^-6); 0x7F and 0xFF are NaN."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


FINITE_CODES = [c for c in range(256) if (c & 0x7F) != 0x7F]
POSITIVE = sorted({decode_e4m3(c) for c in range(0x7F)})  # 0 .. 448, increasing


def check_e4m3_round(fn):
    # 1. representable values are fixed points
    vals = np.array([decode_e4m3(c) for c in FINITE_CODES])
    assert np.array_equal(fn(vals), vals), "a representable value moved"
    # 2. the midpoint of two neighbours goes to the one with the even mantissa
    for c in range(0, 0x7E):
        lo, hi = decode_e4m3(c), decode_e4m3(c + 1)
        want = lo if c % 2 == 0 else hi
        got = fn(np.array([(lo + hi) / 2, -(lo + hi) / 2]))
        assert got[0] == want and got[1] == -want, f"tie between codes {c:#x} and {c + 1:#x}: {got[0]} != {want}"
        # just off the midpoint: the nearer neighbour
        eps = (hi - lo) / 16
        assert fn(np.array([lo + eps]))[0] == lo and fn(np.array([hi - eps]))[0] == hi
    # 3. clamping, zero, NaN
    got = fn(np.array([448.0, 460.0, 1e9, -1e9, 0.0, np.nan]))
    assert np.array_equal(got[:5], [448.0, 448.0, 448.0, -448.0, 0.0]) and np.isnan(got[5])
    # 4. hand values: 1 + 1/16 ties to 1; 1 + 3/16 ties to 1.25; 2^-10 ties to 0; 3·2^-10 ties to 2^-8
    got = fn(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10]))
    assert np.array_equal(got, [1.0, 1.25, 0.0, 2.0 ** -8])
    # 5. library route: torch's float8_e4m3fn cast (nearest even) of clamped fp32 values
    x = torch.randn(20000, generator=torch.Generator().manual_seed(3)) * torch.exp2(
        torch.randint(-14, 10, (20000,), generator=torch.Generator().manual_seed(4)).float())
    x = x.clamp(-448, 448)
    want = x.to(torch.float8_e4m3fn).float().double().numpy()
    assert np.array_equal(fn(x.double().numpy()), want), "differs from torch's e4m3 cast"


def test_e4m3_round_pins():
    check_e4m3_round(fp8.e4m3_round)


def test_e4m3_round_mutants_are_caught():
    def truncate(x):  # rounds toward zero instead of to nearest
        x = np.clip(np.asarray(x, float), -448, 448)
        a = np.abs(x)
        e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
        step = np.exp2(e - 3)
        return np.where(np.isnan(x), np.nan, np.trunc(x / step) * step)

    def ties_away(x):  # rounds ties away from zero
        x = np.clip(np.asarray(x, float), -448, 448)
        a = np.abs(x)
        e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
        step = np.exp2(e - 3)
        return np.where(np.isnan(x), np.nan, np.sign(x) * np.floor(a / step + 0.5) * step)

    def no_subnormals(x):  # flushes the subnormal range to the smallest normal binade's step
        x = np.clip(np.asarray(x, float), -448, 448)
        a = np.abs(x)
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
        step = np.exp2(e - 3)
        return np.where(np.isnan(x), np.nan, np.rint(x / step) * step)

    def two_mantissa_bits(x):
        x = np.clip(np.asarray(x, float), -448, 448)
        a = np.abs(x)
        e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
        step = np.exp2(e - 2)
        return np.where(np.isnan(x), np.nan, np.rint(x / step) * step)

    def no_clamp(x):
        x = np.asarray(x, float)
        a = np.abs(x)
        e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
        step = np.exp2(e - 3)
        return np.where(np.isnan(x), np.nan, np.rint(x / step) * step)

    for mutant in (truncate, ties_away, no_subnormals, two_mantissa_bits, no_clamp):
        with pytest.raises(AssertionError):
            check_e4m3_round(mutant)


def test_descale_and_quantize():
    assert fp8.descale_of(448.0) == 1.0 and fp8.descale_of(0.0) == 1.0
    assert fp8.descale_of(3.5) == float(np.float32(np.float32(3.5) / np.float32(448)))
    x = np.random.default_rng(1).standard_normal(1000) * 3
    ds = fp8.descale_of(np.abs(x).max())
    qv = fp8.quantize(x, ds)
    # every value is descale times a representable e4m3 value, the largest maps near ±448
    assert np.all(np.isin(np.abs(qv / ds), POSITIVE))
    assert abs(np.abs(qv).max() / ds - 448.0) <= 32.0
    # relative error of the normal range at most 2^-4
    big = np.abs(x) / ds >= 2.0 ** -6
    assert np.all(np.abs(qv[big] - x[big]) <= 2.0 ** -4 * np.abs(x[big]) + 1e-15)


def check_rotation(rot_fn, had_fn):
    for d in (1, 2, 4, 8, 16, 64, 128):
        h = had_fn(d)
        # entrywise closed form (−1)^popcount(i & j), and orthogonality H Hᵀ = d I
        i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
        want = np.where(np.vectorize(lambda a: bin(a).count("1") % 2)(i & j) == 1, -1.0, 1.0)
        assert np.array_equal(h, want), f"H_{d} entries"
        assert np.array_equal(h @ h.T, d * np.eye(d)), f"H_{d} not orthogonal"
    d = 64
    s = np.where(np.random.default_rng(2).random(d) < 0.5, -1.0, 1.0)
    # a one-hot row e_j goes to s_j · H[:, j] / √d: every entry of magnitude 1/√d
    for jj in (0, 5, 63):
        e = np.zeros(d)
        e[jj] = 7.0
        y = rot_fn(e[None], s)[0]
        assert np.allclose(y, 7.0 * s[jj] * had_fn(d)[:, jj] / 8.0, atol=1e-15, rtol=0), "R e_j"
    # dot products are kept: (R q)·(R k) = q·k
    q = np.random.default_rng(3).standard_normal((5, d))
    k = np.random.default_rng(4).standard_normal((7, d))
    assert np.allclose(rot_fn(q, s) @ rot_fn(k, s).T, q @ k.T, atol=1e-12, rtol=0), "dot products"


def test_rotation_pins():
    check_rotation(fp8.rotate, fp8.hadamard)


def test_rotation_mutants_are_caught():
    def unnormalised(x, s):
        return np.asarray(x, float) @ (fp8.hadamard(len(s)) * np.asarray(s)[None, :]).T

    def signs_on_the_left(x, s):  # diag(s)·H instead of H·diag(s)
        r = np.asarray(s)[:, None] * fp8.hadamard(len(s)) / np.sqrt(len(s))
        return np.asarray(x, float) @ r.T

    def bad_hadamard(d):  # doubling rule with the sign in the wrong quadrant
        h = np.ones((1, 1))
        while h.shape[0] < d:
            h = np.block([[h, -h], [h, h]])
        return h

    with pytest.raises(AssertionError):
        check_rotation(unnormalised, fp8.hadamard)
    with pytest.raises(AssertionError):
        check_rotation(signs_on_the_left, fp8.hadamard)
    with pytest.raises(AssertionError):
        check_rotation(fp8.rotate, bad_hadamard)


@pytest.mark.parametrize("causal", [False, True])
def test_rotated_queries_and_keys_give_the_same_attention(causal):
    """Incoherent processing leaves the operation unchanged: attention of the
    rotated queries and keys (same rotation) equals attention of the originals
    in fp64, O and LSE, also with outlier channels."""
    B, H, Hkv, N, d = 2, 4, 2, 37, 64
    rng = np.random.default_rng(9)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    q[..., 3] *= 30.0
    k[..., 40] *= 25.0
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    O, L = oracle.attention(q, k, v, 0.05, causal=causal, key_lens=[30, 11])
    Or, Lr = oracle.attention(fp8.rotate(q, s), fp8.rotate(k, s), v, 0.05, causal=causal, key_lens=[30, 11])
    assert np.allclose(Or, O, atol=1e-12, rtol=0) and np.allclose(Lr, L, atol=1e-11, rtol=0)
    # and the rotation spreads the outliers: the largest rotated entry is far below the largest original one
    assert np.abs(fp8.rotate(q, s)).max() < 0.5 * np.abs(q).max()
