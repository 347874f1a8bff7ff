"""fp64 definitions for the fp8 forward pass: the e4m3 format, per-tensor
quantisation, and the rotation used for incoherent processing.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the GPU path
may import this module.

Source: unite.ai page "闪电注意力：革命性地提高Transformer效率", section
"闪电注意力-3": FlashAttention-3 computes in FP8 and uses "incoherent
processing", which the page only describes by its purpose: it lowers the
quantisation error of low-precision formats.  Readings (the page gives no
format, scaling or transform):

* fp8 is OCP e4m3 ("E4M3FN": 1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits, subnormals below 2^-6, largest finite value 448, no
  infinities); a value is rounded to the nearest representable one, ties to
  the even mantissa, after clamping to ±448.
* One fp32 descale factor per tensor: descale = amax / 448 (amax the largest
  magnitude of the tensor; 1 when it is 0), stored = e4m3(x / descale), and
  a stored byte stands for descale · stored.
* Incoherent processing multiplies every query and key row, along the head
  dimension d, by one random orthogonal matrix R = H_d · diag(s) / √d: H_d
  the Sylvester–Hadamard matrix (H_1 = [1], H_2n = [[H_n, H_n], [H_n, −H_n]],
  so H[i, j] = (−1)^popcount(i & j)) and s a vector of random signs.  Since
  RᵀR = I, (R q)·(R k) = q·k: the scores, and hence O and LSE, are those of
  the unrotated inputs, while an outlier channel of q or k is spread evenly
  over all d channels before the per-tensor scale is chosen.  V is not
  rotated.
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6    # smallest normal binade 2^-6
E4M3_MANTISSA_BITS = 3


def hadamard(d):
    """The d × d Sylvester–Hadamard matrix (d a power of two), built by the
    doubling rule H_2n = [[H_n, H_n], [H_n, −H_n]]."""
    assert d >= 1 and d & (d - 1) == 0, "d must be a power of two"
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation(signs):
    """R = H_d · diag(signs) / √d for a sign vector of length d."""
    s = np.asarray(signs, dtype=np.float64)
    d = s.shape[0]
    return hadamard(d) * s[None, :] / np.sqrt(d)


def rotate(x, signs):
    """Every row (last axis) of x multiplied by R: y = R x (fp64)."""
    r = rotation(signs)
    return np.asarray(x, dtype=np.float64) @ r.T


def e4m3_round(x):
    """Nearest OCP e4m3 value (ties to even) of every entry of x (fp64), after
    clamping to ±448; NaN stays NaN.

    A finite y with |y| in the binade [2^e, 2^(e+1)), e ≥ −6, is a multiple of
    the step 2^(e − 3); below 2^-6 (subnormals) the step is 2^-9.  y / step is
    rounded to the nearest integer, ties to even (np.rint), which also keeps
    the last mantissa of a binade correct: rounding up to 2^(e+1) lands on the
    next binade's first value."""
    x = np.asarray(x, dtype=np.float64)
    y = np.clip(x, -E4M3_MAX, E4M3_MAX)
    a = np.abs(y)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, E4M3_MIN_NORMAL_EXP)
    step = np.exp2(e - E4M3_MANTISSA_BITS)
    out = np.rint(y / step) * step
    return np.where(np.isnan(x), np.nan, out)


def descale_of(amax):
    """The per-tensor descale factor for a tensor whose largest magnitude is
    amax: amax / 448 rounded to fp32 (the value the GPU receives), 1 when
    amax is 0."""
    return float(np.float32(np.float32(amax) / np.float32(E4M3_MAX))) if amax > 0 else 1.0


def quantize(x, descale):
    """Values the stored e4m3 bytes stand for: descale · e4m3(x / descale)."""
    return descale * e4m3_round(np.asarray(x, dtype=np.float64) / descale)
