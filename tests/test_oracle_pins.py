"""The fp64 oracle against every pin of tests/pins.py (CPU only)."""

import numpy as np
import pytest

import oracle
from tests import pins


def oracle_fn(q, k, v, scale, causal=False, key_lens=None):
    return oracle.attention(q, k, v, scale, causal=causal, key_lens=key_lens)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_meets_pin(pin):
    pin(oracle_fn)


def test_softmax_rows_closed_form():
    # exp values 1, 2, 5 over a row: weights 1/8, 2/8, 5/8, m = ln 5, ℓ = 8/5
    s = np.log(np.array([[1.0, 2.0, 5.0], [1.0, 1.0, 1.0]])) + np.array([[3.0], [-2.0]])
    p, m, ell = oracle.softmax_rows(s)
    assert np.allclose(p[0], [1 / 8, 2 / 8, 5 / 8], rtol=0, atol=1e-15)
    assert np.allclose(p[1], [1 / 3] * 3, rtol=0, atol=1e-15)
    assert abs(m[0] - (np.log(5.0) + 3.0)) < 1e-15 and abs(ell[0] - 8 / 5) < 1e-15
    assert abs(m[1] + 2.0) < 1e-15
    assert abs(ell[1] - 3.0) < 1e-15


def test_softmax_rows_empty_and_masked():
    s = np.array([[-np.inf, -np.inf], [0.0, -np.inf]])
    p, m, ell = oracle.softmax_rows(s)
    assert np.array_equal(p, [[0.0, 0.0], [1.0, 0.0]])
    assert m[0] == -np.inf and ell[0] == 0.0 and m[1] == 0.0 and ell[1] == 1.0


def test_row_sampling_is_exact():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 4, 37, 8))
    k = rng.standard_normal((2, 2, 37, 8))
    v = rng.standard_normal((2, 2, 37, 8))
    rows = np.array([0, 5, 17, 36])
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, 0.3, causal=causal, key_lens=[30, 11])
        Os, Ls = oracle.attention(q, k, v, 0.3, causal=causal, key_lens=[30, 11], rows=rows)
        assert np.array_equal(Os, O[:, :, rows]) and np.array_equal(Ls, L[:, :, rows])
        # small row chunks give the same values as one chunk
        Oc, Lc = oracle.attention(q, k, v, 0.3, causal=causal, key_lens=[30, 11], row_chunk=3)
        assert np.allclose(Oc, O, atol=1e-15, rtol=0) and np.allclose(Lc, L, atol=1e-15, rtol=0)


def test_key_lens_clamped():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 1, 9, 4))
    k = rng.standard_normal((2, 1, 9, 4))
    v = rng.standard_normal((2, 1, 9, 4))
    O1, L1 = oracle.attention(q, k, v, 0.5, key_lens=[100, -3])
    O2, L2 = oracle.attention(q, k, v, 0.5, key_lens=[9, 0])
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    assert np.all(O2[1] == 0) and np.all(L2[1] == -np.inf)
