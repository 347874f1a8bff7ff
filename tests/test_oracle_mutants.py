"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch each one.

Each mutation is a textual edit of oracle/attention.py applied to an in-memory
copy that is executed as a fresh module; the real oracle is never modified.
A mutation is caught when some pin raises (AssertionError or any error the
mistake provokes).
"""

import os
import types

import pytest

from tests import pins
from tests.test_oracle_blockwise import SHAPES as BW_SHAPES
from tests.test_oracle_blockwise import blockwise_matches_full, merges_match

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")

# (name, old text, new text, which checks must catch it)
MUTATIONS = [
    ("gqa head map h % Hkv", "return h // (H // Hkv)", "return h % Hkv", "pins"),
    ("causal off by one (j < i)", "np.arange(n_keys)[None, :] <= rows[:, None]",
     "np.arange(n_keys)[None, :] < rows[:, None]", "pins"),
    ("causal reversed (j >= i)", "np.arange(n_keys)[None, :] <= rows[:, None]",
     "np.arange(n_keys)[None, :] >= rows[:, None]", "pins"),
    ("causal ignored", "    if causal:\n        ok &=", "    if False:\n        ok &=", "pins"),
    ("scale dropped", "return scale * (_f64(q_rows) @ _f64(k_valid).T)",
     "return (_f64(q_rows) @ _f64(k_valid).T)", "pins"),
    ("scale squared", "return scale * (_f64(q_rows) @ _f64(k_valid).T)",
     "return scale * scale * (_f64(q_rows) @ _f64(k_valid).T)", "pins"),
    ("feature index reversed in K", "return scale * (_f64(q_rows) @ _f64(k_valid).T)",
     "return scale * (_f64(q_rows) @ _f64(k_valid)[:, ::-1].T)", "pins"),
    ("no max subtraction", "e = np.exp(s - np.where(empty, 0.0, m)[:, None])",
     "e = np.exp(s)", "pins"),
    ("row sum replaced by row max", "ell = e.sum(axis=1)", "ell = e.max(axis=1)", "pins"),
    ("no normalisation", "p = e / np.where(empty, 1.0, ell)[:, None]", "p = e", "pins"),
    ("LSE without the max", "live, m + np.log(np.where(live, ell, 1.0)), -np.inf)",
     "live, np.log(np.where(live, ell, 1.0)), -np.inf)", "pins"),
    ("LSE in log2", "live, m + np.log(np.where(live, ell, 1.0)), -np.inf)",
     "live, m + np.log2(np.where(live, ell, 1.0)), -np.inf)", "pins"),
    ("padding off by one", "k_valid = k[b, g, :kl]\n            v_valid = v[b, g, :kl]",
     "k_valid = k[b, g, :kl + 1]\n            v_valid = v[b, g, :kl + 1]", "pins"),
    ("padding ignored", "k_valid = k[b, g, :kl]\n            v_valid = v[b, g, :kl]",
     "k_valid = k[b, g, :N]\n            v_valid = v[b, g, :N]", "pins"),
    ("K used in place of V", "O[b, h, c0:c0 + len(r)] = p @ v_valid",
     "O[b, h, c0:c0 + len(r)] = p @ k_valid", "pins"),
    ("query rows shifted", "s = scores(q[b, h, r], k_valid, scale)",
     "s = scores(q[b, h, (r + 1) % N], k_valid, scale)", "pins"),
    # the tiled recurrence: caught by the blockwise-vs-full brute force
    ("no alpha rescale of the accumulator", "acc[i0:i1] = alpha[:, None] * acc[i0:i1] + p @ v[b, g, j0:j1]",
     "acc[i0:i1] = acc[i0:i1] + p @ v[b, g, j0:j1]", "blockwise"),
    ("no alpha rescale of the running sum", "ell[i0:i1] = alpha * ell[i0:i1] + p.sum(axis=1)",
     "ell[i0:i1] = ell[i0:i1] + p.sum(axis=1)", "blockwise"),
    ("running max not kept", "m[i0:i1] = m_new", "m[i0:i1] = m_old", "blockwise"),
    ("blockwise causal off by one", "s = np.where(jj <= ii, s, -np.inf)",
     "s = np.where(jj < ii, s, -np.inf)", "blockwise"),
    ("blockwise tail block dropped", "for j0 in range(0, kl, block_k)]",
     "for j0 in range(0, kl - block_k + 1, block_k)]", "blockwise"),
    # the merge of partial results
    ("merge weight without reference", "wx = np.where(live, np.exp(lse_x - ref), 0.0)",
     "wx = np.where(live, np.exp(lse_x), 0.0)", "merge"),
    ("merge softmax ignores the other max", "m = np.maximum(mx, my)", "m = mx", "merge"),
]


def _mutant(old, new):
    with open(SRC_PATH) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _caught(check):
    try:
        check()
    except Exception:  # an assertion or any error the mistake provokes
        return True
    return False


@pytest.mark.parametrize("name,old,new,kind", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(name, old, new, kind):
    m = _mutant(old, new)
    if kind == "pins":
        def fn(q, k, v, scale, causal=False, key_lens=None):
            return m.attention(q, k, v, scale, causal=causal, key_lens=key_lens)
        assert any(_caught(lambda p=p: p(fn)) for p in pins.ALL_PINS), f"no pin caught: {name}"
    elif kind == "blockwise":
        import oracle
        assert _caught(lambda: blockwise_matches_full(m.blockwise_attention, oracle.attention,
                                                      BW_SHAPES[:1])), f"not caught: {name}"
    else:
        import oracle
        assert _caught(lambda: merges_match(m.merge_partials, oracle.attention,
                                            m.merge_softmax)), f"not caught: {name}"


def test_unmutated_copy_passes():
    """The copy mechanism itself must not break a correct oracle."""
    m = _mutant("return h // (H // Hkv)", "return h // (H // Hkv)")

    def fn(q, k, v, scale, causal=False, key_lens=None):
        return m.attention(q, k, v, scale, causal=causal, key_lens=key_lens)
    for p in pins.ALL_PINS:
        p(fn)
