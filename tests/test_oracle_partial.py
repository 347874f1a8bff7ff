"""The key-block partial oracle and the S-way merge against the pins of
tests/pins_partial.py, and planted mistakes in a copy of them that the pins
must catch (CPU only)."""

import os
import types

import pytest

import oracle
from tests import pins_partial


def part(q, k, v, scale, causal, q_offset, k_offset):
    return oracle.attention_partial(q, k, v, scale, causal=causal, q_offset=q_offset, k_offset=k_offset)


@pytest.mark.parametrize("pin", pins_partial.ALL_PPINS, ids=lambda p: p.__name__)
def test_partial_oracle_meets_pin(pin):
    pin(part, oracle.merge_many)


SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")

MUTATIONS = [
    ("causal strict", "ok &= keys_abs[None, :] <= rows_abs[:, None]", "ok &= keys_abs[None, :] < rows_abs[:, None]"),
    ("query offset ignored", "rows_abs = q_offset + np.arange(Nq)", "rows_abs = np.arange(Nq)"),
    ("key offset with the wrong sign", "keys_abs = k_offset + np.arange(Nk)", "keys_abs = np.arange(Nk) - k_offset"),
    ("causal ignored in the block", "    if causal:\n        ok &= keys_abs", "    if False:\n        ok &= keys_abs"),
    ("LSE of the block without the max", "LSE[b, h] = np.where(live, m + np.log(np.where(live, ell, 1.0)), -np.inf)",
     "LSE[b, h] = np.where(live, np.log(np.where(live, ell, 1.0)), -np.inf)"),
    ("last part not merged", "for s in range(1, len(o_parts)):", "for s in range(1, len(o_parts) - 1):"),
    ("first part dropped", "o, lse = _f64(o_parts[0]), _f64(lse_parts[0])",
     "o, lse = 0.0 * _f64(o_parts[0]), np.full_like(_f64(lse_parts[0]), -np.inf)"),
]


def _mutant(old, new):
    with open(SRC_PATH) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_partial_mutant")
    exec(compile(src, "oracle_partial_mutant", "exec"), mod.__dict__)
    return mod


def _caught(check):
    try:
        check()
    except Exception:  # an assertion or any error the mistake provokes
        return True
    return False


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_partial_mutant_is_caught(name, old, new):
    m = _mutant(old, new)

    def mpart(q, k, v, scale, causal, q_offset, k_offset):
        return m.attention_partial(q, k, v, scale, causal=causal, q_offset=q_offset, k_offset=k_offset)
    assert any(_caught(lambda p=p: p(mpart, m.merge_many)) for p in pins_partial.ALL_PPINS), f"no pin caught: {name}"
