"""The packed-sequence oracle against the pins of tests/pins_varlen.py, and
planted mistakes in a copy of it that the pins must catch (CPU only)."""

import os
import types

import pytest

import oracle
from tests import pins_varlen


def oracle_varlen(q, k, v, cu, scale, causal):
    return oracle.attention_varlen(q, k, v, cu, scale, causal=causal)


@pytest.mark.parametrize("pin", pins_varlen.ALL_VPINS, ids=lambda p: p.__name__)
def test_varlen_oracle_meets_pin(pin):
    pin(oracle_varlen)


SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")

MUTATIONS = [
    ("sequence end one token late", "s0, s1 = cu[b], cu[b + 1]\n", "s0, s1 = cu[b], min(cu[b + 1] + 1, total)\n"),
    ("sequence start one token early", "s0, s1 = cu[b], cu[b + 1]\n", "s0, s1 = max(cu[b] - 1, 0), cu[b + 1]\n"),
    ("keys of the whole pack", "ks = k[s0:s1].transpose(1, 0, 2)[None]\n        vs = v[s0:s1].transpose(1, 0, 2)[None]",
     "ks = k[:s1].transpose(1, 0, 2)[None]\n        vs = v[:s1].transpose(1, 0, 2)[None]"),
    ("LSE rows of the wrong sequence", "LSE[:, s0:s1] = lse_b[0]", "LSE[:, total - s1:total - s0] = lse_b[0]"),
    ("heads and tokens swapped in q", "qs = q[s0:s1].transpose(1, 0, 2)[None]",
     "qs = q[s0:s1].reshape(q.shape[1], s1 - s0, q.shape[2])[None]"),
    ("causal dropped", "o_b, lse_b = attention(qs, ks, vs, scale, causal=causal)",
     "o_b, lse_b = attention(qs, ks, vs, scale, causal=False)"),
    ("V of the previous token", "vs = v[s0:s1].transpose(1, 0, 2)[None]",
     "vs = np.roll(v, 1, axis=0)[s0:s1].transpose(1, 0, 2)[None]"),
]


def _mutant(old, new):
    with open(SRC_PATH) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_varlen_mutant")
    exec(compile(src, "oracle_varlen_mutant", "exec"), mod.__dict__)
    return mod


def _caught(check):
    try:
        check()
    except Exception:  # an assertion or any error the mistake provokes
        return True
    return False


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_varlen_mutant_is_caught(name, old, new):
    m = _mutant(old, new)

    def fn(q, k, v, cu, scale, causal):
        return m.attention_varlen(q, k, v, cu, scale, causal=causal)
    assert any(_caught(lambda p=p: p(fn)) for p in pins_varlen.ALL_VPINS), f"no pin caught: {name}"
