"""The fp64 backward oracle against the pins of tests/pins_backward.py, and
planted mistakes in a copy of it that the pins must catch (CPU only)."""

import os
import types

import pytest

import oracle
from tests import pins_backward


def oracle_bwd(q, k, v, dout, scale, causal=False, key_lens=None):
    return oracle.attention_backward(q, k, v, dout, scale, causal=causal, key_lens=key_lens)


@pytest.mark.parametrize("pin", pins_backward.ALL_BPINS, ids=lambda p: p.__name__)
def test_backward_oracle_meets_pin(pin):
    pin(oracle_bwd)


SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")

MUTATIONS = [
    ("D not subtracted", "ds = p * (dp - D[:, None])", "ds = p * dp"),
    ("dQ without the scale", "dq[b, h] = scale * (ds @ kv_k)", "dq[b, h] = ds @ kv_k"),
    ("dK without the scale", "dk[b, g, :kl] += scale * (ds.T @ q[b, h])", "dk[b, g, :kl] += ds.T @ q[b, h]"),
    ("dK not summed over the group", "dk[b, g, :kl] += scale * (ds.T @ q[b, h])",
     "dk[b, g, :kl] = scale * (ds.T @ q[b, h])"),
    ("dV not summed over the group", "dv[b, g, :kl] += p.T @ do", "dv[b, g, :kl] = p.T @ do"),
    ("dV from dS", "dv[b, g, :kl] += p.T @ do", "dv[b, g, :kl] += (p * dp).T @ do"),
    ("dP against K", "dp = do @ kv_v.T", "dp = do @ kv_k.T"),
    ("D from P alone", "D = (p * dp).sum(axis=1)", "D = p.sum(axis=1)"),
    ("mask ignored in the backward", "s = np.where(admissible(rows, kl, causal), s, -np.inf)\n            p, _, _",
     "p, _, _"),
    ("dQ against V", "dq[b, h] = scale * (ds @ kv_k)", "dq[b, h] = scale * (ds @ kv_v)"),
    ("dK against dout", "dk[b, g, :kl] += scale * (ds.T @ q[b, h])", "dk[b, g, :kl] += scale * (ds.T @ do)"),
]


def _mutant(old, new):
    src = open(SRC_PATH).read()
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_bwd_mutant")
    exec(compile(src.replace(old, new), "oracle_bwd_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_backward_mutant_is_caught(name, old, new):
    mod = _mutant(old, new)

    def fn(q, k, v, dout, scale, causal=False, key_lens=None):
        return mod.attention_backward(q, k, v, dout, scale, causal=causal, key_lens=key_lens)

    caught = False
    for pin in pins_backward.ALL_BPINS:
        try:
            pin(fn)
        except Exception:
            caught = True
            break
    assert caught, f"mutation {name!r} passed every backward pin"
