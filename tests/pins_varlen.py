"""Pins of the packed-sequence oracle (``oracle.attention_varlen``).

Each pin takes a function ``fn(q, k, v, cu_seqlens, scale, causal) -> (O, LSE)``
with q [total, H, d], k, v [total, Hkv, d], O [total, H, d], LSE [H, total],
and checks it against something other than the oracle itself:

* ``vpin_brute_force``: every output token recomputed with plain Python loops
  straight from the definition (scores of the token against the keys of its own
  sequence, the row max, the exponent sum, the weighted sum of values), on tiny
  inputs with GQA, causal and non-causal, and empty sequences;
* ``vpin_isolation``: changing every token of the other sequences leaves a
  sequence's outputs bit-for-bit unchanged (no attention across sequences);
* ``vpin_order``: packing the same sequences in another order permutes the
  outputs the same way, bit for bit;
* ``vpin_equal_lengths``: with B sequences of one length L the packed problem
  is the dense [B, H, L, d] problem after the layout change, whose definition
  is pinned separately (closed forms, torch, brute force in ``tests/pins.py``).
"""

import math

import numpy as np

TOL = 1e-12


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def _brute(q, k, v, cu, scale, causal):
    """Plain loops over tokens: no arrays beyond indexing."""
    total, H, d = q.shape
    Hkv = k.shape[1]
    O = [[[0.0] * d for _ in range(H)] for _ in range(total)]
    L = [[-math.inf] * total for _ in range(H)]
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        for i in range(s1 - s0):
            t = s0 + i
            for h in range(H):
                g = h // (H // Hkv)
                keys = [j for j in range(s1 - s0) if (not causal or j <= i)]
                if not keys:
                    continue
                s = [scale * sum(float(q[t, h, x]) * float(k[s0 + j, g, x]) for x in range(d)) for j in keys]
                m = max(s)
                e = [math.exp(z - m) for z in s]
                ell = math.fsum(e)
                for x in range(d):
                    O[t][h][x] = math.fsum(e[n] * float(v[s0 + j, g, x]) for n, j in enumerate(keys)) / ell
                L[h][t] = m + math.log(ell)
    return np.array(O), np.array(L)


def _close(a, b, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), what
    assert np.array_equal(a[~fin], b[~fin]), what
    err = np.max(np.abs(a[fin] - b[fin])) if fin.any() else 0.0
    assert err <= TOL, f"{what}: max abs error {err}"


def vpin_brute_force(fn):
    cases = [
        ([3, 1, 4], 2, 1, 3, 0.7),
        ([0, 5, 0, 2], 4, 2, 2, -0.4),
        ([6], 2, 2, 4, 0.5),
    ]
    for n, (lengths, H, Hkv, d, scale) in enumerate(cases):
        cu = _cu(lengths)
        total = int(cu[-1])
        q = _rand((total, H, d), 10 + n)
        k = _rand((total, Hkv, d), 20 + n)
        v = _rand((total, Hkv, d), 30 + n)
        for causal in (False, True):
            O, LSE = fn(q, k, v, cu, scale, causal)
            Ob, Lb = _brute(q, k, v, cu, scale, causal)
            _close(O, Ob, f"O case {n} causal={causal}")
            _close(LSE, Lb, f"LSE case {n} causal={causal}")


def vpin_isolation(fn):
    lengths = [5, 3, 7]
    cu = _cu(lengths)
    total, H, Hkv, d = int(cu[-1]), 4, 2, 3
    q, k, v = _rand((total, H, d), 1), _rand((total, Hkv, d), 2), _rand((total, Hkv, d), 3)
    for causal in (False, True):
        O, LSE = fn(q, k, v, cu, 0.6, causal)
        for b in range(len(lengths)):
            s0, s1 = int(cu[b]), int(cu[b + 1])
            other = np.ones(total, dtype=bool)
            other[s0:s1] = False
            q2, k2, v2 = q.copy(), k.copy(), v.copy()
            q2[other] = _rand(q2[other].shape, 40 + b)
            k2[other] = 5.0 * _rand(k2[other].shape, 50 + b)
            v2[other] = _rand(v2[other].shape, 60 + b) - 3.0
            O2, LSE2 = fn(q2, k2, v2, cu, 0.6, causal)
            assert np.array_equal(O[s0:s1], O2[s0:s1]), f"sequence {b} depends on other sequences"
            assert np.array_equal(LSE[:, s0:s1], LSE2[:, s0:s1]), f"sequence {b} LSE depends on others"


def vpin_order(fn):
    lengths = [4, 0, 6, 2]
    perm = [2, 0, 3, 1]
    cu = _cu(lengths)
    total, H, Hkv, d = int(cu[-1]), 2, 1, 4
    q, k, v = _rand((total, H, d), 7), _rand((total, Hkv, d), 8), _rand((total, Hkv, d), 9)
    idx = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in perm]).astype(np.int64)
    cu_p = _cu([lengths[b] for b in perm])
    for causal in (False, True):
        O, LSE = fn(q, k, v, cu, 1.1, causal)
        Op, LSEp = fn(q[idx], k[idx], v[idx], cu_p, 1.1, causal)
        assert np.array_equal(Op, O[idx]), "outputs do not follow the sequence order"
        assert np.array_equal(LSEp, LSE[:, idx]), "LSE does not follow the sequence order"


def vpin_equal_lengths(fn):
    from tests import pins  # the dense definition's pins live there

    B, L, H, Hkv, d = 3, 9, 4, 2, 5
    q = _rand((B, H, L, d), 11)
    k = _rand((B, Hkv, L, d), 12)
    v = _rand((B, Hkv, L, d), 13)
    cu = _cu([L] * B)
    pack = lambda x: x.transpose(0, 2, 1, 3).reshape(B * L, x.shape[1], d)  # noqa: E731
    for causal in (False, True):
        O, LSE = fn(pack(q), pack(k), pack(v), cu, 0.45, causal)
        Od, LSEd = pins._torch_reference(q, k, v, 0.45, causal, None)
        _close(O, pack(np.asarray(Od)), f"O equal lengths causal={causal}")
        _close(LSE, np.asarray(LSEd).transpose(1, 0, 2).reshape(H, B * L), f"LSE equal lengths causal={causal}")


ALL_VPINS = [vpin_brute_force, vpin_isolation, vpin_order, vpin_equal_lengths]
