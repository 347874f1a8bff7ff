"""Pins of the key-block partial oracle (``oracle.attention_partial``) and
the S-way merge (``oracle.merge_many``).

Each pin takes ``part(q, k, v, scale, causal, q_offset, k_offset) -> (O, LSE)``
(q [B, H, Nq, d], k, v [B, Hkv, Nk, d]) and ``merge(o_parts, lse_parts) ->
(O, LSE)``, and checks them against something other than the oracle:

* ``ppin_brute_force``: plain Python loops over rows and keys from the
  definition at absolute positions (key j admissible for query i iff
  k_offset + j ≤ q_offset + i under a causal mask), with rows that see no key;
* ``ppin_whole_block``: a block holding every key, with equal offsets, is
  torch's fp64 scaled_dot_product_attention (a library route);
* ``ppin_shift``: adding the same amount to both offsets changes nothing, bit
  for bit;
* ``ppin_partition_merge``: the keys of a problem cut into blocks at ragged
  cut points, one partial per block, merged, give torch's fp64 attention of
  the whole problem, causal and not.
"""

import math

import numpy as np

TOL = 1e-12


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _close(a, b, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), what
    assert np.array_equal(a[~fin], b[~fin]), what
    err = np.max(np.abs(a[fin] - b[fin])) if fin.any() else 0.0
    assert err <= TOL, f"{what}: max abs error {err}"


def _brute(q, k, v, scale, causal, q_offset, k_offset):
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    O = np.zeros((B, H, Nq, d))
    L = np.full((B, H, Nq), -math.inf)
    for b in range(B):
        for h in range(H):
            g = h // (H // Hkv)
            for i in range(Nq):
                keys = [j for j in range(Nk) if not causal or k_offset + j <= q_offset + i]
                if not keys:
                    continue
                s = [scale * sum(float(q[b, h, i, x]) * float(k[b, g, j, x]) for x in range(d)) for j in keys]
                m = max(s)
                e = [math.exp(z - m) for z in s]
                ell = math.fsum(e)
                for x in range(d):
                    O[b, h, i, x] = math.fsum(e[n] * float(v[b, g, j, x]) for n, j in enumerate(keys)) / ell
                L[b, h, i] = m + math.log(ell)
    return O, L


def ppin_brute_force(part, merge):
    B, H, Hkv, Nq, Nk, d = 1, 2, 1, 5, 4, 3
    q, k, v = _rand((B, H, Nq, d), 1), _rand((B, Hkv, Nk, d), 2), _rand((B, Hkv, Nk, d), 3)
    for q_offset, k_offset in ((0, 0), (6, 2), (2, 4), (0, 9), (10, 0)):
        for causal in (False, True):
            O, L = part(q, k, v, 0.8, causal, q_offset, k_offset)
            Ob, Lb = _brute(q, k, v, 0.8, causal, q_offset, k_offset)
            _close(O, Ob, f"O offsets {q_offset},{k_offset} causal={causal}")
            _close(L, Lb, f"LSE offsets {q_offset},{k_offset} causal={causal}")


def ppin_whole_block(part, merge):
    from tests import pins

    B, H, Hkv, N, d = 2, 4, 2, 11, 5
    q, k, v = _rand((B, H, N, d), 4), _rand((B, Hkv, N, d), 5), _rand((B, Hkv, N, d), 6)
    for causal in (False, True):
        O, L = part(q, k, v, 0.3, causal, 7, 7)
        Ot, Lt = pins._torch_reference(q, k, v, 0.3, causal, None)
        _close(O, Ot, f"whole block O causal={causal}")
        _close(L, Lt, f"whole block LSE causal={causal}")


def ppin_shift(part, merge):
    B, H, Hkv, Nq, Nk, d = 1, 2, 2, 6, 9, 4
    q, k, v = _rand((B, H, Nq, d), 7), _rand((B, Hkv, Nk, d), 8), _rand((B, Hkv, Nk, d), 9)
    O, L = part(q, k, v, 0.5, True, 4, 1)
    O2, L2 = part(q, k, v, 0.5, True, 4 + 37, 1 + 37)
    assert np.array_equal(O, O2) and np.array_equal(L, L2), "result depends on more than q_offset − k_offset"


def ppin_partition_merge(part, merge):
    from tests import pins

    B, H, Hkv, N, d = 2, 2, 1, 13, 3
    q, k, v = _rand((B, H, N, d), 10), _rand((B, Hkv, N, d), 11), _rand((B, Hkv, N, d), 12)
    for cuts in ((0, 5, 13), (0, 1, 2, 9, 13), (0, 13)):
        for causal in (False, True):
            parts = [part(q, k[:, :, a:b], v[:, :, a:b], 0.7, causal, 0, a) for a, b in zip(cuts, cuts[1:])]
            O, L = merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
            Ot, Lt = pins._torch_reference(q, k, v, 0.7, causal, None)
            _close(O, Ot, f"merged O cuts={cuts} causal={causal}")
            _close(L, Lt, f"merged LSE cuts={cuts} causal={causal}")


ALL_PPINS = [ppin_brute_force, ppin_whole_block, ppin_shift, ppin_partition_merge]
