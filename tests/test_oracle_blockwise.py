"""Pin P4: the tiled online-softmax recurrence equals the full softmax.

Brute force on tiny fp64 inputs: every query-block size and every key-block
size from 1 to N (divisors or not), both loop orders (query-block outer as in
the code sketches, key-block outer as in the algorithm outline of the unite.ai
page, section "闪电注意力算法"), with causal and key-padding masks, must reproduce
the materialised result to 1e-12.  The merge of partial results over two
disjoint key ranges (unite.ai page, section "闪电注意力的数学原理", formula 2, in its
corrected reading) is checked at every split point.
"""

import numpy as np
import pytest

import oracle

TOL = 1e-12


def _inputs(B, H, Hkv, N, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d)) * 1.5
    k = rng.standard_normal((B, Hkv, N, d)) * 1.5
    v = rng.standard_normal((B, Hkv, N, d))
    return q, k, v


def blockwise_matches_full(blockwise, full, shapes, tol=TOL):
    """Raise AssertionError unless ``blockwise`` equals ``full`` for every
    block size pair, loop order and mask on the given shapes."""
    for si, (B, H, Hkv, N, d) in enumerate(shapes):
        q, k, v = _inputs(B, H, Hkv, N, d, 1000 + si)
        for causal in (False, True):
            for kls in (None, [N, max(N - 3, 0)][:B], [0, N // 2 + 1][:B]):
                O, L = full(q, k, v, 0.8, causal=causal, key_lens=kls)
                for bq in range(1, N + 1):
                    for bk in range(1, N + 1):
                        for kv_outer in (False, True):
                            Ob, Lb = blockwise(q, k, v, 0.8, bq, bk, causal=causal,
                                               key_lens=kls, kv_outer=kv_outer)
                            err = np.max(np.abs(Ob - O))
                            assert err <= tol, (B, H, N, d, causal, kls, bq, bk, kv_outer, err)
                            assert np.array_equal(np.isneginf(Lb), np.isneginf(L))
                            fin = ~np.isneginf(L)
                            lerr = np.max(np.abs(Lb[fin] - L[fin])) if fin.any() else 0.0
                            assert lerr <= tol, (B, H, N, d, causal, kls, bq, bk, kv_outer, lerr)


SHAPES = [(2, 2, 1, 9, 3), (1, 1, 1, 12, 4), (2, 3, 3, 5, 2)]


def test_every_block_size_both_loop_orders():
    blockwise_matches_full(oracle.blockwise_attention, oracle.attention, SHAPES)


def merges_match(merge_partials, attention, merge_softmax):
    rng = np.random.default_rng(7)
    B, H, Hkv, N, d = 2, 2, 2, 10, 3
    q, k, v = _inputs(B, H, Hkv, N, d, 77)
    O, L = attention(q, k, v, 0.9)
    for t in range(0, N + 1):
        # attention over keys [0, t) and over keys [t, N), merged
        Ox, Lx = attention(q, k, v, 0.9, key_lens=[t] * B)
        ky = np.concatenate([k[:, :, t:], k[:, :, :t]], axis=2)
        vy = np.concatenate([v[:, :, t:], v[:, :, :t]], axis=2)
        Oy, Ly = attention(q, ky, vy, 0.9, key_lens=[N - t] * B)
        Om, Lm = merge_partials(Ox, Lx, Oy, Ly)
        assert np.max(np.abs(Om - O)) <= TOL, ("merge O", t)
        assert np.max(np.abs(Lm - L)) <= TOL, ("merge LSE", t)
    for n, spread in ((2, 0.0), (5, 0.0), (11, 0.0), (6, 800.0), (7, -800.0)):
        # a large spread puts the two halves ~800 apart, so a merge that does
        # not take the larger max as reference overflows
        x = rng.standard_normal(n) * 4
        x[n // 2:] += spread
        full = np.exp(x - x.max()) / np.exp(x - x.max()).sum()
        for t in range(1, n):
            got = merge_softmax(x[:t], x[t:])
            assert np.max(np.abs(got - full)) <= TOL, ("merge softmax", n, t)


def test_merge_at_every_split():
    merges_match(oracle.merge_partials, oracle.attention, oracle.merge_softmax)


def test_merge_with_empty_side():
    o = np.arange(6.0).reshape(1, 2, 3)
    lse = np.array([[0.5, -1.0]])
    empty_o = np.zeros_like(o)
    empty_l = np.full_like(lse, -np.inf)
    Om, Lm = oracle.merge_partials(o, lse, empty_o, empty_l)
    assert np.array_equal(Om, o) and np.array_equal(Lm, lse)
    Om, Lm = oracle.merge_partials(empty_o, empty_l, empty_o, empty_l)
    assert np.all(Om == 0) and np.all(Lm == -np.inf)


@pytest.mark.parametrize("bs", [64, 128, 256])
def test_page_block_sizes_on_wider_input(bs):
    """The block sizes the pages' sketches use (64, 128, 256) on an input
    several blocks long with a ragged tail."""
    q, k, v = _inputs(1, 2, 1, 300, 8, 5)
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, 0.35, causal=causal, key_lens=[271])
        Ob, Lb = oracle.blockwise_attention(q, k, v, 0.35, bs, bs, causal=causal, key_lens=[271])
        assert np.max(np.abs(Ob - O)) <= TOL and np.max(np.abs(Lb - L)) <= TOL
