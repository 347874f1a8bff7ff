"""Running the fp64 oracle over every head of a full-size workload.

The oracle computes one (b, h) head at a time; the heads are independent, so
they are spread over a thread pool (numpy releases the interpreter lock inside
its array operations and BLAS calls) with the BLAS pool limited to one thread
per worker.  The arithmetic is the oracle's own, unchanged: this only decides
which heads run at the same time.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from threadpoolctl import threadpool_limits

import oracle
from workloads import as_f64


def workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def parallel_heads(fn, items):
    """fn(item) for every item, on `workers()` threads with single-threaded BLAS;
    results in the order of `items`."""
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers()) as ex:
        return list(ex.map(fn, items))


def oracle_all_heads(q, k, v, scale, causal, key_lens):
    """oracle.attention over every (b, h) head of q [B, H, N, d] (k, v
    [B, Hkv, N, d]; key_lens None or B integers): (O [B, H, N, d], LSE [B, H, N])."""
    q64, k64, v64 = as_f64(q), as_f64(k), as_f64(v)
    B, H, N, d = q64.shape
    group = H // k64.shape[1]
    heads = [(b, h) for b in range(B) for h in range(H)]

    def one(bh):
        b, h = bh
        g = h // group
        return oracle.attention(q64[b:b + 1, h:h + 1], k64[b:b + 1, g:g + 1], v64[b:b + 1, g:g + 1], scale,
                                causal=causal, key_lens=None if key_lens is None else [int(key_lens[b])])

    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    for (b, h), (o, lse) in zip(heads, parallel_heads(one, heads)):
        O[b, h] = o[0, 0]
        L[b, h] = lse[0, 0]
    return O, L
