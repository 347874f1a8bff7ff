"""Checks that fix what an attention forward pass must return, independently of
any implementation of it.

Each ``pin_*`` takes ``fn(q, k, v, scale, causal=False, key_lens=None) ->
(O, LSE)`` on fp64 numpy arrays (q: [B, H, N, d]; k, v: [B, Hkv, N, d]) and
raises ``AssertionError`` on a mismatch.  The expected values come from closed
forms worked out from the definition of attention (the standard attention code
block of the zsdodo.com page; softmax with the max subtracted, unite.ai page,
section "闪电注意力的数学原理", formula 1), from invariants of that definition, from
a hand-derived fixture, or from a library routine (torch's fp64 CPU
scaled-dot-product attention) — never from the oracle itself.  The oracle must
pass all of them; ``test_oracle_mutants.py`` plants plausible mistakes in the
oracle and checks that some pin catches each one.
"""

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_closed_form.json")
TOL = 1e-12

# (B, H, Hkv, N, d): several tiny shapes with grouped heads and odd lengths
SHAPES = [(2, 4, 2, 13, 8), (1, 3, 1, 7, 5), (2, 2, 2, 1, 4), (1, 6, 3, 20, 3)]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    ninf_a, ninf_b = np.isneginf(a), np.isneginf(b)
    assert np.array_equal(ninf_a, ninf_b), f"{what}: -inf pattern differs"
    fa, fb = a[~ninf_a], b[~ninf_b]
    assert np.all(np.isfinite(fa)), f"{what}: non-finite values"
    err = np.max(np.abs(fa - fb)) if fa.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _key_len_cases(B, N):
    return [None, [max(N - 2, 1) if b % 2 == 0 else max(N // 2, 1) for b in range(B)]]


def _group(H, Hkv):
    return H // Hkv


def _admissible_count(i, key_len, causal):
    n = key_len
    if causal:
        n = min(n, i + 1)
    return n


# ---------------------------------------------------------------- P1
def pin_rows_sum_to_one(fn):
    """With every V entry equal to 1, each output entry is Σ_j P_ij, which must
    be 1 on any row with an admissible key (P is a probability distribution
    over the admissible keys), and 0 on a row with none (the empty-row
    reading)."""
    for si, (B, H, Hkv, N, d) in enumerate(SHAPES):
        q = _rand((B, H, N, d), 10 + si)
        k = _rand((B, Hkv, N, d), 20 + si)
        v = np.ones((B, Hkv, N, d))
        for causal in (False, True):
            for kls in _key_len_cases(B, N) + [[0] * B]:
                O, _ = fn(q, k, v, 0.7, causal=causal, key_lens=kls)
                want = np.ones_like(O)
                if kls is not None:
                    for b in range(B):
                        if kls[b] == 0:
                            want[b] = 0.0
                _close(O, want, what=f"rows-sum-to-1 {B,H,Hkv,N,d} causal={causal} kl={kls}")


# ---------------------------------------------------------------- P2
def pin_constant_scores_mean(fn):
    """Q ≡ 0 (or scale = 0) makes every admissible score equal, so O_i is the
    plain mean of v_j over the admissible keys and LSE_i = ln(count)."""
    for si, (B, H, Hkv, N, d) in enumerate(SHAPES):
        k = _rand((B, Hkv, N, d), 30 + si)
        v = _rand((B, Hkv, N, d), 40 + si)
        qr = _rand((B, H, N, d), 50 + si)
        for causal in (False, True):
            for kls in _key_len_cases(B, N):
                for q, scale in ((np.zeros((B, H, N, d)), 1.3), (qr, 0.0)):
                    O, L = fn(q, k, v, scale, causal=causal, key_lens=kls)
                    wantO = np.zeros_like(O)
                    wantL = np.zeros_like(L)
                    for b in range(B):
                        kl = N if kls is None else kls[b]
                        for h in range(H):
                            g = h // _group(H, Hkv)
                            for i in range(N):
                                n = _admissible_count(i, kl, causal)
                                wantO[b, h, i] = v[b, g, :n].sum(axis=0) / n
                                wantL[b, h, i] = math.log(n)
                    _close(O, wantO, what=f"mean-of-V O {B,H,Hkv,N,d} causal={causal} kl={kls}")
                    _close(L, wantL, what=f"mean-of-V LSE {B,H,Hkv,N,d} causal={causal} kl={kls}")


# ---------------------------------------------------------------- P3
def pin_one_hot_dominant(fn):
    """If one admissible key scores 60 above every other key, its V row is the
    output and its score is LSE, both to within N·e^-60 (below fp64 rounding)."""
    for si, (B, H, Hkv, N, d) in enumerate(SHAPES):
        if d < 2:
            continue
        v = _rand((B, Hkv, N, d), 60 + si)
        q = np.zeros((B, H, N, d))
        q[..., 0] = 1.0                       # every query is e_0
        for causal in (False, True):
            for kls in _key_len_cases(B, N):
                # dominant key: key 0 under causal (admissible for every row),
                # else the last admissible key
                k = _rand((B, Hkv, N, d), 70 + si) * 0.1
                k[..., 0] = 0.0
                jstar = []
                for b in range(B):
                    kl = N if kls is None else kls[b]
                    js = 0 if causal else kl - 1
                    k[b, :, js, 0] = 60.0
                    jstar.append(js)
                O, L = fn(q, k, v, 1.0, causal=causal, key_lens=kls)
                for b in range(B):
                    for h in range(H):
                        g = h // _group(H, Hkv)
                        want = np.broadcast_to(v[b, g, jstar[b]], O[b, h].shape)
                        # the other keys' weight (N·e^-60) is far below fp64
                        # rounding, so only rounding error remains
                        _close(O[b, h], want, tol=1e-13,
                               what=f"one-hot O b={b} h={h} causal={causal}")
                        _close(L[b, h], np.full(N, 60.0), tol=1e-13,
                               what=f"one-hot LSE b={b} h={h} causal={causal}")


# ---------------------------------------------------------------- P5
def _torch_reference(q, k, v, scale, causal, key_lens):
    import torch
    import torch.nn.functional as F
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    ok = torch.ones((B, 1, N, N), dtype=torch.bool)
    if causal:
        ok &= torch.tril(torch.ones((N, N), dtype=torch.bool))
    if key_lens is not None:
        for b in range(B):
            ok[b, :, :, key_lens[b]:] = False
    O = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=ok, scale=scale,
                                       enable_gqa=(H != Hkv))
    kr = tk.repeat_interleave(H // Hkv, dim=1)
    s = scale * (tq @ kr.transpose(-1, -2))
    s = s.masked_fill(~ok, float("-inf"))
    L = torch.logsumexp(s, dim=-1)
    return O.numpy(), L.numpy()


def pin_library_route(fn):
    """torch's fp64 CPU scaled_dot_product_attention (and logsumexp of the
    masked scores for LSE) must agree to 1e-12 on small shapes."""
    for si, (B, H, Hkv, N, d) in enumerate(SHAPES):
        q = _rand((B, H, N, d), 80 + si)
        k = _rand((B, Hkv, N, d), 90 + si)
        v = _rand((B, Hkv, N, d), 100 + si)
        for causal in (False, True):
            for kls in _key_len_cases(B, N):
                O, L = fn(q, k, v, 0.37, causal=causal, key_lens=kls)
                tO, tL = _torch_reference(q, k, v, 0.37, causal, kls)
                _close(O, tO, what=f"torch-sdpa O {B,H,Hkv,N,d} causal={causal} kl={kls}")
                _close(L, tL, what=f"torch-sdpa LSE {B,H,Hkv,N,d} causal={causal} kl={kls}")


# ---------------------------------------------------------------- P6
def pin_invariants(fn):
    """Properties of the definition that any correct result keeps."""
    B, H, Hkv, N, d = 2, 4, 2, 11, 6
    q = _rand((B, H, N, d), 111)
    k = _rand((B, Hkv, N, d), 112)
    v = _rand((B, Hkv, N, d), 113)
    scale = 0.45
    O, L = fn(q, k, v, scale)

    # permuting keys (K and V together) changes nothing when every key is admissible
    perm = np.random.default_rng(114).permutation(N)
    Op, Lp = fn(q, k[:, :, perm], v[:, :, perm], scale)
    _close(Op, O, what="key permutation O")
    _close(Lp, L, what="key permutation LSE")

    # adding u to every key shifts every score of row i by scale·q_i·u
    u = _rand((d,), 115) * 3.0
    Os, Ls = fn(q, k + u, v, scale)
    shift = scale * np.einsum("bhnd,d->bhn", q, u)
    _close(Os, O, tol=1e-11, what="key shift O")
    _close(Ls, L + shift, tol=1e-11, what="key shift LSE")

    # a huge shared shift must not overflow (max subtracted before exp)
    big = np.zeros((B, H, N, d))
    big[..., 0] = 1.0
    kb = k.copy()
    kb[..., 0] += 2.0e3
    Ob, Lb = fn(big, kb, v, 1.0)
    Ob0, Lb0 = fn(big, k, v, 1.0)
    _close(Ob, Ob0, tol=1e-9, what="overflow guard O")
    _close(Lb, Lb0 + 2.0e3, tol=1e-9, what="overflow guard LSE")

    # grouped heads equal multi-head attention on repeated K/V heads
    rep = H // Hkv
    Om, Lm = fn(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), scale)
    _close(Om, O, what="GQA == MHA(repeat) O")
    _close(Lm, L, what="GQA == MHA(repeat) LSE")

    # padding equals truncating K/V (query rows are unaffected in count)
    kls = [7, 3]
    Opad, Lpad = fn(q, k, v, scale, key_lens=kls)
    for b in range(B):
        kl = kls[b]
        # the first kl query rows of a padded run equal an unpadded run on
        # the sequence cut to its first kl positions
        Ot, Lt = fn(q[b:b + 1, :, :kl], k[b:b + 1, :, :kl], v[b:b + 1, :, :kl], scale)
        _close(Opad[b:b + 1, :, :kl], Ot, what="padding == truncation O")
        _close(Lpad[b:b + 1, :, :kl], Lt, what="padding == truncation LSE")
        # padded K/V content must not matter, whatever it is
        k2, v2 = k.copy(), v.copy()
        k2[b, :, kl:] = 1e4
        v2[b, :, kl:] = np.nan
        O2, L2 = fn(q, k2, v2, scale, key_lens=kls)
        _close(O2, Opad, what="padded content ignored O")
        _close(L2, Lpad, what="padded content ignored LSE")

    # causal row 0 sees only key 0; causal row N-1 sees every key
    Oc, Lc = fn(q, k, v, scale, causal=True)
    for b in range(B):
        for h in range(H):
            g = h // rep
            _close(Oc[b, h, 0], v[b, g, 0], what="causal row 0 O")
            _close(Lc[b, h, 0], scale * q[b, h, 0] @ k[b, g, 0], what="causal row 0 LSE")
    _close(Oc[:, :, -1], O[:, :, -1], what="causal last row O")
    _close(Lc[:, :, -1], L[:, :, -1], what="causal last row LSE")

    # causal equals non-causal on the prefix: row i under causal equals row i
    # of an unmasked run over the first i+1 keys
    for i in (1, 4, 9):
        Oi, Li = fn(q[:, :, :i + 1], k[:, :, :i + 1], v[:, :, :i + 1], scale)
        _close(Oc[:, :, i], Oi[:, :, i], what=f"causal prefix row {i} O")
        _close(Lc[:, :, i], Li[:, :, i], what=f"causal prefix row {i} LSE")


# ---------------------------------------------------------------- P7
def _load_golden():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    out = []
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)[None, None]
        k = np.array(c["k"], dtype=np.float64)[None, None]
        v = np.array(c["v"], dtype=np.float64)[None, None]
        O = np.array(c["O"], dtype=np.float64)[None, None]
        L = np.array([float(x) for x in c["LSE"]], dtype=np.float64)[None, None]
        out.append((c["name"], q, k, v, c["scale"], c["causal"], c["key_len"], O, L))
    return out


def pin_golden_tiny(fn):
    """Hand-derived values of tests/golden/tiny_closed_form.json."""
    for name, q, k, v, scale, causal, kl, O, L in _load_golden():
        gO, gL = fn(q, k, v, scale, causal=causal, key_lens=[kl])
        _close(gO, O, tol=1e-14, what=f"golden {name} O")
        _close(gL, L, tol=1e-14, what=f"golden {name} LSE")


ALL_PINS = [
    pin_rows_sum_to_one,
    pin_constant_scores_mean,
    pin_one_hot_dominant,
    pin_library_route,
    pin_invariants,
    pin_golden_tiny,
]
