"""Checks that fix the gradients of attention, independently of any
implementation of them.

Each ``bpin_*`` takes ``fn(q, k, v, dout, scale, causal=False, key_lens=None)
-> (dQ, dK, dV)`` on fp64 numpy arrays (q, dout: [B, H, N, d]; k, v:
[B, Hkv, N, d]) — the gradients of L = Σ O ∘ dout with O the exact attention of
the standard attention code block of the zsdodo.com page (masked as the
forward pass is) — and raises ``AssertionError`` on a mismatch.  Expected
values come from torch's fp64 CPU autograd through the plain definition, from
central finite differences of the forward definition on tiny inputs, and from
invariants of the definition; never from the oracle's backward itself.
"""

import numpy as np

from tests.pins import SHAPES, _close, _key_len_cases, _rand

TOL = 1e-11


def _torch_forward(q, k, v, scale, causal, key_lens):
    """O = softmax(scale·Q Kᵀ, masked) V in torch fp64 (rows with no admissible
    key must not occur here: torch's softmax gives NaN on them)."""
    import torch
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    ok = torch.ones((B, 1, N, N), dtype=torch.bool)
    if causal:
        ok &= torch.tril(torch.ones((N, N), dtype=torch.bool))
    if key_lens is not None:
        for b in range(B):
            ok[b, :, :, key_lens[b]:] = False
    kr = k.repeat_interleave(H // Hkv, dim=1)
    vr = v.repeat_interleave(H // Hkv, dim=1)
    s = scale * (q @ kr.transpose(-1, -2))
    s = s.masked_fill(~ok, float("-inf"))
    return torch.softmax(s, dim=-1) @ vr


def _torch_grads(q, k, v, dout, scale, causal, key_lens):
    import torch
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    O = _torch_forward(tq, tk, tv, scale, causal, key_lens)
    O.backward(torch.tensor(dout, dtype=torch.float64))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def bpin_library_route(fn):
    """torch fp64 CPU autograd of the definition agrees to 1e-11."""
    for si, (B, H, Hkv, N, d) in enumerate(SHAPES):
        q = _rand((B, H, N, d), 300 + si)
        k = _rand((B, Hkv, N, d), 310 + si)
        v = _rand((B, Hkv, N, d), 320 + si)
        do = _rand((B, H, N, d), 330 + si)
        for causal in (False, True):
            for kls in _key_len_cases(B, N):
                got = fn(q, k, v, do, 0.41, causal=causal, key_lens=kls)
                ref = _torch_grads(q, k, v, do, 0.41, causal, kls)
                for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
                    _close(a, b, tol=TOL, what=f"autograd {name} {B,H,Hkv,N,d} causal={causal} kl={kls}")


def _loss(q, k, v, dout, scale, causal, key_lens):
    """Σ O ∘ dout with O written out from the definition in numpy fp64."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    total = 0.0
    for b in range(B):
        kl = N if key_lens is None else key_lens[b]
        for h in range(H):
            g = h // (H // Hkv)
            for i in range(N):
                n = min(kl, i + 1) if causal else kl
                if n <= 0:
                    continue
                s = scale * (k[b, g, :n] @ q[b, h, i])
                w = np.exp(s - s.max())
                total += (w / w.sum()) @ v[b, g, :n] @ dout[b, h, i]
    return total


def bpin_finite_differences(fn):
    """Central differences of the loss (step 1e-5) match every gradient entry
    to 1e-7 on tiny inputs (causal, padded, grouped heads)."""
    B, H, Hkv, N, d = 2, 2, 1, 5, 3
    q = _rand((B, H, N, d), 340)
    k = _rand((B, Hkv, N, d), 341)
    v = _rand((B, Hkv, N, d), 342)
    do = _rand((B, H, N, d), 343)
    for causal, kls in ((False, None), (True, None), (False, [3, 5]), (True, [4, 2])):
        got = fn(q, k, v, do, 0.7, causal=causal, key_lens=kls)
        for gi, x in enumerate((q, k, v)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp = x.copy(); xp[idx] += 1e-5
                xm = x.copy(); xm[idx] -= 1e-5
                args_p = [q, k, v]; args_p[gi] = xp
                args_m = [q, k, v]; args_m[gi] = xm
                num[idx] = (_loss(*args_p, do, 0.7, causal, kls) - _loss(*args_m, do, 0.7, causal, kls)) / 2e-5
            _close(got[gi], num, tol=1e-7, what=f"finite differences d{'QKV'[gi]} causal={causal} kl={kls}")


def bpin_invariants(fn):
    """Σ_j dV_j = Σ of dout over the rows that see a key; Σ_j dK_j = 0 (the
    softmax Jacobian's rows sum to zero); padded keys get zero gradients;
    scale = 0 gives dQ = dK = 0 and dV_j = Σ_i dout_i / count_i; grouped heads
    equal separate heads on repeated K/V with their gradients summed; a
    sequence with key length 0 gets all-zero gradients."""
    B, H, Hkv, N, d = 2, 4, 2, 11, 4
    G = H // Hkv
    q = _rand((B, H, N, d), 350)
    k = _rand((B, Hkv, N, d), 351)
    v = _rand((B, Hkv, N, d), 352)
    do = _rand((B, H, N, d), 353)
    for causal in (False, True):
        kls = [7, 11]
        dq, dk, dv = fn(q, k, v, do, 0.5, causal=causal, key_lens=kls)
        for b in range(B):
            for g in range(Hkv):
                rows_sum = do[b, g * G:(g + 1) * G].sum(axis=(0, 1))
                _close(dv[b, g].sum(axis=0), rows_sum, tol=1e-11, what="sum of dV")
                _close(dk[b, g].sum(axis=0), np.zeros(d), tol=1e-11, what="sum of dK")
                assert np.all(dk[b, g, kls[b]:] == 0) and np.all(dv[b, g, kls[b]:] == 0), "padded keys"
        # scale 0: uniform weights over the admissible keys
        dq0, dk0, dv0 = fn(q, k, v, do, 0.0, causal=causal, key_lens=kls)
        _close(dq0, np.zeros_like(dq0), tol=1e-14, what="dQ at scale 0")
        _close(dk0, np.zeros_like(dk0), tol=1e-14, what="dK at scale 0")
        want = np.zeros_like(dv0)
        for b in range(B):
            for h in range(H):
                g = h // G
                for i in range(N):
                    n = min(kls[b], i + 1) if causal else kls[b]
                    want[b, g, :n] += do[b, h, i] / n
        _close(dv0, want, tol=1e-12, what="dV at scale 0")
        # grouped heads = separate heads on repeated K/V, gradients summed per group
        kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
        dqm, dkm, dvm = fn(q, kr, vr, do, 0.5, causal=causal, key_lens=kls)
        _close(dq, dqm, tol=1e-12, what="GQA dQ")
        _close(dk, dkm.reshape(B, Hkv, G, N, d).sum(axis=2), tol=1e-12, what="GQA dK")
        _close(dv, dvm.reshape(B, Hkv, G, N, d).sum(axis=2), tol=1e-12, what="GQA dV")
    # an empty sequence
    dq, dk, dv = fn(q, k, v, do, 0.5, causal=False, key_lens=[0, 11])
    assert np.all(dq[0] == 0) and np.all(dk[0] == 0) and np.all(dv[0] == 0), "key length 0"


ALL_BPINS = [bpin_library_route, bpin_finite_differences, bpin_invariants]
