"""fp64 attention written out from its definition, plus the tiled recurrence.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the GPU path
may import this module.

Sources (web pages on exact tiled attention):

* "AI训练的最大障碍不是算力,而是“内存墙”" (zsdodo.com): the code block of
  standard PyTorch attention (scores = Q·Kᵀ/√d_k, softmax over the key axis,
  weights·V) and the ``safe_softmax_block`` code block (running max m and
  running exponent sum ℓ).
* "闪电注意力：革命性地提高Transformer效率" (unite.ai): section "闪电注意力的数学原理"
  (softmax decomposition, formula 1, and softmax merge, formula 2) and section
  "闪电注意力算法" (outer loop over K/V blocks, inner loop over Q blocks).
* "第四章 注意力机制实战案例" (aiknowledge.cn), §4.1.3: accumulated output scaled by
  α = exp(m_old − m_new) plus exp(S − m_new)·V, tail blocks cut with min(), and
  one division by the running sum at the end.
* aifi multi-head attention page (qqiyuan.cn), section "动态序列处理": padded
  positions are ignored through an attention mask.
* same unite.ai page, section "闪电注意力-2": grouped-query attention.
* aifi page, PyTorch example: activations stored token-major with the heads
  side by side (``b n (h d)``), the layout of the packed-sequence oracle.

Readings where the pages are silent:
causal admits keys j ≤ i; key padding admits j < key_len_b; grouped query
heads map to kv head h // (H / Hkv); a row with no admissible key has O = 0
and LSE = −∞; LSE is the natural-log log-sum-exp m + ln ℓ of the scaled
scores; ``scale`` is used exactly as passed (callers pass the fp32 value the
GPU receives).
"""

import numpy as np

__all__ = [
    "kv_head_of",
    "admissible",
    "scores",
    "softmax_rows",
    "attention",
    "blockwise_attention",
    "merge_partials",
    "merge_softmax",
    "attention_backward",
    "attention_varlen",
    "attention_partial",
    "merge_many",
]


def _f64(x):
    """Exact upcast of a float array (fp32 or bf16-valued fp32) to fp64."""
    return np.asarray(x, dtype=np.float64)


def kv_head_of(h, H, Hkv):
    """KV head read by query head ``h``: consecutive groups of H/Hkv query
    heads share one KV head (grouped-query attention, unite.ai page, section
    "闪电注意力-2"; the grouping rule itself is a reading)."""
    return h // (H // Hkv)


def admissible(rows, n_keys, causal):
    """Boolean [len(rows), n_keys]: key j is admissible for query row i.

    ``n_keys`` is already cut to the sequence's key length, so padding is
    handled by the caller truncating K and V (padded positions are ignored,
    aifi page, section "动态序列处理").  Causal keeps j ≤ i (a reading: no page
    defines a causal mask)."""
    rows = np.asarray(rows)
    ok = np.ones((rows.shape[0], n_keys), dtype=bool)
    if causal:
        ok &= np.arange(n_keys)[None, :] <= rows[:, None]
    return ok


def scores(q_rows, k_valid, scale):
    """S = scale · Q Kᵀ for the given query rows against the valid keys
    (step 1 of standard attention, zsdodo page)."""
    return scale * (_f64(q_rows) @ _f64(k_valid).T)


def softmax_rows(s):
    """Row softmax with the row max subtracted first (unite.ai page, section
    "闪电注意力的数学原理", formula 1: softmax(x) = exp(x − m)/Σ exp(x − m)).

    ``s`` is fp64 [R, n] with −∞ at inadmissible keys.  Returns
    (P, m, ℓ): P the normalised weights, m the row max, ℓ = Σ exp(s − m).
    A row with no finite entry gets P = 0, m = −∞, ℓ = 0."""
    s = _f64(s)
    if s.shape[1] == 0:
        r = s.shape[0]
        return np.zeros_like(s), np.full(r, -np.inf), np.zeros(r)
    m = s.max(axis=1)
    empty = m == -np.inf
    e = np.exp(s - np.where(empty, 0.0, m)[:, None])
    ell = e.sum(axis=1)
    p = e / np.where(empty, 1.0, ell)[:, None]
    return p, m, ell


def attention(q, k, v, scale, causal=False, key_lens=None, rows=None, row_chunk=512):
    """Exact attention, materialising S one chunk of query rows at a time.

    q: [B, H, N, d]; k, v: [B, Hkv, N, d] (any float dtype, upcast exactly to
    fp64).  key_lens: None or length-B integers (clamped to [0, N]).
    rows: None (all N query rows) or a 1-D array of query-row indices, the
    same for every (b, h) — row sampling is exact because softmax is taken
    row by row (the aifi and Blockwise Parallel Transformer pages both chunk
    the queries while keeping all keys).

    Returns (O, LSE): O fp64 [B, H, R, d], LSE fp64 [B, H, R] with
    LSE_i = m_i + ln ℓ_i (natural log), R = number of rows.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d) and v.shape == k.shape and H % Hkv == 0
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    O = np.zeros((B, H, R, d))
    LSE = np.full((B, H, R), -np.inf)
    for b in range(B):
        kl = N if key_lens is None else int(min(max(int(key_lens[b]), 0), N))
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            k_valid = k[b, g, :kl]
            v_valid = v[b, g, :kl]
            for c0 in range(0, R, row_chunk):
                r = rows[c0:c0 + row_chunk]
                s = scores(q[b, h, r], k_valid, scale)
                s = np.where(admissible(r, kl, causal), s, -np.inf)
                p, m, ell = softmax_rows(s)
                O[b, h, c0:c0 + len(r)] = p @ v_valid
                live = m > -np.inf
                LSE[b, h, c0:c0 + len(r)] = np.where(
                    live, m + np.log(np.where(live, ell, 1.0)), -np.inf)
    return O, LSE


def blockwise_attention(q, k, v, scale, block_q, block_k, causal=False,
                        key_lens=None, kv_outer=False):
    """The tiled forward pass, one (query block, key block) pair at a time.

    For each pair: S_blk = scale·Q_blk K_blkᵀ (inadmissible → −∞);
    m_new = max(m, rowmax S_blk); P = exp(S_blk − m_new);
    ℓ_new = exp(m − m_new)·ℓ + rowsum P (``safe_softmax_block``, zsdodo page);
    O ← exp(m − m_new)·O + P·V_blk (aiknowledge.cn §4.1.3); after the last
    block O ← O/ℓ and LSE = m + ln ℓ.  Tail blocks are cut at the sequence
    end.  ``kv_outer`` swaps the loops to the key-block-outer order of the
    unite.ai page, section "闪电注意力算法".  A row that has seen no admissible
    key keeps m = −∞; its exponent offset is taken as 0 so that no
    exp(−∞ − (−∞)) arises (a reading: the pages are silent).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    O_out = np.zeros((B, H, N, d))
    LSE_out = np.full((B, H, N), -np.inf)
    for b in range(B):
        kl = N if key_lens is None else int(min(max(int(key_lens[b]), 0), N))
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            m = np.full(N, -np.inf)
            ell = np.zeros(N)
            acc = np.zeros((N, d))
            qb = [(i0, min(i0 + block_q, N)) for i0 in range(0, N, block_q)]
            kb = [(j0, min(j0 + block_k, kl)) for j0 in range(0, kl, block_k)]
            pairs = ([(i, j) for j in kb for i in qb] if kv_outer
                     else [(i, j) for i in qb for j in kb])
            for (i0, i1), (j0, j1) in pairs:
                s = scale * (q[b, h, i0:i1] @ k[b, g, j0:j1].T)
                if causal:
                    ii = np.arange(i0, i1)[:, None]
                    jj = np.arange(j0, j1)[None, :]
                    s = np.where(jj <= ii, s, -np.inf)
                m_old = m[i0:i1]
                m_new = np.maximum(m_old, s.max(axis=1))
                off = np.where(m_new == -np.inf, 0.0, m_new)
                p = np.exp(s - off[:, None])
                alpha = np.exp(m_old - off)
                ell[i0:i1] = alpha * ell[i0:i1] + p.sum(axis=1)
                acc[i0:i1] = alpha[:, None] * acc[i0:i1] + p @ v[b, g, j0:j1]
                m[i0:i1] = m_new
            live = ell > 0
            O_out[b, h] = acc / np.where(live, ell, 1.0)[:, None]
            LSE_out[b, h] = np.where(live, m + np.log(np.where(live, ell, 1.0)), -np.inf)
    return O_out, LSE_out


def merge_partials(o_x, lse_x, o_y, lse_y):
    """Combine two attention results taken over disjoint key sets X and Y.

    Reading of the garbled softmax-merge formula (unite.ai page, section
    "闪电注意力的数学原理", formula 2): with LSE = ln(e^{LSE_x} + e^{LSE_y}),
    O = e^{LSE_x − LSE}·O_x + e^{LSE_y − LSE}·O_y.  Either side may be empty
    (LSE = −∞, O = 0)."""
    o_x, o_y = _f64(o_x), _f64(o_y)
    lse_x, lse_y = _f64(lse_x), _f64(lse_y)
    lse = np.logaddexp(lse_x, lse_y)
    live = lse > -np.inf
    ref = np.where(live, lse, 0.0)
    wx = np.where(live, np.exp(lse_x - ref), 0.0)
    wy = np.where(live, np.exp(lse_y - ref), 0.0)
    return wx[..., None] * o_x + wy[..., None] * o_y, lse


def merge_softmax(x, y):
    """softmax of the concatenation [x, y] from the two halves' statistics.

    With m = max(m_x, m_y) and ℓ = e^{m_x−m}ℓ_x + e^{m_y−m}ℓ_y, the result is
    [e^{m_x−m}ℓ_x·softmax(x), e^{m_y−m}ℓ_y·softmax(y)] / ℓ (the corrected
    reading of formula 2 in section "闪电注意力的数学原理" of the unite.ai page).
    x, y: 1-D score vectors, each with at least one finite entry."""
    px, mx, lx = softmax_rows(_f64(x)[None, :])
    py, my, ly = softmax_rows(_f64(y)[None, :])
    m = np.maximum(mx, my)
    wx = np.exp(mx - m) * lx
    wy = np.exp(my - m) * ly
    ell = wx + wy
    return np.concatenate([wx[:, None] * px, wy[:, None] * py], axis=1)[0] / ell[0]


def attention_backward(q, k, v, dout, scale, causal=False, key_lens=None):
    """Gradients of the loss L = Σ O ∘ dO through exact attention.

    The pages only say that the tiled method recomputes the attention weights
    in the backward pass instead of storing them (unite.ai page, section
    "闪电注意力的到来", key idea 2) and that FlashAttention-2 speeds the backward
    pass up (section "闪电注意力-2"); the gradients themselves are those of the
    definition above, written out by the chain rule (a reading), for each
    (b, h) with g = its kv head and A the admissible keys:

        P = softmax(S) with S = scale·Q Kᵀ over A,   O = P V
        dV_g += Pᵀ dO
        dP    = dO Vᵀ
        D_i   = Σ_j P_ij dP_ij   (= Σ_d dO_i,d O_i,d)
        dS    = P ∘ (dP − D)     (the softmax Jacobian applied to dP)
        dQ    = scale · dS K
        dK_g += scale · dSᵀ Q

    q, dout: [B, H, N, d]; k, v: [B, Hkv, N, d]; key_lens as in
    ``attention``.  Returns fp64 (dQ [B, H, N, d], dK [B, Hkv, N, d],
    dV [B, Hkv, N, d]).  Padded keys (j ≥ key_len) get dK = dV = 0; a row
    with no admissible key contributes nothing.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d) and v.shape == k.shape and dout.shape == q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rows = np.arange(N)
    for b in range(B):
        kl = N if key_lens is None else int(min(max(int(key_lens[b]), 0), N))
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            kv_k, kv_v = k[b, g, :kl], v[b, g, :kl]
            s = scores(q[b, h], kv_k, scale)
            s = np.where(admissible(rows, kl, causal), s, -np.inf)
            p, _, _ = softmax_rows(s)
            do = dout[b, h]
            dv[b, g, :kl] += p.T @ do
            dp = do @ kv_v.T
            D = (p * dp).sum(axis=1)
            ds = p * (dp - D[:, None])
            dq[b, h] = scale * (ds @ kv_k)
            dk[b, g, :kl] += scale * (ds.T @ q[b, h])
    return dq, dk, dv


def attention_varlen(q, k, v, cu_seqlens, scale, causal=False):
    """Exact attention over packed sequences.

    The sequences of a batch are laid end to end along the token axis of
    q [total, H, d] and k, v [total, Hkv, d] (the token-major ``b n (h d)``
    activations of the aifi page's PyTorch example, one sequence after the
    other), so padding never exists (aifi page, section "动态序列处理": padded
    positions must take no part).  Sequence b is tokens cu_seqlens[b] ..
    cu_seqlens[b + 1] − 1; it is the standard attention problem on its own
    tokens (query row i = its i-th token, keys = its tokens, causal keeps
    j ≤ i within the sequence), solved by ``attention`` with B = 1.

    Returns (O, LSE): O fp64 [total, H, d], LSE fp64 [H, total].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    total, H, d = q.shape
    Hkv = k.shape[1]
    cu = [int(x) for x in cu_seqlens]
    assert k.shape == (total, Hkv, d) and v.shape == k.shape
    assert cu[0] == 0 and cu[-1] == total and all(a <= b for a, b in zip(cu, cu[1:]))
    O = np.zeros((total, H, d))
    LSE = np.full((H, total), -np.inf)
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        if s1 == s0:
            continue
        # [len, heads, d] -> [1, heads, len, d]
        qs = q[s0:s1].transpose(1, 0, 2)[None]
        ks = k[s0:s1].transpose(1, 0, 2)[None]
        vs = v[s0:s1].transpose(1, 0, 2)[None]
        o_b, lse_b = attention(qs, ks, vs, scale, causal=causal)
        O[s0:s1] = o_b[0].transpose(1, 0, 2)
        LSE[:, s0:s1] = lse_b[0]
    return O, LSE


def attention_partial(q, k, v, scale, causal=False, q_offset=0, k_offset=0):
    """Attention of the queries over one block of keys, normalised within the
    block: the split-KV building block whose results the softmax-merge rule
    (unite.ai page, section "闪电注意力的数学原理", formula 2) combines.

    q: [B, H, Nq, d] with query i at position q_offset + i of the sequence;
    k, v: [B, Hkv, Nk, d] with key j at position k_offset + j.  Under a causal
    mask key j is admissible for query i iff k_offset + j ≤ q_offset + i (the
    causal reading at absolute positions).  Returns (O, LSE) over the block's
    admissible keys: O fp64 [B, H, Nq, d], LSE fp64 [B, H, Nq]; a row with no
    admissible key gets O = 0 and LSE = −∞.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    O = np.zeros((B, H, Nq, d))
    LSE = np.full((B, H, Nq), -np.inf)
    rows_abs = q_offset + np.arange(Nq)
    keys_abs = k_offset + np.arange(Nk)
    ok = np.ones((Nq, Nk), dtype=bool)
    if causal:
        ok &= keys_abs[None, :] <= rows_abs[:, None]
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            s = np.where(ok, scores(q[b, h], k[b, g], scale), -np.inf)
            p, m, ell = softmax_rows(s)
            O[b, h] = p @ v[b, g]
            live = m > -np.inf
            LSE[b, h] = np.where(live, m + np.log(np.where(live, ell, 1.0)), -np.inf)
    return O, LSE


def merge_many(o_parts, lse_parts):
    """Combine S partial results (o_parts [S, ..., d], lse_parts [S, ...]) over
    disjoint key sets by folding the two-way merge ``merge_partials`` (the
    merge is associative: LSE = ln Σ_s e^{LSE_s}, O = Σ_s e^{LSE_s − LSE} O_s)."""
    o, lse = _f64(o_parts[0]), _f64(lse_parts[0])
    for s in range(1, len(o_parts)):
        o, lse = merge_partials(o, lse, o_parts[s], lse_parts[s])
    return o, lse
