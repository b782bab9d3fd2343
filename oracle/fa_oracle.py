"""fp64 CPU oracle for the FlashAttention forward and backward passes and split-KV decode.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code, table or constant with the HIP library and imports nothing from it.

What it computes is the plain definition of attention, written out so that it can
be checked by eye against the pages:

* the scaled score row  x[j] = q . K[j,:] * scale   (Kernel visualization: Flash
  Attention 1, "Derivation"; the page uses scale = 1/sqrt(d), here the caller
  passes it);
* the safe softmax  p_j = e^{x_j - m} / sum_t e^{x_t - m},  m = max_t x_t
  (Softmax and FlashAttention, first "Concept" on online softmax);
* the output as the softmax-weighted mean of the rows of V  (Flash Attention 1
  page, "Derivation");
* LSE = m + ln(sum_t e^{x_t - m}), natural log of the scaled scores, one fp32
  number per query row in the kernel's output (Attention kernel chains, "The
  log-sum-exp merge" and "What the backward pass saves");
* the bottom-right causal rule: with T queries over S keys, query row i sits at
  position S - T + i and sees key j iff j <= i + (S - T)  (Attention kernel
  chains, "The causal mask for a decode step");
* GQA: query head h reads KV head h // g, g = H_q / H_kv, contiguous groups
  (Attention kernel chains, "GQA loads KV once per group");
* paged KV: token j of sequence b lives in pool page block_table[b, j // P],
  slot j % P  (Attention kernel chains, "The block-table cost of paged attention");
* the LSE merge of normalized partials: lse = ln sum_s e^{lse_s},
  O = sum_s e^{lse_s - lse} O_s  (Attention kernel chains, "The log-sum-exp merge");
* the backward pass: dQ, dK, dV for an upstream gradient dO, with the extra row
  vector D = rowsum(dO * O)  (Attention kernel chains, "What the backward pass
  saves"); the other steps are the chain rule of the definition above.

The two online recurrences at the bottom (``online_softmax_fa2`` and
``online_softmax_fa1``) follow the steps of the pages' derivation in the pages'
notation.  They are not used to produce expected values for the GPU: they exist
so that the pin tests can show, on the pages' own worked example and by brute
force, that the streamed recurrence equals the two-pass definition above.

Rows that see no key at all (causal with N_q > N_k, or an empty key range) have
O = 0 and LSE = -inf; that reading is the oracle's, the pages are silent on it.
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# The causal mask, bottom-right aligned
# ---------------------------------------------------------------------------

def is_visible(i: int, j: int, n_q: int, n_k: int, causal: bool) -> bool:
    """Whether query row ``i`` (of ``n_q``) may attend to key ``j`` (of ``n_k``).

    Attention kernel chains, "The causal mask for a decode step": T new queries
    over S keys, query row i is at absolute position S - T + i, and key j is
    visible when j <= i + (S - T).  Here T = n_q and S = n_k.
    """
    if not (0 <= j < n_k):
        return False
    if not causal:
        return True
    return j <= i + (n_k - n_q)


def visible_mask(n_q: int, n_k: int, causal: bool, rows=None) -> np.ndarray:
    """Boolean [len(rows), n_k] matrix of ``is_visible`` for the given query rows
    (default: all n_q rows).  Same rule, vectorised."""
    i = (np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64))[:, None]
    j = np.arange(n_k)[None, :]
    if not causal:
        return np.ones((i.shape[0], n_k), dtype=bool)
    return j <= i + (n_k - n_q)


# ---------------------------------------------------------------------------
# Safe softmax and one attention head
# ---------------------------------------------------------------------------

def safe_softmax(x: np.ndarray) -> np.ndarray:
    """p_i = e^{x_i - m} / sum_j e^{x_j - m} with m = max_j x_j, along the last axis.

    Softmax and FlashAttention, "Concept" (online softmax paragraph).
    """
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def logsumexp(x: np.ndarray) -> np.ndarray:
    """ln sum_j e^{x_j}, computed as m + ln sum_j e^{x_j - m}; -inf for an empty or all -inf row."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] == 0:
        return np.full(x.shape[:-1], NEG_INF)
    m = np.max(x, axis=-1, keepdims=True)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    s = np.sum(np.exp(x - m_safe), axis=-1, keepdims=True)
    with np.errstate(divide="ignore"):
        out = np.where(finite, m_safe + np.log(s), NEG_INF)
    return out[..., 0]


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   causal: bool, rows=None, row_chunk: int = 512):
    """One (batch, head): O [n, d] and LSE [n] in fp64.

    q: [n_q, d] (all query rows of the head); k, v: [n_k, d].  ``rows`` selects
    which query rows to compute (default: all); the mask uses their true index.

    Naive three steps per row, exactly as the definition reads: the full score
    row x = scale * q K^T (a library matmul), the mask, the safe softmax, then
    the weighted sum P V.  Rows are processed ``row_chunk`` at a time only to
    bound memory; each row is still computed whole.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q = q.shape[0]
    n_k = k.shape[0]
    sel = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(sel), v.shape[1]), dtype=np.float64)
    lse = np.full((len(sel),), NEG_INF, dtype=np.float64)
    if n_k == 0:
        return out, lse
    for r0 in range(0, len(sel), row_chunk):
        r = sel[r0:r0 + row_chunk]
        x = scale * (q[r] @ k.T)                          # scores, [rows, n_k]
        x = np.where(visible_mask(n_q, n_k, causal, rows=r), x, NEG_INF)
        m = np.max(x, axis=1, keepdims=True)              # row max over visible keys
        seen = np.isfinite(m[:, 0])                       # rows with at least one visible key
        m_safe = np.where(seen[:, None], m, 0.0)
        e = np.exp(x - m_safe)                            # e^{x_j - m}; 0 where masked
        l = np.sum(e, axis=1, keepdims=True)              # the softmax denominator
        p = np.divide(e, l, out=np.zeros_like(e), where=l > 0)
        out[r0:r0 + len(r)] = p @ v
        with np.errstate(divide="ignore"):
            lse[r0:r0 + len(r)] = np.where(seen, m_safe[:, 0] + np.log(np.where(seen, l[:, 0], 1.0)), NEG_INF)
    return out, lse


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, causal: bool,
              rows=None):
    """Multi-head attention with GQA.

    Q: [B, H_q, N_q, d]; K, V: [B, H_kv, N_k, d]; H_q % H_kv == 0 and query
    head h reads KV head h // (H_q // H_kv).  Returns O [B, H_q, N_q, d] and
    LSE [B, H_q, N_q] in fp64.

    ``rows`` (optional): query-row indices to compute instead of all of them
    (sampled checks at full size); N_q in the outputs becomes len(rows).  The
    mask still uses the full N_q, so sampled rows equal the rows of the full
    result.
    """
    B, H_q, N_q, d = Q.shape
    _, H_kv, N_k, _ = K.shape
    assert H_q % H_kv == 0, "H_q must be a multiple of H_kv"
    g = H_q // H_kv
    n = N_q if rows is None else len(rows)
    O = np.zeros((B, H_q, n, V.shape[-1]), dtype=np.float64)
    L = np.full((B, H_q, n), NEG_INF, dtype=np.float64)
    for b in range(B):
        for h in range(H_q):
            O[b, h], L[b, h] = attention_head(Q[b, h], K[b, h // g], V[b, h // g],
                                              scale, causal, rows=rows)
    return O, L


# ---------------------------------------------------------------------------
# Paged KV
# ---------------------------------------------------------------------------

def gather_pages(pool: np.ndarray, block_table: np.ndarray, n_k: int, page_size: int) -> np.ndarray:
    """Contiguous K (or V) [B, H_kv, n_k, d] from a paged pool.

    pool: [num_pages, page_size, H_kv, d]; block_table: [B, pages_per_seq] int.
    Token j of sequence b is pool[block_table[b, j // page_size], j % page_size]
    (Attention kernel chains, "The block-table cost of paged attention": one
    int32 per 16-token block).
    """
    B = block_table.shape[0]
    _, ps, H_kv, d = pool.shape
    assert ps == page_size
    out = np.empty((B, H_kv, n_k, d), dtype=pool.dtype)
    for b in range(B):
        for j in range(0, n_k, page_size):
            page = int(block_table[b, j // page_size])
            cnt = min(page_size, n_k - j)
            out[b, :, j:j + cnt, :] = np.transpose(pool[page, :cnt], (1, 0, 2))
    return out


def decode(Q, K, V, scale: float, causal: bool, block_table=None, page_size=None,
           n_k=None, rows=None):
    """Decode attention: T = Q.shape[2] new queries over the N_k cached keys.

    K, V are contiguous [B, H_kv, N_k, d]; or, when ``block_table`` is given,
    pools [num_pages, page_size, H_kv, d] whose sequences hold ``n_k`` tokens
    (default pages_per_seq * page_size).  The result is the unsplit attention:
    a split-KV kernel must reproduce it for any split of the keys (Attention
    kernel chains, "The log-sum-exp merge").
    """
    if block_table is not None:
        if n_k is None:
            n_k = block_table.shape[1] * page_size
        K = gather_pages(K, block_table, n_k, page_size)
        V = gather_pages(V, block_table, n_k, page_size)
    return attention(Q, K, V, scale, causal, rows=rows)


# ---------------------------------------------------------------------------
# Split partials and the LSE merge
# ---------------------------------------------------------------------------

def split_partials(Q, K, V, scale: float, causal: bool, bounds):
    """Normalized partial outputs over key ranges: for each [a, b) in ``bounds``,
    attention restricted to keys a..b-1 (with the global causal rule), giving
    (O_s normalized by its own sum, lse_s).  An empty range, or a range a row
    cannot see, gives O_s = 0 and lse_s = -inf.

    Attention kernel chains, "The log-sum-exp merge": a split's result is its
    output already divided by its own softmax sum, kept together with that sum's log.
    """
    B, H_q, N_q, d = Q.shape
    _, H_kv, N_k, _ = K.shape
    g = H_q // H_kv
    vis = visible_mask(N_q, N_k, causal)
    O_parts = np.zeros((len(bounds), B, H_q, N_q, V.shape[-1]))
    L_parts = np.full((len(bounds), B, H_q, N_q), NEG_INF)
    for s, (a, e_) in enumerate(bounds):
        if e_ <= a:
            continue
        for b in range(B):
            for h in range(H_q):
                hk = h // g
                x = scale * (np.asarray(Q[b, h], np.float64) @ np.asarray(K[b, hk, a:e_], np.float64).T)
                x = np.where(vis[:, a:e_], x, NEG_INF)
                m = np.max(x, axis=1, keepdims=True)
                m_safe = np.where(np.isfinite(m), m, 0.0)
                ex = np.exp(x - m_safe)
                l = np.sum(ex, axis=1, keepdims=True)
                p = np.divide(ex, l, out=np.zeros_like(ex), where=l > 0)
                O_parts[s, b, h] = p @ np.asarray(V[b, hk, a:e_], np.float64)
                with np.errstate(divide="ignore"):
                    L_parts[s, b, h] = np.where(l[:, 0] > 0, m_safe[:, 0] + np.log(l[:, 0]), NEG_INF)
    return O_parts, L_parts


def lse_merge(O_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge normalized partials.  O_parts: [ns, ..., d]; lse_parts: [ns, ...].

    lse = ln sum_s e^{lse_s} (computed against m* = max_s lse_s),
    O = sum_s e^{lse_s - lse} O_s.   Attention kernel chains, "The log-sum-exp
    merge".  When every lse_s is -inf the row saw no key: O = 0, lse = -inf.
    """
    O_parts = np.asarray(O_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = np.max(lse_parts, axis=0)
    seen = np.isfinite(m)
    m_safe = np.where(seen, m, 0.0)
    s = np.sum(np.exp(lse_parts - m_safe[None]), axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(seen, m_safe + np.log(np.where(seen, s, 1.0)), NEG_INF)
    lse_safe = np.where(seen, lse, 0.0)
    w = np.where(seen[None], np.exp(lse_parts - lse_safe[None]), 0.0)   # e^{lse_s - lse}
    O = np.sum(w[..., None] * O_parts, axis=0)
    return O, lse


# ---------------------------------------------------------------------------
# Backward pass
# ---------------------------------------------------------------------------

def attention_head_backward(q, k, v, do, scale: float, causal: bool, o=None, row_chunk: int = 512):
    """Gradients dQ [n_q, d], dK [n_k, d], dV [n_k, d] of one head, in fp64, for the
    upstream gradient dO [n_q, d] of O = softmax(scale * q K^T, masked) V.

    Attention kernel chains, "What the backward pass saves": the backward keeps Q, K,
    V, O and the per-row LSE, rebuilds P from them, and needs one extra vector per
    row, D = rowsum(dO * O).  The pages give no more of it; the remaining steps are
    the chain rule of the forward definition, written out:

        P   = the masked safe softmax of the score row (zeros for a row with no key)
        O   = P V,                 D_i = sum_c dO[i,c] O[i,c]
        dV  = P^T dO               (O is linear in V)
        dP  = dO V^T
        dS  = P * (dP - D)         (softmax Jacobian: dS_ij = P_ij (dP_ij - sum_t P_it dP_it))
        dQ  = scale dS K,          dK = scale dS^T q

    ``o`` (optional): the output O [n_q, d] as the forward saved it (for instance rounded
    to bf16); D is then taken from it, as the backward receives it.  Default: the exact O.
    With the exact O the result is the exact gradient.

    Rows are taken ``row_chunk`` at a time only to bound memory; dK and dV are the
    sums of the chunks' contributions.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n_q, n_k = q.shape[0], k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if n_k == 0:  # no key: every row sees nothing, O = 0 does not depend on q
        return dq, dk, dv
    for r0 in range(0, n_q, row_chunk):
        r = np.arange(r0, min(n_q, r0 + row_chunk))
        x = scale * (q[r] @ k.T)
        x = np.where(visible_mask(n_q, n_k, causal, rows=r), x, NEG_INF)
        m = np.max(x, axis=1, keepdims=True)
        m_safe = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(x - m_safe)
        l = np.sum(e, axis=1, keepdims=True)
        p = np.divide(e, l, out=np.zeros_like(e), where=l > 0)
        o_rows = p @ v if o is None else np.asarray(o, dtype=np.float64)[r]
        D = np.sum(do[r] * o_rows, axis=1)
        dv += p.T @ do[r]
        dp = do[r] @ v.T
        ds = p * (dp - D[:, None])
        dq[r] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r])
    return dq, dk, dv


def attention_backward(Q, K, V, dO, scale: float, causal: bool, heads=None, O=None):
    """dQ [B, H_q, N_q, d], dK and dV [B, H_kv, N_k, d] in fp64.  ``O`` (optional): the
    saved forward output [B, H_q, N_q, d] that D is taken from (default: the exact O).

    GQA (Attention kernel chains, "GQA loads KV once per group"): query head h reads
    KV head h // g, so the gradient of KV head hk is the sum over the g query heads
    of its group.  ``heads`` (optional): a list of (b, hk) KV heads to compute; the
    other entries stay zero (sampled checks at full size).
    """
    B, H_q, N_q, d = Q.shape
    _, H_kv, N_k, _ = K.shape
    assert H_q % H_kv == 0, "H_q must be a multiple of H_kv"
    g = H_q // H_kv
    dQ = np.zeros(Q.shape, dtype=np.float64)
    dK = np.zeros(K.shape, dtype=np.float64)
    dV = np.zeros(V.shape, dtype=np.float64)
    todo = [(b, hk) for b in range(B) for hk in range(H_kv)] if heads is None else heads
    for b, hk in todo:
        for h in range(hk * g, (hk + 1) * g):
            dq, dk, dv = attention_head_backward(Q[b, h], K[b, hk], V[b, hk], dO[b, h], scale, causal,
                                                 o=None if O is None else O[b, h])
            dQ[b, h] = dq
            dK[b, hk] += dk
            dV[b, hk] += dv
    return dQ, dK, dV


# ---------------------------------------------------------------------------
# The streamed recurrences of the derivation (used by the pin tests only)
# ---------------------------------------------------------------------------

def online_softmax_fa2(x: np.ndarray, V: np.ndarray, blocks):
    """One query row streamed block by block with the unnormalized accumulator.

    Carries (Flash Attention 1 page, "Derivation"): running max m, running
    denominator d' (called l on the other pages), unnormalized numerator u;
    starting values m = -inf, d' = 0, u = 0.  Per block (the tiled version):
    m_new = max(m, max of the block); d' <- d' e^{m - m_new} + sum e^{x - m_new};
    u <- u e^{m - m_new} + sum e^{x - m_new} V[j,:].  One division at the end
    (Attention kernel chains, "The online softmax on numbers": dividing once
    at the end is the FlashAttention-2 change).

    ``blocks`` is a list of index arrays partitioning the keys, in stream order.
    Returns (o = u / d', lse = m + ln d', history) where history holds
    (m, d', alpha) after each block.
    """
    x = np.asarray(x, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    m = NEG_INF
    dp = 0.0
    u = np.zeros(V.shape[1])
    history = []
    for blk in blocks:
        blk = np.asarray(blk, dtype=np.int64)
        if blk.size == 0:
            continue
        m_local = float(np.max(x[blk]))
        m_new = max(m, m_local)
        alpha = 0.0 if m == NEG_INF else float(np.exp(m - m_new))
        w = np.exp(x[blk] - m_new)
        dp = dp * alpha + float(np.sum(w))
        u = u * alpha + w @ V[blk]
        m = m_new
        history.append((m, dp, alpha))
    return u / dp, m + np.log(dp), history


def online_softmax_fa1(x: np.ndarray, V: np.ndarray, blocks):
    """The same row with the normalized output o' carried and a division every
    block (Flash Attention 1 page, the tiled recurrence): o' <- o' d'_old e^{m - m_new} / d'_new
    + sum (e^{x - m_new} / d'_new) V[j,:].  Returns (o', lse)."""
    x = np.asarray(x, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    m = NEG_INF
    dp = 0.0
    o = np.zeros(V.shape[1])
    for blk in blocks:
        blk = np.asarray(blk, dtype=np.int64)
        if blk.size == 0:
            continue
        m_new = max(m, float(np.max(x[blk])))
        corr = 0.0 if m == NEG_INF else float(np.exp(m - m_new))
        w = np.exp(x[blk] - m_new)
        dp_new = dp * corr + float(np.sum(w))
        o = o * (dp * corr / dp_new) + (w / dp_new) @ V[blk]
        m, dp = m_new, dp_new
    return o, m + np.log(dp)
