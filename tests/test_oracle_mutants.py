"""Plausible mistakes planted in the oracle (on the CPU) must each fail at least
one pin: this shows the pins constrain every step of the oracle, not only the
paths the worked examples happen to touch."""

import numpy as np
import pytest

import oracle.fa_oracle as orc
import pins

real_attention_head = orc.attention_head
real_visible_mask = orc.visible_mask
real_gather_pages = orc.gather_pages
real_lse_merge = orc.lse_merge
real_online_fa2 = orc.online_softmax_fa2
real_head_backward = orc.attention_head_backward


def _head_backward_variant(kind):
    """attention_head_backward with one planted mistake of the given kind."""
    def mutant(q, k, v, do, scale, causal, o=None, row_chunk=512):
        q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
        n_q, n_k = q.shape[0], k.shape[0]
        x = scale * (q @ k.T)
        x = np.where(orc.visible_mask(n_q, n_k, causal), x, -np.inf)
        m = np.max(x, axis=1, keepdims=True)
        e = np.exp(x - np.where(np.isfinite(m), m, 0.0))
        l = np.sum(e, axis=1, keepdims=True)
        p = np.divide(e, l, out=np.zeros_like(e), where=l > 0)
        o = p @ v if (o is None or kind == "ignores_saved_o") else np.asarray(o, dtype=np.float64)
        D = np.sum(do * o, axis=1)
        dp = do @ v.T
        ds = {"no_D": p * dp, "sign": p * (D[:, None] - dp)}.get(kind, p * (dp - D[:, None]))
        dq = (ds @ k) if kind == "dq_no_scale" else scale * (ds @ k)
        dk = scale * (ds.T @ (do if kind == "dk_wrong_operand" else q))
        dv = (ds.T @ do) if kind == "dv_uses_ds" else p.T @ do
        return dq, dk, dv
    mutant.__doc__ = {"no_D": "backward: dS = P * dP (D dropped)",
                      "sign": "backward: dS = P * (D - dP) (sign flipped)",
                      "dq_no_scale": "backward: dQ without the scale",
                      "dk_wrong_operand": "backward: dK = scale dS^T dO instead of dS^T Q",
                      "dv_uses_ds": "backward: dV = dS^T dO instead of P^T dO",
                      "ignores_saved_o": "backward: D from the recomputed O, not the saved O passed in"}[kind]
    return mutant


def backward_gqa_last_head(Q, K, V, dO, scale, causal, heads=None, O=None):
    """backward GQA: dK/dV of a KV head taken from the last head of its group, not the sum"""
    B, H_q = Q.shape[:2]
    H_kv = K.shape[1]
    g = H_q // H_kv
    dQ, dK, dV = np.zeros(Q.shape), np.zeros(K.shape), np.zeros(V.shape)
    for b in range(B):
        for h in range(H_q):
            dq, dk, dv = real_head_backward(Q[b, h], K[b, h // g], V[b, h // g], dO[b, h], scale, causal)
            dQ[b, h], dK[b, h // g], dV[b, h // g] = dq, dk, dv
    return dQ, dK, dV


def mask_strict(n_q, n_k, causal, rows=None):
    """off by one: j < i + (N_k - N_q)"""
    i = (np.arange(n_q) if rows is None else np.asarray(rows))[:, None]
    j = np.arange(n_k)[None, :]
    if not causal:
        return np.ones((i.shape[0], n_k), dtype=bool)
    return j < i + (n_k - n_q)


def mask_top_left(n_q, n_k, causal, rows=None):
    """top-left alignment: j <= i"""
    i = (np.arange(n_q) if rows is None else np.asarray(rows))[:, None]
    j = np.arange(n_k)[None, :]
    if not causal:
        return np.ones((i.shape[0], n_k), dtype=bool)
    return j <= i


def head_no_scale(q, k, v, scale, causal, rows=None, row_chunk=512):
    """scale dropped"""
    return real_attention_head(q, k, v, 1.0, causal, rows=rows, row_chunk=row_chunk)


def head_lse_log2(q, k, v, scale, causal, rows=None, row_chunk=512):
    """LSE in base 2 instead of the natural log"""
    o, lse = real_attention_head(q, k, v, scale, causal, rows=rows, row_chunk=row_chunk)
    m = np.max(np.where(orc.visible_mask(q.shape[0], k.shape[0], causal, rows=rows),
                        scale * (np.asarray(q, float)[rows if rows is not None else slice(None)] @ np.asarray(k, float).T),
                        -np.inf), axis=1)
    return o, m + (lse - m) / np.log(2.0)


def head_reversed_v(q, k, v, scale, causal, rows=None, row_chunk=512):
    """P applied to V with its key axis reversed (a transposed/flipped operand)"""
    return real_attention_head(q, k, np.asarray(v)[::-1], scale, causal, rows=rows, row_chunk=row_chunk)


def attention_gqa_modulo(Q, K, V, scale, causal, rows=None):
    """GQA mapping h % H_kv instead of h // g"""
    B, H_q, N_q, d = Q.shape
    H_kv = K.shape[1]
    n = N_q if rows is None else len(rows)
    O = np.zeros((B, H_q, n, V.shape[-1]))
    L = np.zeros((B, H_q, n))
    for b in range(B):
        for h in range(H_q):
            O[b, h], L[b, h] = real_attention_head(Q[b, h], K[b, h % H_kv], V[b, h % H_kv], scale, causal, rows=rows)
    return O, L


def gather_swapped(pool, block_table, n_k, page_size):
    """page and slot swapped: pool[table[b, j % P], j // P]"""
    B = block_table.shape[0]
    _, ps, H_kv, d = pool.shape
    out = np.empty((B, H_kv, n_k, d))
    for b in range(B):
        for j in range(n_k):
            out[b, :, j] = pool[block_table[b, j % ps] if j % ps < block_table.shape[1] else 0, min(j // ps, ps - 1)]
    return out


def merge_unnormalized(O_parts, lse_parts):
    """weights e^{lse_s - m*} without dividing by their sum"""
    m = np.max(lse_parts, axis=0)
    O, lse = real_lse_merge(O_parts, lse_parts)
    w = np.exp(lse_parts - np.where(np.isfinite(m), m, 0.0)[None])
    return np.sum(w[..., None] * O_parts, axis=0), lse


def online_no_rescale(x, V, blocks):
    """the accumulator is not rescaled by alpha when the max rises"""
    x = np.asarray(x, float)
    V = np.asarray(V, float)
    m, dp, u, hist = -np.inf, 0.0, np.zeros(V.shape[1]), []
    for blk in blocks:
        blk = np.asarray(blk)
        if blk.size == 0:
            continue
        m_new = max(m, float(np.max(x[blk])))
        alpha = 0.0 if m == -np.inf else float(np.exp(m - m_new))
        w = np.exp(x[blk] - m_new)
        dp = dp * alpha + w.sum()
        u = u + w @ V[blk]
        m = m_new
        hist.append((m, dp, alpha))
    return u / dp, m + np.log(dp), hist


MUTANTS = [
    ("visible_mask", mask_strict),
    ("visible_mask", mask_top_left),
    ("attention_head", head_no_scale),
    ("attention_head", head_lse_log2),
    ("attention_head", head_reversed_v),
    ("attention", attention_gqa_modulo),
    ("gather_pages", gather_swapped),
    ("lse_merge", merge_unnormalized),
    ("online_softmax_fa2", online_no_rescale),
    ("attention_head_backward", _head_backward_variant("no_D")),
    ("attention_head_backward", _head_backward_variant("sign")),
    ("attention_head_backward", _head_backward_variant("dq_no_scale")),
    ("attention_head_backward", _head_backward_variant("dk_wrong_operand")),
    ("attention_head_backward", _head_backward_variant("dv_uses_ds")),
    ("attention_head_backward", _head_backward_variant("ignores_saved_o")),
    ("attention_backward", backward_gqa_last_head),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=lambda m: m if isinstance(m, str) else m.__doc__.split(":")[0][:40])
def test_planted_mistake_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(orc, name, mutant)
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, IndexError, ValueError):
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake in {name}: {mutant.__doc__}"
