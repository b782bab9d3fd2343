"""Checks that pin the fp64 oracle to what the pages and the mathematics fix.

Each ``check_*`` takes the oracle module and raises AssertionError on a mismatch,
so the same checks run against the real oracle (test_oracle_pins.py) and against
oracles with a planted mistake (test_oracle_mutants.py), where at least one of
them must fail.  Expected values come from the pages (tests/golden/*.json, each
with its citation), from closed forms, from invariants, or from independent
library routines (torch's scaled_dot_product_attention, scipy's softmax and
logsumexp) -- never from the oracle itself or from the HIP path.
"""

from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import scipy.special
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def printed_close(value, printed, decimals):
    """``value`` agrees with a number printed to ``decimals`` places (half a unit of the last place,
    plus a hair for the pages' own intermediate rounding)."""
    return abs(float(value) - float(printed)) <= 0.5 * 10.0 ** (-decimals) + 1e-3 * 10.0 ** (-decimals) * 2


# --- the pages' worked numbers -------------------------------------------------

def check_softmax_123(orc):
    g = golden("softmax_1_2_3.json")
    p = orc.safe_softmax(np.array(g["scores"]))
    for a, b in zip(p, g["softmax"]):
        assert printed_close(a, b, g["printed_decimals"]), (p, g["softmax"])
    # The same numbers through the full attention definition: one query (1,0,0)
    # against key rows (1,0,0),(2,0,0),(3,0,0), scale 1, V = I, so O is the softmax row.
    q = np.array([[1.0, 0.0, 0.0]])
    K = np.array([[1.0, 0, 0], [2.0, 0, 0], [3.0, 0, 0]])
    O, lse = orc.attention_head(q, K, np.eye(3), 1.0, False)
    for a, b in zip(O[0], g["softmax"]):
        assert printed_close(a, b, g["printed_decimals"]), O
    assert abs(lse[0] - math.log(math.e + math.e ** 2 + math.e ** 3)) < 1e-12


def check_online_numbers(orc):
    g = golden("online_softmax_on_numbers.json")
    dec = g["printed_decimals"]
    x = np.array(g["blocks"][0] + g["blocks"][1])
    blocks = [np.arange(len(g["blocks"][0])), np.arange(len(g["blocks"][0]), len(x))]
    o, lse, hist = orc.online_softmax_fa2(x, np.eye(len(x)), blocks)
    (m1, l1, _), (m2, l2, a2) = hist
    assert m1 == g["after_block_1"]["m"] and printed_close(l1, g["after_block_1"]["l"], dec), hist
    assert printed_close(a2, g["alpha_block_2"], dec), hist
    assert m2 == g["after_block_2"]["m"] and printed_close(l2, g["after_block_2"]["l"], dec), hist
    assert printed_close(o[-1], g["weight_of_score_3"], dec), o
    o1, lse1 = orc.online_softmax_fa1(x, np.eye(len(x)), blocks)
    assert printed_close(o1[-1], g["weight_of_score_3"], dec), o1


def check_lse_merge_numbers(orc):
    g = golden("lse_merge_two_workers.json")
    dec = g["printed_decimals"]
    w1, w2 = g["workers"]
    l1 = orc.logsumexp(np.array(w1))
    l2 = orc.logsumexp(np.array(w2))
    assert printed_close(l1, g["lse_parts"][0], dec) and printed_close(l2, g["lse_parts"][1], dec)
    # Partials over V = I_3: worker 1 holds keys 0,1, worker 2 key 2.
    q = np.array([[1.0, 0.0, 0.0]])
    K = np.array([[1.0, 0, 0], [2.0, 0, 0], [3.0, 0, 0]])
    V = np.eye(3)
    Q4 = q[None, None]
    K4, V4 = K[None, None], V[None, None]
    Op, Lp = orc.split_partials(Q4, K4, V4, 1.0, False, [(0, 2), (2, 3)])
    assert printed_close(Lp[0, 0, 0, 0], g["lse_parts"][0], dec)
    assert printed_close(Lp[1, 0, 0, 0], g["lse_parts"][1], dec)
    O, lse = orc.lse_merge(Op, Lp)
    assert printed_close(lse[0, 0, 0], g["merged_lse"], dec), lse
    weights = np.exp(Lp[:, 0, 0, 0] - lse[0, 0, 0])
    for a, b in zip(weights, g["weights"]):
        assert printed_close(a, b, dec), weights
    # "0.335 is 0.090 + 0.245": the first worker's share is the softmax mass of its keys.
    sm = golden("softmax_1_2_3.json")["softmax"]
    assert abs(weights[0] - sum(sm[i] for i in g["first_worker_share_equals_softmax_sum_of"])) < 2e-3
    # and the merged output is the plain softmax row
    assert np.allclose(O[0, 0, 0], scipy.special.softmax([1.0, 2.0, 3.0]), atol=1e-14)


def check_decode_mask(orc):
    g = golden("causal_decode_step.json")
    T, S = g["T"], g["S"]
    lo, hi = g["bottom_right_visible_keys"]
    vis = orc.visible_mask(T, S, True)
    assert vis.shape == (T, S)
    assert vis[0, lo] and vis[0, hi] and vis[0].sum() == hi - lo + 1
    assert orc.is_visible(0, hi, T, S, True) and not orc.is_visible(0, S, T, S, True)
    # On data: a decode step with the causal flag equals the unmasked result, and
    # differs from what a top-left mask would give (attention to key 0 only: O = V[0]).
    rng = np.random.default_rng(7)
    Q = rng.standard_normal((1, 2, T, 16))
    K = rng.standard_normal((1, 2, S, 16))
    V = rng.standard_normal((1, 2, S, 16))
    Oc, Lc = orc.attention(Q, K, V, 0.25, True)
    On, Ln = orc.attention(Q, K, V, 0.25, False)
    assert np.allclose(Oc, On, atol=1e-13) and np.allclose(Lc, Ln, atol=1e-13)
    assert not np.allclose(Oc[0, :, 0], V[0, :, 0], atol=1e-3)


# --- closed forms ----------------------------------------------------------------

def check_mask_counts_closed_form(orc):
    """Q = 0 makes every visible score 0, so LSE[i] = ln |visible(i)| = ln(i + 1 + N_k - N_q)
    exactly and O[i] is the plain mean of the visible V rows (rows with no visible key:
    O = 0, LSE = -inf)."""
    rng = np.random.default_rng(11)
    for n_q, n_k in [(5, 9), (9, 9), (12, 7), (1, 6), (4, 1)]:
        Q = np.zeros((1, 1, n_q, 8))
        K = rng.standard_normal((1, 1, n_k, 8))
        V = rng.standard_normal((1, 1, n_k, 8))
        O, L = orc.attention(Q, K, V, 0.5, True)
        for i in range(n_q):
            cnt = min(n_k, i + 1 + n_k - n_q)
            if cnt <= 0:
                assert L[0, 0, i] == -np.inf and np.all(O[0, 0, i] == 0)
            else:
                assert abs(L[0, 0, i] - math.log(cnt)) < 1e-12, (n_q, n_k, i, L[0, 0, i])
                assert np.allclose(O[0, 0, i], V[0, 0, :cnt].mean(axis=0), atol=1e-12)
        O, L = orc.attention(Q, K, V, 0.5, False)
        assert np.allclose(L, math.log(n_k), atol=1e-12)


def check_v_identity_gives_probabilities(orc):
    """With V = I (N_k = d) the output row is the probability row itself; compared with
    scipy's softmax of the masked scores."""
    rng = np.random.default_rng(12)
    n_q, n_k = 6, 10
    q = rng.standard_normal((n_q, 4))
    k = rng.standard_normal((n_k, 4))
    O, _ = orc.attention_head(q, k, np.eye(n_k), 0.7, True)
    s = 0.7 * np.einsum("id,jd->ij", q, k)
    for i in range(n_q):
        vis = i + (n_k - n_q) + 1
        ref = np.zeros(n_k)
        ref[:vis] = scipy.special.softmax(s[i, :vis])
        assert np.allclose(O[i], ref, atol=1e-14), (i, O[i], ref)


def check_v_ones(orc):
    rng = np.random.default_rng(13)
    Q = rng.standard_normal((2, 3, 7, 8))
    K = rng.standard_normal((2, 3, 11, 8)) * 4
    O, _ = orc.attention(Q, K, np.ones((2, 3, 11, 8)), 0.3, True)
    assert np.allclose(O, 1.0, atol=1e-13)


# --- independent library routine -------------------------------------------------

def _sdpa_reference(Q, K, V, scale, causal):
    """torch's scaled_dot_product_attention in fp64 on the CPU with an explicit
    bottom-right boolean mask (never is_causal=True, which aligns top-left), plus
    LSE from torch.logsumexp.  GQA is expanded with repeat_interleave."""
    Qt = torch.from_numpy(Q)
    g = Q.shape[1] // K.shape[1]
    Kt = torch.from_numpy(K).repeat_interleave(g, dim=1)
    Vt = torch.from_numpy(V).repeat_interleave(g, dim=1)
    n_q, n_k = Q.shape[2], K.shape[2]
    i = torch.arange(n_q)[:, None]
    j = torch.arange(n_k)[None, :]
    mask = (j <= i + (n_k - n_q)) if causal else torch.ones(n_q, n_k, dtype=torch.bool)
    O = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, attn_mask=mask, scale=scale)
    S = torch.matmul(Qt, Kt.transpose(-1, -2).contiguous()) * scale
    S = S.masked_fill(~mask, float("-inf"))
    L = torch.logsumexp(S, dim=-1)
    return O.numpy(), L.numpy()


def check_vs_sdpa(orc):
    rng = np.random.default_rng(14)
    for (B, Hq, Hkv, n_q, n_k, d, causal) in [(2, 4, 2, 37, 53, 16, True), (1, 3, 3, 40, 40, 32, False),
                                              (1, 8, 2, 5, 70, 8, True)]:
        Q = rng.standard_normal((B, Hq, n_q, d))
        K = rng.standard_normal((B, Hkv, n_k, d))
        V = rng.standard_normal((B, Hkv, n_k, d))
        O, L = orc.attention(Q, K, V, 0.37, causal)
        Or, Lr = _sdpa_reference(Q, K, V, 0.37, causal)
        assert np.allclose(O, Or, atol=1e-12), np.abs(O - Or).max()
        assert np.allclose(L, Lr, atol=1e-12), np.abs(L - Lr).max()


# --- invariants -----------------------------------------------------------------

def check_gqa_is_mha_on_repeated_kv(orc):
    rng = np.random.default_rng(15)
    Q = rng.standard_normal((2, 8, 9, 16))
    K = rng.standard_normal((2, 2, 13, 16))
    V = rng.standard_normal((2, 2, 13, 16))
    O, L = orc.attention(Q, K, V, 0.25, True)
    Km = np.repeat(K, 4, axis=1)     # head h of the MHA copy is KV head h // 4
    Vm = np.repeat(V, 4, axis=1)
    Om, Lm = orc.attention(Q, Km, Vm, 0.25, True)
    assert np.allclose(O, Om, atol=1e-13) and np.allclose(L, Lm, atol=1e-13)
    # and each head-group slice equals single-KV-head attention computed on its own
    for h in range(8):
        Oh, _ = orc.attention(Q[:, h:h + 1], K[:, h // 4:h // 4 + 1], V[:, h // 4:h // 4 + 1], 0.25, True)
        assert np.allclose(O[:, h:h + 1], Oh, atol=1e-13)


def check_paged_equals_contiguous(orc):
    """Scatter a contiguous cache into randomly permuted pages by brute force, then
    paged decode must equal contiguous decode; gather must invert the scatter."""
    rng = np.random.default_rng(16)
    B, Hq, Hkv, T, n_k, d, ps = 3, 4, 2, 2, 45, 8, 16
    pps = -(-n_k // ps)
    num_pages = B * pps + 5
    table = rng.permutation(num_pages)[: B * pps].reshape(B, pps)
    K = rng.standard_normal((B, Hkv, n_k, d))
    V = rng.standard_normal((B, Hkv, n_k, d))
    Kp = np.full((num_pages, ps, Hkv, d), np.nan)
    Vp = np.full((num_pages, ps, Hkv, d), np.nan)
    for b in range(B):
        for j in range(n_k):
            for h in range(Hkv):
                Kp[table[b, j // ps], j % ps, h] = K[b, h, j]
                Vp[table[b, j // ps], j % ps, h] = V[b, h, j]
    assert np.array_equal(orc.gather_pages(Kp, table, n_k, ps), K)
    Q = rng.standard_normal((B, Hq, T, d))
    O1, L1 = orc.decode(Q, Kp, Vp, 0.3, True, block_table=table, page_size=ps, n_k=n_k)
    O2, L2 = orc.decode(Q, K, V, 0.3, True)
    assert np.allclose(O1, O2, atol=1e-14) and np.allclose(L1, L2, atol=1e-14)


def check_merge_partition_invariance(orc):
    """Any split of the keys merges to the unsplit result: contiguous ranges, empty
    ranges, one range, a permutation of the partials, and ranges a row cannot see."""
    rng = np.random.default_rng(17)
    B, Hq, Hkv, n_q, n_k, d = 1, 4, 2, 3, 50, 8
    Q = rng.standard_normal((B, Hq, n_q, d))
    K = rng.standard_normal((B, Hkv, n_k, d)) * 2
    V = rng.standard_normal((B, Hkv, n_k, d))
    O, L = orc.attention(Q, K, V, 0.4, True)
    cases = [[(0, 50)], [(0, 10), (10, 50)], [(0, 1), (1, 2), (2, 50)],
             [(0, 16), (16, 32), (32, 48), (48, 64), (64, 64)], [(0, 0), (0, 49), (49, 50)],
             [(0, 7), (7, 13), (13, 29), (29, 31), (31, 50)]]
    for bounds in cases:
        Op, Lp = orc.split_partials(Q, K, V, 0.4, True, bounds)
        Om, Lm = orc.lse_merge(Op, Lp)
        assert np.allclose(Om, O, atol=1e-13), bounds
        assert np.allclose(Lm, L, atol=1e-13), bounds
        perm = rng.permutation(len(bounds))
        Om2, Lm2 = orc.lse_merge(Op[perm], Lp[perm])
        assert np.allclose(Om2, O, atol=1e-13) and np.allclose(Lm2, L, atol=1e-13)
    # every partial -inf: the row saw no key
    Om, Lm = orc.lse_merge(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(Om == 0) and np.all(Lm == -np.inf)


def _compositions(n):
    """Every split of 0..n-1 into consecutive non-empty blocks."""
    for cuts in itertools.product([False, True], repeat=n - 1):
        blocks, cur = [], [0]
        for i, c in enumerate(cuts, start=1):
            if c:
                blocks.append(cur)
                cur = [i]
            else:
                cur.append(i)
        blocks.append(cur)
        yield blocks


def check_online_equals_two_pass(orc):
    """Softmax and FlashAttention, "Maths": the online recurrence equals the two-pass
    softmax in exact arithmetic and differs in fp64 only by rounding (~1e-16).  Brute
    force: every block split of random rows of length 1..8, in stream order and in a
    shuffled key order, both the FA1 (normalize every block) and the FA2 (divide once)
    forms, against the two-pass definition."""
    rng = np.random.default_rng(18)
    worst = 0.0
    for n in range(1, 9):
        for trial in range(3):
            x = rng.standard_normal(n) * (1 + 4 * trial)
            V = rng.standard_normal((n, 5))
            o_ref = orc.safe_softmax(x) @ V
            lse_ref = scipy.special.logsumexp(x)
            order = rng.permutation(n)
            for blocks in _compositions(n):
                for key_order in (np.arange(n), order):
                    bl = [key_order[b] for b in blocks]
                    o2, lse2, _ = orc.online_softmax_fa2(x, V, bl)
                    o1, lse1 = orc.online_softmax_fa1(x, V, bl)
                    worst = max(worst, np.abs(o2 - o_ref).max(), np.abs(o1 - o_ref).max(),
                                abs(lse2 - lse_ref), abs(lse1 - lse_ref))
    assert worst <= 1e-14, worst


# --- the backward pass -----------------------------------------------------------

def _sdpa_grads(Q, K, V, dO, scale, causal):
    """dQ, dK, dV by torch autograd through scaled_dot_product_attention in fp64 on the
    CPU (explicit bottom-right mask; GQA by repeat_interleave, whose backward sums the
    group)."""
    Qt, Kt, Vt = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (Q, K, V))
    g = Q.shape[1] // K.shape[1]
    n_q, n_k = Q.shape[2], K.shape[2]
    i = torch.arange(n_q)[:, None]
    j = torch.arange(n_k)[None, :]
    mask = (j <= i + (n_k - n_q)) if causal else torch.ones(n_q, n_k, dtype=torch.bool)
    O = torch.nn.functional.scaled_dot_product_attention(
        Qt, Kt.repeat_interleave(g, dim=1), Vt.repeat_interleave(g, dim=1), attn_mask=mask, scale=scale)
    (O * torch.from_numpy(dO)).sum().backward()
    return Qt.grad.numpy(), Kt.grad.numpy(), Vt.grad.numpy()


def check_backward_vs_autograd(orc):
    rng = np.random.default_rng(21)
    for (B, Hq, Hkv, n_q, n_k, d, causal) in [(2, 4, 2, 37, 53, 16, True), (1, 3, 3, 40, 40, 32, False),
                                              (1, 8, 2, 5, 70, 8, True), (1, 2, 1, 33, 33, 8, True)]:
        Q, dO = rng.standard_normal((B, Hq, n_q, d)), rng.standard_normal((B, Hq, n_q, d))
        K, V = rng.standard_normal((B, Hkv, n_k, d)), rng.standard_normal((B, Hkv, n_k, d))
        got = orc.attention_backward(Q, K, V, dO, 0.41, causal)
        ref = _sdpa_grads(Q, K, V, dO, 0.41, causal)
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            assert a.shape == b.shape and np.allclose(a, b, atol=1e-12), (name, np.abs(a - b).max())


def check_backward_finite_differences(orc):
    """Central differences of L = sum(O * dO), with O from torch's attention (not the
    oracle), against every gradient entry: tiny causal GQA case with N_q < N_k."""
    rng = np.random.default_rng(22)
    B, Hq, Hkv, n_q, n_k, d, scale = 1, 2, 1, 4, 6, 3, 0.7
    Q, dO = rng.standard_normal((B, Hq, n_q, d)), rng.standard_normal((B, Hq, n_q, d))
    K, V = rng.standard_normal((B, Hkv, n_k, d)), rng.standard_normal((B, Hkv, n_k, d))

    def loss(Q_, K_, V_):
        return float(np.sum(_sdpa_reference(Q_, K_, V_, scale, True)[0] * dO))

    got = orc.attention_backward(Q, K, V, dO, scale, True)
    h = 1e-5
    for which, (X, G) in enumerate(zip((Q, K, V), got)):
        assert G.shape == X.shape
        for idx in itertools.product(*(range(n) for n in X.shape)):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args_p = [Q, K, V]
            args_m = [Q, K, V]
            args_p[which], args_m[which] = Xp, Xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - G[idx]) <= 1e-7, ("dQ dK dV".split()[which], idx, fd, G[idx])


def check_backward_closed_forms(orc):
    rng = np.random.default_rng(23)
    # one key: P = 1, so dV = sum of dO over the rows, and dQ = dK = 0
    Q, dO = rng.standard_normal((1, 1, 7, 4)), rng.standard_normal((1, 1, 7, 4))
    K, V = rng.standard_normal((1, 1, 1, 4)), rng.standard_normal((1, 1, 1, 4))
    dQ, dK, dV = orc.attention_backward(Q, K, V, dO, 0.5, False)
    assert np.allclose(dQ, 0, atol=1e-14) and np.allclose(dK, 0, atol=1e-14)
    assert np.allclose(dV[0, 0, 0], dO[0, 0].sum(axis=0), atol=1e-13)
    # Q = 0: P is uniform over the visible keys, dV_j = sum over rows i that see j of dO_i / n_i
    n_q, n_k = 5, 8
    dO = rng.standard_normal((1, 1, n_q, 3))
    K, V = rng.standard_normal((1, 1, n_k, 3)), rng.standard_normal((1, 1, n_k, 3))
    _, _, dV = orc.attention_backward(np.zeros((1, 1, n_q, 3)), K, V, dO, 1.0, True)
    want = np.zeros((n_k, 3))
    for i in range(n_q):
        seen = i + (n_k - n_q) + 1
        for j in range(seen):
            want[j] += dO[0, 0, i] / seen
    assert np.allclose(dV[0, 0], want, atol=1e-14)
    # adding one vector to every key leaves each softmax row unchanged: sum_j dK_j = 0
    Q, dO = rng.standard_normal((2, 4, 9, 5)), rng.standard_normal((2, 4, 9, 5))
    K, V = rng.standard_normal((2, 2, 12, 5)), rng.standard_normal((2, 2, 12, 5))
    _, dK, _ = orc.attention_backward(Q, K, V, dO, 0.3, True)
    assert np.allclose(dK.sum(axis=2), 0, atol=1e-12)
    # rows that see no key (causal, N_q > N_k) get dQ = 0 and add nothing to dK, dV
    Q, dO = rng.standard_normal((1, 2, 6, 4)), rng.standard_normal((1, 2, 6, 4))
    K, V = rng.standard_normal((1, 1, 3, 4)), rng.standard_normal((1, 1, 3, 4))
    dQ, dK, dV = orc.attention_backward(Q, K, V, dO, 0.6, True)
    dQ2, dK2, dV2 = orc.attention_backward(Q[:, :, 3:], K, V, dO[:, :, 3:], 0.6, True)
    assert np.allclose(dQ[:, :, :3], 0, atol=1e-15)
    assert np.allclose(dQ[:, :, 3:], dQ2, atol=1e-14)
    assert np.allclose(dK, dK2, atol=1e-14) and np.allclose(dV, dV2, atol=1e-14)


def check_backward_saved_state(orc):
    """The page's recipe: P rebuilt as exp(S - LSE) from the forward's LSE is the softmax,
    and D = rowsum(dO * O) equals sum_j P_ij dP_ij; the gradients built from those saved
    values equal the oracle's."""
    rng = np.random.default_rng(24)
    n_q, n_k, d, scale = 11, 17, 6, 0.45
    q, k, v, do = (rng.standard_normal(s) for s in ((n_q, d), (n_k, d), (n_k, d), (n_q, d)))
    O, lse = orc.attention_head(q, k, v, scale, True)
    vis = np.array([[j <= i + (n_k - n_q) for j in range(n_k)] for i in range(n_q)])
    S = np.where(vis, scale * (q @ k.T), -np.inf)
    P = np.exp(S - lse[:, None])
    assert np.allclose(P.sum(axis=1), 1.0, atol=1e-14)
    D = np.sum(do * O, axis=1)
    dP = do @ v.T
    assert np.allclose(D, np.sum(P * dP, axis=1), atol=1e-12)
    dS = P * (dP - D[:, None])
    dq, dk, dv = orc.attention_head_backward(q, k, v, do, scale, True)
    assert np.allclose(dq, scale * dS @ k, atol=1e-12)
    assert np.allclose(dk, scale * dS.T @ q, atol=1e-12)
    assert np.allclose(dv, P.T @ do, atol=1e-12)
    # D from a saved O that is off by dO_i * delta: dV is unchanged, D moves by
    # delta_i |dO_i|^2, and dQ_i moves by -scale * delta_i |dO_i|^2 * (P K)_i
    delta = rng.standard_normal(n_q) * 1e-3
    o_saved = O + delta[:, None] * do
    dq2, dk2, dv2 = orc.attention_head_backward(q, k, v, do, scale, True, o=o_saved)
    dD = delta * np.sum(do * do, axis=1)
    assert np.allclose(dv2, dv, atol=1e-14)
    assert np.allclose(dq2 - dq, -scale * dD[:, None] * (P @ k), atol=1e-12)
    assert np.allclose(dk2 - dk, -scale * (P * dD[:, None]).T @ q, atol=1e-12)
    dq3, dk3, dv3 = orc.attention_head_backward(q, k, v, do, scale, True, o=O)
    assert np.allclose(dq3, dq, atol=1e-13) and np.allclose(dk3, dk, atol=1e-13)


ALL_CHECKS = [
    check_softmax_123, check_online_numbers, check_lse_merge_numbers, check_decode_mask,
    check_mask_counts_closed_form, check_v_identity_gives_probabilities, check_v_ones,
    check_vs_sdpa, check_gqa_is_mha_on_repeated_kv, check_paged_equals_contiguous,
    check_merge_partition_invariance, check_online_equals_two_pass,
    check_backward_vs_autograd, check_backward_finite_differences, check_backward_closed_forms,
    check_backward_saved_state,
]
