"""fa_fwd_paged (chunked prefill over a paged KV cache) on the GPU against the fp64
oracle, through the C ABI.

Small cases compare every element: chunks that sit at the end of a longer cache (the
bottom-right mask), N_q = N_k, N_q > N_k (rows that see no key), GQA, page sizes that
do not divide the key tile or the sequence, a page size of one and pages larger than a
tile.  The full-size chunk compares sampled rows of every query block with the oracle.
Both also compare with fa_fwd on the same keys gathered into a contiguous cache: at d = 64
the two launches tile the keys alike and run the same arithmetic in the same order, so
the results are bit-identical; at d = 128 the contiguous kernel takes 128-key tiles and
the paged one 64-key tiles, so the two agree only to rounding (both are checked against
the oracle above)."""

import numpy as np
import pytest
import torch

import oracle.fa_oracle as orc
from online_softmax_07_amd import fa, workloads
from parity import check_lse, check_o

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def host(t):
    return t.float().numpy()


def run_paged(q, k, v, bt, n_k, causal, scale, out_dtype=torch.bfloat16):
    o = torch.full(q.shape, float("nan"), dtype=out_dtype, device=DEV)   # NaN canary
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd_paged(q, k, v, bt, n_k, o, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def gathered(pool, bt, n_k):
    """[num_pages, ps, H_kv, d] pool -> contiguous [B, H_kv, n_k, d] through the table
    (torch indexing: plumbing for the bit-identity check, not a reference)."""
    ps = pool.shape[1]
    rows = pool[bt.long()].reshape(bt.shape[0], bt.shape[1] * ps, pool.shape[2], pool.shape[3])
    return rows[:, :n_k].permute(0, 2, 1, 3).contiguous()


def run_contiguous(q, k, v, causal, scale, out_dtype=torch.bfloat16):
    o = torch.empty(q.shape, dtype=out_dtype, device=DEV)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    fa.fa_fwd(q, k, v, o, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def same_bits(a, b, what):
    assert torch.equal(a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                       b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)), what


def agrees_with_contiguous(o, lse, oc, lc, d, what):
    """Bit-identical at d = 64 (same tiling); at d = 128, equal to rounding: bf16 O within two
    bf16 ulps of the larger value plus 1e-3, LSE within 1e-4."""
    if d == 64:
        same_bits(o, oc, what + ": O")
        same_bits(lse, lc, what + ": LSE")
        return
    a, b = o.float(), oc.float()
    tol = 2.0 ** -6 * torch.maximum(a.abs(), b.abs()) + 1e-3
    assert bool(((a - b).abs() <= tol).all()), what + ": O"
    fin = torch.isfinite(lc)
    assert torch.equal(torch.isfinite(lse), fin), what + ": LSE -inf pattern"
    if bool(fin.any()):
        assert float((lse[fin] - lc[fin]).abs().max()) <= 1e-4, what + ": LSE"


# B, H_q, H_kv, N_q, N_k, d, causal, page_size
SMALL = [
    (1, 2, 1, 128, 300, 128, True, 16),      # a chunk at the end of the cache
    (2, 4, 2, 100, 333, 64, True, 5),        # odd page size, ragged chunk and cache
    (1, 2, 2, 77, 77, 128, True, 16),        # the whole sequence is the chunk
    (2, 8, 2, 200, 1000, 128, False, 64),    # no mask
    (1, 2, 1, 300, 200, 64, True, 7),        # N_q > N_k: the first 100 rows see no key
    (1, 4, 1, 1, 513, 128, True, 1),         # one query, one-token pages
    (3, 4, 1, 129, 4100, 128, True, 32),     # many tiles, GQA group of 4
    (1, 2, 1, 64, 700, 64, True, 256),       # pages larger than a tile
    (1, 2, 1, 257, 257, 64, False, 3),
    (2, 8, 1, 150, 900, 64, True, 16),       # GQA group of 8 at d = 64
    (1, 4, 4, 300, 2000, 128, False, 48),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_paged_prefill_small(case):
    B, Hq, Hkv, Nq, Nk, d, causal, ps = case
    w = workloads.decode(B, Hq, Hkv, Nq, Nk, d, seed=2000 + sum(case), causal=causal, page_size=ps,
                         num_pages=B * (-(-Nk // ps)) + 5)
    say("paged prefill", case)
    bt = w.block_table.numpy()
    O, L = orc.decode(host(w.q), host(w.k), host(w.v), w.scale, causal, block_table=bt, page_size=ps, n_k=Nk)
    q, k, v, btd = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), w.block_table.to(DEV)
    o, lse = run_paged(q, k, v, btd, Nk, causal, w.scale)
    check_o(o, O, "bf16")
    check_lse(lse, L)
    o32, lse32 = run_paged(q, k, v, btd, Nk, causal, w.scale, torch.float32)
    check_o(o32, O, "fp32out")
    check_lse(lse32, L)
    kc, vc = gathered(k, btd, Nk), gathered(v, btd, Nk)
    oc, lc = run_contiguous(q, kc, vc, causal, w.scale)
    agrees_with_contiguous(o, lse, oc, lc, d, "paged vs fa_fwd on the gathered cache")


def test_paged_prefill_lse_optional():
    w = workloads.decode(1, 2, 1, 96, 400, 128, seed=2500, causal=True, page_size=16)
    q, k, v, bt = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), w.block_table.to(DEV)
    o1, _ = run_paged(q, k, v, bt, 400, True, w.scale)
    o2 = torch.empty_like(o1)
    fa.fa_fwd_paged(q, k, v, bt, 400, o2, None, causal=True, scale=w.scale, want_lse=False)
    torch.cuda.synchronize()
    same_bits(o1, o2, "O depends on whether LSE is written")


def test_chunked_prefill_full_size():
    """The bench workload: 2048-token chunks over 8192 positions, 32/8 heads, 16-token
    pages; every query block sampled, plus agreement with the contiguous kernel on every
    row."""
    w = workloads.chunked_prefill_paged()
    s = w.shape
    say(w.name)
    q, k, v, bt = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), w.block_table.to(DEV)
    o, lse = run_paged(q, k, v, bt, w.n_k, w.causal, w.scale)
    N = s["T"]
    rows = sorted({0, 1, N - 1, N - 2} | {qb * 128 + (37 * qb + 11) % 128 for qb in range(N // 128)})
    rows = np.array(rows)
    say("oracle on", len(rows), "rows")
    O, L = orc.decode(host(w.q), host(w.k), host(w.v), w.scale, w.causal, block_table=w.block_table.numpy(),
                      page_size=w.page_size, n_k=w.n_k, rows=rows)
    ri = torch.as_tensor(rows, device=DEV)
    check_o(o[:, :, ri], O, "bf16")
    check_lse(lse[:, :, ri], L)
    kc, vc = gathered(k, bt, w.n_k), gathered(v, bt, w.n_k)
    del k, v
    oc, lc = run_contiguous(q, kc, vc, w.causal, w.scale)
    agrees_with_contiguous(o, lse, oc, lc, s["d"], "paged vs fa_fwd on the gathered cache")
