"""A seeded sweep of shapes for every entry point against the fp64 oracle, through the C ABI.

Sizes are drawn from lengths that straddle the tile boundaries (the forward's 64- and 128-key
tiles and 256-row blocks, the decode's 32-key chunks and 16-row chunks, the backward's 64-row
steps and 128-key blocks), with GQA groups of 1 to 8, both head dimensions, causal and not,
and page sizes that do and do not divide a tile.  The cases come from numpy's seeded
generator, so the list is fixed; every element of every output is compared (bf16 and fp32
outputs for the forward, LSE, all three gradients)."""

import numpy as np
import pytest
import torch

import oracle.fa_oracle as orc
from online_softmax_07_amd import fa, workloads
from parity import check_grad, check_lse, check_o

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

LENGTHS = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 191, 255, 256, 257, 300, 383, 384, 385, 511, 513]
PAGE_SIZES = [1, 3, 16, 48, 64, 100]


def say(*a):
    print(*a, flush=True)


def host(t):
    return t.float().numpy()


def draw(seed, n, lengths=LENGTHS):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        h_kv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8]))
        cases.append(dict(B=int(rng.integers(1, 3)), H_q=g * h_kv, H_kv=h_kv,
                          N_q=int(rng.choice(lengths)), N_k=int(rng.choice(lengths)),
                          d=int(rng.choice([64, 128])), causal=bool(rng.integers(0, 2)),
                          page_size=int(rng.choice(PAGE_SIZES)), T=int(rng.choice([1, 2, 3, 5, 16])),
                          ns=int(rng.choice([0, 1, 2, 3, 7, 12]))))
    return cases


def cid(c):
    return "-".join(f"{k}{int(v)}" for k, v in c.items())


FWD = draw(9001, 24)
PAGED = draw(9002, 12)
DECODE = draw(9003, 16, lengths=LENGTHS + [1000, 2047, 4100])
BWD = draw(9004, 12, lengths=[1, 31, 33, 63, 64, 65, 127, 129, 200, 257])


@pytest.mark.parametrize("c", FWD, ids=cid)
def test_sweep_fwd(c):
    say("sweep fwd", c)
    w = workloads.prefill(c["B"], c["H_q"], c["H_kv"], c["N_q"], c["N_k"], c["d"], seed=sum(c.values()) + 1,
                          causal=c["causal"])
    O, L = orc.attention(host(w.q), host(w.k), host(w.v), w.scale, w.causal)
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    for out_dtype, mode in ((torch.bfloat16, "bf16"), (torch.float32, "fp32out")):
        o = torch.full(q.shape, float("nan"), dtype=out_dtype, device=DEV)
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
        fa.fa_fwd(q, k, v, o, lse, causal=w.causal, scale=w.scale)
        torch.cuda.synchronize()
        check_o(o, O, mode)
        check_lse(lse, L)


@pytest.mark.parametrize("c", PAGED, ids=cid)
def test_sweep_fwd_paged(c):
    say("sweep fwd_paged", c)
    ps = c["page_size"]
    w = workloads.decode(c["B"], c["H_q"], c["H_kv"], c["N_q"], c["N_k"], c["d"], seed=sum(c.values()) + 2,
                         causal=c["causal"], page_size=ps, num_pages=c["B"] * (-(-c["N_k"] // ps)) + 2)
    O, L = orc.decode(host(w.q), host(w.k), host(w.v), w.scale, w.causal, block_table=w.block_table.numpy(),
                      page_size=ps, n_k=w.n_k)
    q, k, v, bt = (t.to(DEV) for t in (w.q, w.k, w.v, w.block_table))
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd_paged(q, k, v, bt, w.n_k, o, lse, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    check_o(o, O, "bf16")
    check_lse(lse, L)


@pytest.mark.parametrize("c", DECODE, ids=cid)
def test_sweep_decode(c):
    say("sweep decode", c)
    paged = c["causal"]   # half the cases paged (the draw's causal bit), all causal by the decode rule
    ps = c["page_size"] if paged else 0
    w = workloads.decode(c["B"], c["H_q"], c["H_kv"], c["T"], c["N_k"], c["d"], seed=sum(c.values()) + 3,
                         causal=True, page_size=ps,
                         num_pages=None if ps == 0 else c["B"] * (-(-c["N_k"] // ps)) + 2)
    bt_h = None if w.block_table is None else w.block_table.numpy()
    O, L = orc.decode(host(w.q), host(w.k), host(w.v), w.scale, True, block_table=bt_h,
                      page_size=ps or None, n_k=w.n_k)
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    bt = None if w.block_table is None else w.block_table.to(DEV)
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_decode_splitkv(q, k, v, o, lse, causal=True, scale=w.scale, num_splits=c["ns"], block_table=bt,
                         n_k=w.n_k)
    torch.cuda.synchronize()
    check_o(o, O, "bf16")
    check_lse(lse, L)


@pytest.mark.parametrize("c", BWD, ids=cid)
def test_sweep_bwd(c):
    say("sweep bwd", c)
    w = workloads.prefill(c["B"], c["H_q"], c["H_kv"], c["N_q"], c["N_k"], c["d"], seed=sum(c.values()) + 4,
                          causal=c["causal"])
    do = workloads.grad_output(tuple(w.q.shape), sum(c.values()) + 5)
    O, L = orc.attention(host(w.q), host(w.k), host(w.v), w.scale, w.causal)
    o_saved = torch.from_numpy(O).to(torch.float32).to(torch.bfloat16)
    dQ, dK, dV = orc.attention_backward(host(w.q), host(w.k), host(w.v), host(do), w.scale, w.causal,
                                        O=host(o_saved))
    q, k, v, g = (t.to(DEV) for t in (w.q, w.k, w.v, do))
    o = o_saved.to(DEV)
    lse = torch.from_numpy(L).to(torch.float32).to(DEV)
    dq, dk, dv = (torch.full(t.shape, float("nan"), dtype=torch.float32, device=DEV) for t in (q, k, v))
    fa.fa_bwd(q, k, v, o, g, lse, dq, dk, dv, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    check_grad(dq, dQ, "dQ", False)
    check_grad(dk, dK, "dK", False)
    check_grad(dv, dV, "dV", False)
