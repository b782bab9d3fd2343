"""Empty inputs on the GPU, through the C ABI: no key at all (N_k = 0) and no query
(N_q = 0 / T = 0 / zero rows), for every entry point.  A row that sees no key has O = 0 and
LSE = -inf (the oracle's reading for such rows); the oracle's own results for these
shapes are the reference, and NaN canaries check that every output element is written."""

import numpy as np
import pytest
import torch

import oracle.fa_oracle as orc
from online_softmax_07_amd import fa, workloads
from parity import check_lse, check_o, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def host(t):
    return t.float().numpy()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_fwd_no_keys(d, causal, dtype):
    say("fwd N_k=0", d, causal, dtype)
    w = workloads.prefill(2, 4, 2, 77, 0, d, seed=4000 + d, causal=causal, dtype=dtype)
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    o = torch.full(q.shape, float("nan"), dtype=q.dtype, device=DEV)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd(q, k, v, o, lse, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    O, L = orc.attention(host(w.q), host(w.k), host(w.v), w.scale, causal)
    assert np.all(O == 0) and np.all(np.isneginf(L))
    check_o(o, O, "fp32" if dtype == "fp32" else "bf16")
    check_lse(lse, L)


def test_fwd_no_queries():
    say("fwd N_q=0")
    w = workloads.prefill(1, 2, 1, 0, 50, 128, seed=4100, causal=True)
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    o, lse = fa.fa_fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 128) and lse.shape == (1, 2, 0)


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_paged_no_keys(d):
    say("fwd_paged N_k=0", d)
    w = workloads.decode(2, 4, 2, 33, 0, d, seed=4200 + d, causal=True, page_size=16, num_pages=3)
    assert w.block_table.shape == (2, 0)
    q, k, v, bt = (t.to(DEV) for t in (w.q, w.k, w.v, w.block_table))
    o = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd_paged(q, k, v, bt, 0, o, lse, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("ns", [1, 3, 0])
def test_decode_no_keys(paged, ns):
    say("decode N_k=0", paged, ns)
    w = workloads.decode(2, 8, 2, 3, 0, 128, seed=4300, causal=True, page_size=16 if paged else 0,
                         num_pages=2 if paged else None)
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    bt = w.block_table.to(DEV) if paged else None
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_decode_splitkv(q, k, v, o, lse, causal=True, scale=w.scale, num_splits=ns, block_table=bt, n_k=0)
    torch.cuda.synchronize()
    O, L = orc.decode(host(w.q), host(w.k), host(w.v), w.scale, True,
                      block_table=None if bt is None else w.block_table.numpy(), page_size=16 if paged else None,
                      n_k=0)
    check_o(o, O, "bf16")
    check_lse(lse, L)


def test_decode_no_queries_and_empty_merge():
    say("decode T=0, merge rows=0")
    w = workloads.decode(2, 8, 2, 0, 100, 128, seed=4400, causal=True)
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    o, lse = fa.fa_decode_splitkv(q, k, v, causal=True, scale=w.scale, num_splits=4)
    op = torch.zeros(4, 0, 128, dtype=torch.float32, device=DEV)
    lp = torch.zeros(4, 0, dtype=torch.float32, device=DEV)
    om, lm = fa.fa_lse_merge(op, lp)
    torch.cuda.synchronize()
    assert o.shape == (2, 8, 0, 128) and om.shape == (0, 128) and lm.shape == (0,)


def run_bwd_zero(B, Hq, Hkv, Nq, Nk, d, seed):
    w = workloads.prefill(B, Hq, Hkv, Nq, Nk, d, seed=seed, causal=True)
    do = workloads.grad_output(tuple(w.q.shape), seed + 1)
    O, L = orc.attention(host(w.q), host(w.k), host(w.v), w.scale, True)
    ref = orc.attention_backward(host(w.q), host(w.k), host(w.v), host(do), w.scale, True)
    q, k, v, g = (t.to(DEV) for t in (w.q, w.k, w.v, do))
    o = torch.from_numpy(O).float().to(torch.bfloat16).to(DEV)
    lse = torch.from_numpy(L).float().to(DEV)
    nan = float("nan")
    dq = torch.full(q.shape, nan, dtype=torch.float32, device=DEV)
    dk = torch.full(k.shape, nan, dtype=torch.float32, device=DEV)
    dv = torch.full(v.shape, nan, dtype=torch.float32, device=DEV)
    fa.fa_bwd(q, k, v, o, g, lse, dq, dk, dv, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    return (dq, dk, dv), ref


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_no_queries(d):
    say("bwd N_q=0", d)
    got, ref = run_bwd_zero(1, 4, 2, 0, 200, d, 4500 + d)
    assert got[0].numel() == 0
    for name, g, r in zip(("dK", "dV"), got[1:], ref[1:]):
        assert np.all(r == 0)
        assert torch.all(g == 0), name   # every key written, and written as zero


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_no_keys(d):
    say("bwd N_k=0", d)
    got, ref = run_bwd_zero(1, 4, 2, 70, 0, d, 4600 + d)
    assert got[1].numel() == 0 and got[2].numel() == 0
    assert np.all(ref[0] == 0)
    assert torch.all(got[0] == 0)
    assert np.array_equal(to_np(got[0]), ref[0])
