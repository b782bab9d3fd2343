"""fa_bwd on the GPU against the fp64 oracle, through the C ABI.

The saved forward state the backward takes (O in bf16, LSE in fp32) comes from the
oracle's forward, rounded to those types, and the oracle's backward takes D from the same
bf16 O (D = rowsum(dO * O) of the saved O, as the backward receives it).  Small cases
compare every element (ragged blocks, GQA, causal with N_q < N_k and N_q > N_k, a single
query, d = 64 and 128); the full-size prefill shape compares whole heads, sampled.  A
separate end-to-end case runs the GPU forward and then the backward on its output, as a
training step would, against the exact gradient (whole-tensor bound only: the bf16 O then
differs from the exact O, which moves D by a few bf16 ulps of dO . O).

Tolerance (from the arithmetic): the kernels multiply bf16 operands exactly and add in
fp32, but P and dS are rounded to bf16 (unit roundoff u = 2^-8) before the dV, dK and dQ
products, and D uses the bf16-rounded O.  Each gradient entry is then a sum whose terms
carry independent relative errors of at most u, so its error is about u/sqrt(3) times the
root-sum-square of its terms.  The d entries of one gradient row (one query's dQ, one key's
dK or dV) share their terms up to a factor, so the row's own root mean square sets the
scale of their errors: an entry that is small by cancellation still carries the error of
its row.  Rows differ by orders of magnitude under the causal mask (the first keys and
queries have the largest gradients), so the bound is per row:
  * ||g - r||_2 <= 2^-6 ||r||_2 over the whole tensor    (expected ~2^-9, ~5x margin)
  * |g - r| <= 2^-4 (|r| + rms_row(r)) + 2^-10 rms(r) elementwise, plus half a bf16 ulp of
    r for bf16 outputs (no entry, ragged rows and keys included, may be off by a sizeable
    fraction of its row).  The small absolute floor covers rows whose exact value is 0
    but whose terms are not (the first causal query sees one key: P = 1, dS = dP - D
    vanishes only up to the rounding of two different fp32 dot products).
"""

import numpy as np
import pytest
import torch

import oracle.fa_oracle as orc
from online_softmax_07_amd import fa, workloads
from parity import check_grad, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def host(t):
    return t.float().numpy()


def saved_state(w, O, L):
    """The oracle forward's O and LSE as a forward pass saves them: bf16 O, fp32 LSE."""
    o = torch.from_numpy(O).to(torch.float32).to(torch.bfloat16)
    lse = torch.from_numpy(L).to(torch.float32)
    return o, lse


def run_bwd(q, k, v, do, causal, scale, out_dtype, o=None, lse=None):
    if o is None:   # the GPU forward's own output, as in a training step
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
        fa.fa_fwd(q, k, v, o, lse, causal=causal, scale=scale)
    nan = float("nan")
    dq = torch.full(q.shape, nan, dtype=out_dtype, device=DEV)   # NaN canaries: every element is written
    dk = torch.full(k.shape, nan, dtype=out_dtype, device=DEV)
    dv = torch.full(v.shape, nan, dtype=out_dtype, device=DEV)
    fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


# B, H_q, H_kv, N_q, N_k, d, causal
SMALL = [
    (1, 1, 1, 128, 128, 128, False),
    (1, 2, 1, 128, 128, 128, True),
    (2, 4, 2, 100, 77, 64, True),      # N_q > N_k: the first 23 rows see no key
    (1, 2, 2, 77, 300, 128, True),     # a chunk at the end of a longer sequence
    (1, 8, 2, 256, 320, 128, False),   # GQA group of 4, ragged key block
    (1, 1, 1, 1, 129, 64, True),       # one query
    (1, 1, 1, 300, 33, 128, True),
    (1, 2, 1, 513, 513, 64, True),
    (2, 2, 2, 200, 1000, 128, False),
    (1, 8, 1, 200, 300, 64, True),     # GQA group of 8, d = 64, chunk at the end
    (1, 4, 2, 64, 64, 128, True),      # one 64-row step, one key block
    (1, 4, 2, 256, 384, 64, False),    # d = 64 non-causal, whole key blocks: no masked step
    (2, 2, 1, 130, 200, 64, False),    # d = 64 non-causal, ragged rows and keys
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_bwd_small(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    w = workloads.prefill(B, Hq, Hkv, Nq, Nk, d, seed=3000 + sum(case), causal=causal)
    do = workloads.grad_output(tuple(w.q.shape), 3500 + sum(case))
    say("bwd", case)
    O, L = orc.attention(host(w.q), host(w.k), host(w.v), w.scale, causal)
    o_saved, lse_saved = saved_state(w, O, L)
    dQ, dK, dV = orc.attention_backward(host(w.q), host(w.k), host(w.v), host(do), w.scale, causal,
                                        O=host(o_saved))
    q, k, v, g = (t.to(DEV) for t in (w.q, w.k, w.v, do))
    o_d, lse_d = o_saved.to(DEV), lse_saved.to(DEV)
    for odt in (torch.float32, torch.bfloat16):
        dq, dk, dv = run_bwd(q, k, v, g, causal, w.scale, odt, o_d, lse_d)
        bf = odt == torch.bfloat16
        check_grad(dq, dQ, "dQ", bf)
        check_grad(dk, dK, "dK", bf)
        check_grad(dv, dV, "dV", bf)


@pytest.mark.parametrize("case", [(1, 2, 1, 513, 513, 64, True), (2, 4, 2, 300, 700, 128, True),
                                  (1, 2, 2, 256, 256, 128, False)], ids=lambda c: "-".join(map(str, c)))
def test_bwd_after_gpu_forward(case):
    """Forward then backward on the GPU, against the exact gradient (whole-tensor bound)."""
    B, Hq, Hkv, Nq, Nk, d, causal = case
    w = workloads.prefill(B, Hq, Hkv, Nq, Nk, d, seed=3700 + sum(case), causal=causal)
    do = workloads.grad_output(tuple(w.q.shape), 3800 + sum(case))
    say("fwd+bwd", case)
    ref = orc.attention_backward(host(w.q), host(w.k), host(w.v), host(do), w.scale, causal)
    q, k, v, g = (t.to(DEV) for t in (w.q, w.k, w.v, do))
    got = run_bwd(q, k, v, g, causal, w.scale, torch.float32)
    for name, a, r in zip(("dQ", "dK", "dV"), got, ref):
        a = to_np(a)
        rel = float(np.sqrt(np.sum((a - r) ** 2)) / np.sqrt(np.sum(r * r)))
        say(f"  {name}: rel-l2 {rel:.2e}")
        assert np.all(np.isfinite(a)) and rel <= 2.0 ** -6, (name, rel)


def test_bwd_deterministic():
    w = workloads.prefill(1, 4, 2, 300, 300, 128, seed=3900, causal=True)
    do = workloads.grad_output(tuple(w.q.shape), 3901)
    q, k, v, g = (t.to(DEV) for t in (w.q, w.k, w.v, do))
    a = run_bwd(q, k, v, g, True, w.scale, torch.float32)
    b = run_bwd(q, k, v, g, True, w.scale, torch.float32)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_full_size_sampled_heads():
    """The prefill shape B=4, H=16, N=4096, d=128, causal: three whole heads against the
    oracle (dQ, dK, dV of each), in the launch configuration the bench times."""
    w, do = workloads.backward_4x16x4096()
    say(w.name)
    heads = [(0, 0), (1, 7), (3, 15)]
    # saved state: the oracle forward's O (bf16) and LSE for the sampled heads; the other
    # heads get O = 0, LSE = 0 (valid inputs whose gradients are not compared; with
    # H_q = H_kv every head's backward reads only its own saved state)
    o_saved = torch.zeros(w.q.shape, dtype=torch.bfloat16)
    lse_saved = torch.zeros(w.q.shape[:3], dtype=torch.float32)
    for b, h in heads:
        Oh, Lh = orc.attention_head(host(w.q[b, h]), host(w.k[b, h]), host(w.v[b, h]), w.scale, True)
        o_saved[b, h], lse_saved[b, h] = saved_state(w, Oh, Lh)
    q, k, v, g = (t.to(DEV) for t in (w.q, w.k, w.v, do))
    dq, dk, dv = run_bwd(q, k, v, g, True, w.scale, torch.bfloat16, o_saved.to(DEV), lse_saved.to(DEV))
    for b, h in heads:
        say(" head", b, h)
        rdq, rdk, rdv = orc.attention_head_backward(host(w.q[b, h]), host(w.k[b, h]), host(w.v[b, h]),
                                                    host(do[b, h]), w.scale, True, o=host(o_saved[b, h]))
        check_grad(dq[b, h], rdq, "dQ", True)
        check_grad(dk[b, h], rdk, "dK", True)
        check_grad(dv[b, h], rdv, "dV", True)
