"""Sizes past 32-bit element offsets: a causal prefill whose Q, K, V and O each hold more
than 2^31 elements (4.3 GB in bf16), so every head after the first few sits beyond any
32-bit index, and a backward whose Q, O, dO and dQ do.  Inputs are drawn on the device
(workloads.prefill_on_device, grad_output_on_device); the heads the tests check, the
first, a middle one and the last, are copied to the host for the oracle."""

import numpy as np
import pytest
import torch

import oracle.fa_oracle as orc
from online_softmax_07_amd import fa, workloads
from parity import check_grad, check_lse, check_o

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def test_prefill_past_32bit_offsets():
    B, H, N, d = 1, 264, 65536, 128
    assert B * H * N * d > 2 ** 31
    say("large prefill: drawing inputs on the device")
    w = workloads.prefill_on_device(B, H, H, N, N, d, seed=5000, device=DEV, causal=True)
    say("large prefill: fa_fwd")
    o, lse = fa.fa_fwd(w.q, w.k, w.v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 4095, 4096, 30000, N - 2, N - 1}))
    for h in (0, H // 2, H - 1):
        say(" head", h)
        q, k, v = (t[0, h].float().cpu().numpy() for t in (w.q, w.k, w.v))
        O, L = orc.attention_head(q, k, v, w.scale, True, rows=rows)
        ri = torch.as_tensor(rows, device=DEV)
        check_o(o[0, h, ri], O, "bf16")
        check_lse(lse[0, h, ri], L)


def test_backward_past_32bit_offsets():
    """264 heads of 65536 queries over 256 keys, non-causal: Q, O, dO and dQ hold 2.2e9
    elements each.  The saved state is the GPU forward's (bf16 O, fp32 LSE), and the oracle
    takes D from that same O; whole heads are compared (dQ of every row, dK and dV)."""
    B, H, Nq, Nk, d = 1, 264, 65536, 256, 128
    assert B * H * Nq * d > 2 ** 31
    say("large backward: drawing inputs on the device")
    w = workloads.prefill_on_device(B, H, H, Nq, Nk, d, seed=5100, device=DEV, causal=False)
    do = workloads.grad_output_on_device(tuple(w.q.shape), 5101, DEV)
    say("large backward: fa_fwd")
    o, lse = fa.fa_fwd(w.q, w.k, w.v, causal=False, scale=w.scale)
    dq = torch.empty(w.q.shape, dtype=torch.bfloat16, device=DEV)
    dk = torch.empty(w.k.shape, dtype=torch.bfloat16, device=DEV)
    dv = torch.empty(w.v.shape, dtype=torch.bfloat16, device=DEV)
    say("large backward: fa_bwd")
    fa.fa_bwd(w.q, w.k, w.v, o, do, lse, dq, dk, dv, causal=False, scale=w.scale)
    torch.cuda.synchronize()
    for h in (0, H // 2, H - 1):
        say(" head", h)
        q, k, v, g, oh = (t[0, h].float().cpu().numpy() for t in (w.q, w.k, w.v, do, o))
        rdq, rdk, rdv = orc.attention_head_backward(q, k, v, g, w.scale, False, o=oh)
        check_grad(dq[0, h], rdq, "dQ", True)
        check_grad(dk[0, h], rdk, "dK", True)
        check_grad(dv[0, h], rdv, "dV", True)
