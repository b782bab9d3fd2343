"""Sizes past 32-bit element offsets: a causal prefill whose Q, K, V and O each hold more
than 2^31 elements (4.3 GB in bf16), so every head after the first few sits beyond any
32-bit index.  Inputs are drawn on the device (workloads.prefill_on_device); the heads the
test checks, the first, a middle one and the last, are copied to the host for the oracle,
which computes sampled rows of each."""

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
