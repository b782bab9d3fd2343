"""fa_fwd on the GPU against the fp64 oracle, through the C ABI.

Small cases compare every element (several tiles, ragged tails, GQA, causal with
N_q < N_k and N_q > N_k); the full-size workloads compare sampled rows that cover
every query block and many in-block positions, in the launch configuration the bench
times, plus properties that hold for every row."""

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


def run_fwd(w, out_dtype=None):
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    o = torch.full(q.shape, float("nan"), dtype=out_dtype or q.dtype, device=DEV)   # NaN canary
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd(q, k, v, o, lse, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o, lse


def sample_rows(n, per_block=2, block=128):
    rows = {0, 1, n - 1, n - 2}
    for qb in range((n + block - 1) // block):
        for j, (a, c) in enumerate([(37, 0), (53, 64), (29, 96)][:per_block]):
            r = qb * block + (qb * a + c) % block
            if r < n:
                rows.add(r)
    return np.array(sorted(rows))


# ---------------------------------------------------------------------------
# fp32 path
# ---------------------------------------------------------------------------

def test_single_head_fp32_full():
    w = workloads.single_head_fp32()
    say("fp32 single head 128x64")
    o, lse = run_fwd(w)
    O, L = orc.attention(host(w.q), host(w.k), host(w.v), w.scale, w.causal)
    check_o(o, O, "fp32")
    check_lse(lse, L, tol=1e-5)


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal", [
    (1, 2, 1, 100, 77, 64, False), (2, 4, 2, 77, 100, 128, True), (1, 1, 1, 130, 130, 128, True),
    (1, 2, 2, 70, 33, 64, True), (1, 1, 1, 1, 513, 64, False),
])
def test_fp32_cases(B, Hq, Hkv, Nq, Nk, d, causal):
    w = workloads.prefill(B, Hq, Hkv, Nq, Nk, d, seed=1000 + Nq, causal=causal, dtype="fp32")
    say("fp32", B, Hq, Hkv, Nq, Nk, d, causal)
    o, lse = run_fwd(w)
    O, L = orc.attention(host(w.q), host(w.k), host(w.v), w.scale, causal)
    check_o(o, O, "fp32")
    check_lse(lse, L, tol=1e-5)


@pytest.mark.parametrize("causal", [False, True])
def test_fp32_more_row_blocks_than_16_bits(causal):
    """N_q of 2^16 64-row blocks and more (4.19 million rows; the grid is one-dimensional),
    against the oracle on sampled rows around each 2^16-block boundary.  Causal with
    N_q > N_k: only the last N_k rows see a key, every other row must be O = 0, LSE = -inf."""
    n_q, n_k, d = 65536 * 64 + 100, 8, 64
    w = workloads.prefill(1, 1, 1, n_q, n_k, d, seed=1100 + causal, causal=causal, dtype="fp32")
    say("fp32, 4.19M rows, causal", causal)
    o, lse = run_fwd(w)
    idx = np.array([0, 1, 65535 * 64, 65536 * 64 - 1, 65536 * 64, n_q - n_k - 1, n_q - n_k, n_q - 1])
    O, L = orc.attention(host(w.q), host(w.k), host(w.v), w.scale, causal, rows=idx)
    check_o(o[:, :, idx], O, "fp32")
    check_lse(lse[:, :, idx], L, tol=1e-5)


# ---------------------------------------------------------------------------
# bf16 MFMA path, every element
# ---------------------------------------------------------------------------

SMALL = [
    (1, 1, 1, 128, 128), (2, 4, 2, 256, 320), (1, 2, 1, 100, 77), (1, 2, 2, 77, 100), (1, 1, 1, 1, 129),
    (1, 2, 1, 300, 200), (1, 1, 1, 513, 513), (1, 8, 1, 64, 1000), (1, 1, 1, 129, 1),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_bf16_small(shape, causal, d):
    B, Hq, Hkv, Nq, Nk = shape
    w = workloads.prefill(B, Hq, Hkv, Nq, Nk, d, seed=7 * Nq + Nk + d, causal=causal)
    say("bf16", shape, causal, d)
    O, L = orc.attention(host(w.q), host(w.k), host(w.v), w.scale, causal)
    o, lse = run_fwd(w)
    check_o(o, O, "bf16")
    check_lse(lse, L)
    o32, lse32 = run_fwd(w, out_dtype=torch.float32)
    check_o(o32, O, "fp32out")
    check_lse(lse32, L)


def test_bf16_scale_and_large_scores():
    """A large scale drives scores to +-100s: the max subtraction must keep exp finite."""
    w = workloads.prefill(1, 2, 2, 200, 300, 128, seed=3, causal=True, scale=2.0)
    say("bf16 scale 2.0")
    O, L = orc.attention(host(w.q), host(w.k), host(w.v), w.scale, True)
    o, lse = run_fwd(w, out_dtype=torch.float32)
    check_o(o, O, "fp32out")
    check_lse(lse, L)


def test_bf16_lse_optional():
    w = workloads.prefill(1, 2, 2, 130, 130, 64, seed=4, causal=False)
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    o, lse = fa.fa_fwd(q, k, v, causal=False, want_lse=False)
    assert lse is None
    torch.cuda.synchronize()
    O, _ = orc.attention(host(w.q), host(w.k), host(w.v), w.scale, False)
    check_o(o, O, "bf16")


# ---------------------------------------------------------------------------
# full-size workloads, sampled rows
# ---------------------------------------------------------------------------

def check_sampled(w, o, lse, mode):
    rows = sample_rows(w.q.shape[2])
    O, L = orc.attention(host(w.q), host(w.k), host(w.v), w.scale, w.causal, rows=rows)
    check_o(o[:, :, rows].cpu(), O, mode)
    check_lse(lse[:, :, rows].cpu(), L)
    # every row: finite, and a convex combination of V rows (|O| <= max |V| of its KV head)
    og = o.float()
    assert torch.isfinite(og).all() and torch.isfinite(lse).all()
    g = w.q.shape[1] // w.k.shape[1]
    vmax = w.v.float().abs().amax(dim=(2, 3)).repeat_interleave(g, dim=1).to(DEV)
    assert (og.abs().amax(dim=(2, 3)) <= vmax * 1.01 + 1e-3).all()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_4x16x4096(d, causal):
    w = workloads.prefill_4x16x4096(d, causal)
    say(w.name)
    o, lse = run_fwd(w)
    check_sampled(w, o, lse, "bf16")
    del o, lse
    o32, lse32 = run_fwd(w, out_dtype=torch.float32)
    check_sampled(w, o32, lse32, "fp32out")


def test_long_prefill_8192_heavy_keys():
    w = workloads.long_prefill_8192()
    say(w.name)
    o, lse = run_fwd(w)
    check_sampled(w, o, lse, "bf16")
    del o, lse
    o32, lse32 = run_fwd(w, out_dtype=torch.float32)
    check_sampled(w, o32, lse32, "fp32out")
    # rows right after a heavy key see a sharply peaked softmax: check them too
    hv = np.sort(w.heavy_rows[0, 0])
    rows = np.unique(np.clip(np.concatenate([hv, hv + 1, hv + 63]), 0, 8191))[:64]
    O, L = orc.attention(host(w.q[:, :1]), host(w.k[:, :1]), host(w.v[:, :1]), w.scale, True, rows=rows)
    check_o(o32[:, :1, rows].cpu(), O, "fp32out")
    check_lse(lse32[:, :1, rows].cpu(), L)
