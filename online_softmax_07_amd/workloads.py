"""Seeded synthetic inputs for the attention workloads.

This module only draws numbers: it holds none of the attention arithmetic, so the
HIP path and the fp64 oracle can both be fed from it without sharing any of the
method.  Values are iid N(0,1) fp32 from ``numpy.random.default_rng(seed)``
(PCG64), drawn in the order Q, K, V and then any extras, and rounded to bf16 by
round-to-nearest-even (torch's CPU conversion).  The same bits go to the GPU and,
upcast exactly to fp32/fp64, to the oracle.

The shapes are the pages' workloads:

* a single 128x64 fp32 head (Kernel visualization: Flash Attention 1 works on
  one head with N keys and head dimension D);
* prefill at N = 4096, d in {64, 128} and N = 8192, d = 128 (Softmax and
  FlashAttention, table "One head, forward pass"; Attention kernel chains,
  "What FlashAttention removes from HBM");
* decode at batch 1, 8 KV heads, 128K context (Attention kernel chains, "How
  many splits for decode") and one GPU's share (H_q = 8, H_kv = 1) of a
  64-query-head / 8-KV-head model at batch 64, 8K context, 16-token pages
  ("GQA loads KV once per group", "The block-table cost of paged attention");
* the attention backward at the prefill shape (B=4, H=16, N=4096, d=128, causal) with
  an N(0,1) upstream gradient dO (Attention kernel chains, "What the backward pass
  saves", sized there for N = 8192 and 32 heads);
* chunked prefill over the same kind of paged cache: the last 2048 of 8192 positions
  of 4 sequences at 32 query / 8 KV heads (the decode model's head layout), 16-token
  pages ("The causal mask for a decode step": the new queries sit at the end).

N(0,1) values stand in for activations; no dataset is involved.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """fp32 numpy -> bf16 torch (CPU), round-to-nearest-even."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


@dataclass
class Prefill:
    name: str
    q: torch.Tensor          # [B, H_q, N_q, d]
    k: torch.Tensor          # [B, H_kv, N_k, d]
    v: torch.Tensor          # [B, H_kv, N_k, d]
    scale: float
    causal: bool
    heavy_rows: Optional[np.ndarray] = None   # [B, H_kv, n_heavy] key rows scaled x8, if any

    @property
    def shape(self):
        B, H_q, N_q, d = self.q.shape
        return dict(B=B, H_q=H_q, H_kv=self.k.shape[1], N_q=N_q, N_k=self.k.shape[2], d=d)


@dataclass
class Decode:
    name: str
    q: torch.Tensor          # [B, H_q, T, d]
    k: torch.Tensor          # contiguous [B, H_kv, N_k, d] or pool [pages, page_size, H_kv, d]
    v: torch.Tensor
    scale: float
    causal: bool
    n_k: int
    block_table: Optional[torch.Tensor] = None   # [B, pages_per_seq] int32
    page_size: int = 0
    num_splits: list = field(default_factory=lambda: [1])

    @property
    def shape(self):
        B, H_q, T, d = self.q.shape
        H_kv = self.k.shape[1] if self.block_table is None else self.k.shape[2]
        return dict(B=B, H_q=H_q, H_kv=H_kv, T=T, N_k=self.n_k, d=d)


def prefill(B, H_q, H_kv, N_q, N_k, d, seed, causal=False, dtype="bf16",
            heavy_frac=0.0, heavy_factor=8.0, scale=None, name="prefill") -> Prefill:
    """Q, K, V iid N(0,1).  ``heavy_frac`` > 0 picks, per (b, h_kv), round(heavy_frac * N_k)
    distinct key rows (seeded, drawn after V) and multiplies them by ``heavy_factor``
    after bf16 rounding (x8 is exact in bf16)."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, H_q, N_q, d))
    k = _normal(rng, (B, H_kv, N_k, d))
    v = _normal(rng, (B, H_kv, N_k, d))
    heavy = None
    if dtype == "bf16":
        qt, kt, vt = to_bf16(q), to_bf16(k), to_bf16(v)
    elif dtype == "fp32":
        qt, kt, vt = torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)
    else:
        raise ValueError(dtype)
    if heavy_frac > 0:
        n_heavy = int(round(heavy_frac * N_k))
        heavy = np.stack([np.stack([rng.choice(N_k, size=n_heavy, replace=False)
                                    for _ in range(H_kv)]) for _ in range(B)])
        for b in range(B):
            for h in range(H_kv):
                idx = torch.from_numpy(heavy[b, h])
                kt[b, h, idx] = kt[b, h, idx] * heavy_factor
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Prefill(name, qt, kt, vt, scale, causal, heavy)


def decode(B, H_q, H_kv, T, N_k, d, seed, causal=True, page_size=0, num_pages=None,
           scale=None, num_splits=(1,), name="decode") -> Decode:
    """Contiguous (page_size == 0) or paged KV.  Paged: K/V pools of ``num_pages``
    pages [num_pages, page_size, H_kv, d]; the block table is
    ``rng.permutation(num_pages)[: B * pages_per_seq]`` reshaped to [B, pages_per_seq]
    (drawn after the pools), pages_per_seq = ceil(N_k / page_size)."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, H_q, T, d))
    bt = None
    if page_size == 0:
        k = _normal(rng, (B, H_kv, N_k, d))
        v = _normal(rng, (B, H_kv, N_k, d))
    else:
        pps = -(-N_k // page_size)
        if num_pages is None:
            num_pages = B * pps
        assert num_pages >= B * pps
        k = _normal(rng, (num_pages, page_size, H_kv, d))
        v = _normal(rng, (num_pages, page_size, H_kv, d))
        bt = torch.from_numpy(rng.permutation(num_pages)[: B * pps].reshape(B, pps).astype(np.int32))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Decode(name, to_bf16(q), to_bf16(k), to_bf16(v), scale, causal, N_k, bt,
                  page_size, list(num_splits))


def prefill_on_device(B, H_q, H_kv, N_q, N_k, d, seed, device, causal=True, name="prefill_device") -> Prefill:
    """Q, K, V iid N(0,1) in bf16 drawn directly on `device` by torch's seeded generator, for
    inputs too large to draw on the host (element offsets past 2^31).  Both sides still see
    the same bits: tests copy the heads they check to the host for the oracle."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    q = torch.randn((B, H_q, N_q, d), generator=g, device=device, dtype=torch.bfloat16)
    k = torch.randn((B, H_kv, N_k, d), generator=g, device=device, dtype=torch.bfloat16)
    v = torch.randn((B, H_kv, N_k, d), generator=g, device=device, dtype=torch.bfloat16)
    return Prefill(name, q, k, v, 1.0 / math.sqrt(d), causal)


def grad_output(shape, seed) -> torch.Tensor:
    """The upstream gradient dO for a backward step: iid N(0,1) rounded to bf16, from its
    own seeded stream (so the forward inputs are the same with and without it)."""
    rng = np.random.default_rng(seed)
    return to_bf16(_normal(rng, shape))


def grad_output_on_device(shape, seed, device) -> torch.Tensor:
    """dO iid N(0,1) in bf16 drawn on `device` by torch's seeded generator (the companion of
    prefill_on_device for tensors too large to draw on the host)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.bfloat16)


# The five workloads, by what they are.
def single_head_fp32() -> Prefill:
    """Single head, non-causal, fp32, 128x64, scale 1/8."""
    return prefill(1, 1, 1, 128, 128, 64, seed=100, causal=False, dtype="fp32",
                   name="single_head_fp32_128x64")


def prefill_4x16x4096(d: int, causal: bool) -> Prefill:
    """B=4, H=16, N=4096, d in {64, 128}, bf16; the same inputs serve causal and not."""
    seed = {64: 200, 128: 201}[d]
    return prefill(4, 16, 16, 4096, 4096, d, seed=seed, causal=causal,
                   name=f"prefill_b4_h16_n4096_d{d}_{'causal' if causal else 'full'}")


def long_prefill_8192() -> Prefill:
    """B=1, H=32, N=8192, d=128, bf16, causal, 1% of key rows x8."""
    return prefill(1, 32, 32, 8192, 8192, 128, seed=300, causal=True, heavy_frac=0.01,
                   name="long_prefill_b1_h32_n8192_d128_causal_heavy1pct")


def decode_splitkv_128k() -> Decode:
    """B=1, T=1, H_q=32, H_kv=8, d=128, S=131072 contiguous, causal (bottom-right)."""
    return decode(1, 32, 8, 1, 131072, 128, seed=400, causal=True,
                  num_splits=(1, 8, 16, 32, 64), name="decode_splitkv_b1_hq32_hkv8_s131072")


def backward_4x16x4096() -> tuple:
    """The causal d=128 prefill inputs and a seeded dO of O's shape (seed 700): one
    training step's attention backward at the prefill shape."""
    w = prefill_4x16x4096(128, True)
    w.name = "backward_b4_h16_n4096_d128_causal"
    return w, grad_output(tuple(w.q.shape), 700)


def chunked_prefill_paged() -> Decode:
    """B=4, H_q=32, H_kv=8, d=128: a 2048-token chunk over 8192 cached positions (the chunk's
    own keys included), 16-token pages in a shuffled pool of 4*512 + 64 pages, causal."""
    return decode(4, 32, 8, 2048, 8192, 128, seed=600, causal=True, page_size=16,
                  num_pages=4 * 512 + 64, name="chunked_prefill_paged_b4_hq32_hkv8_q2048_ctx8192_p16")


def decode_paged_b64() -> Decode:
    """B=64, T=1, H_q=8, H_kv=1, d=128, ctx 8192, 16-token pages, pool of 64*512 pages."""
    return decode(64, 8, 1, 1, 8192, 128, seed=500, causal=True, page_size=16,
                  num_pages=64 * 512, num_splits=(1, 2, 4, 8),
                  name="decode_paged_b64_hq8_hkv1_ctx8192_p16")
