"""Work and byte accounting for the attention workloads, and the MI355X peaks.

FLOPs (page "Attention kernel chains", chain "What FlashAttention removes from HBM"):
4 * N_q * N_k * d per (batch, query head) -- two matrix products of 2 * N_q * N_k * d
each -- the same count whatever the tile sizes; causal work is counted as half of that.

HBM bytes per head with e bytes per value (page "Softmax and FlashAttention", "Maths"):
  standard attention       e * (2Nd + 4N^2 + 2Nd)
  FlashAttention-2         e * (2Nd + 2N^2 d / B_r)      (no K/V re-read hits a cache)
  floor                    4 e N d                       (every value read or written once)

Decode is a K/V-bytes problem (page "Attention kernel chains", chain "GQA loads KV once
per group"): the algorithmic bytes are K and V once per KV head, Q, O, the fp32 LSE and
the int32 block table, each once.
"""

from __future__ import annotations

# Published MI355X figures.
PEAK_BF16_MFMA_TFLOPS = 2500.0   # dense bf16 matrix throughput (256 CU x 4096 FLOP/clk x 2.4 GHz = 2516.6)
PEAK_HBM_GBPS = 8000.0           # HBM3E bandwidth
NUM_CU = 256


def prefill_flops(B, H_q, N_q, N_k, d, causal) -> float:
    f = 4.0 * N_q * N_k * d * B * H_q
    return f / 2 if causal else f


def visible_pairs(N_q, N_k, causal) -> int:
    """Exact count of (query, key) pairs a head computes: with the bottom-right mask,
    query i sees max(0, i + N_k - N_q + 1) keys (never more than N_k)."""
    if not causal:
        return N_q * N_k
    shift = N_k - N_q
    lo = max(0, -shift)   # first query that sees a key
    n = N_q - lo          # queries that see one
    return n * (lo + shift + 1) + n * (n - 1) // 2


def chunked_prefill_flops(B, H_q, N_q, N_k, d, causal) -> float:
    """4 d FLOPs per visible (query, key) pair, counted exactly."""
    return 4.0 * d * visible_pairs(N_q, N_k, causal) * B * H_q


def prefill_bytes_floor(B, H_q, H_kv, N_q, N_k, d, e=2, lse=True) -> float:
    """Q and O once, K and V once per KV head, plus the fp32 LSE."""
    b = e * (2.0 * B * H_q * N_q * d + 2.0 * B * H_kv * N_k * d)
    if lse:
        b += 4.0 * B * H_q * N_q
    return b


def standard_attention_bytes(N, d, e=2) -> float:
    return e * (2.0 * N * d + 4.0 * N * N + 2.0 * N * d)


def flash_bytes_no_reuse(N, d, Br, e=2) -> float:
    return e * (2.0 * N * d + 2.0 * N * N * d / Br)


def flash_bytes_floor(N, d, e=2) -> float:
    return 4.0 * e * N * d


def flash_bytes_model(N_q, N_k, d, Br, causal, e=2, lse=True) -> float:
    """HBM bytes of one (batch, head) under the no-cache-reuse model of the FlashAttention-2
    loop order: Q and O once, and K and V read once per query block of Br rows.  Without the
    mask every block reads all N_k keys, which is e(2Nd + 2N^2 d / Br) for N_q = N_k = N;
    with the bottom-right causal mask block i (rows i Br ..) reads only the keys its last
    row sees, counted exactly.  Plus the fp32 LSE when `lse`."""
    n_blocks = -(-N_q // Br)
    kv_rows = 0
    for i in range(n_blocks):
        last_row = min((i + 1) * Br, N_q) - 1
        kv_rows += N_k if not causal else max(0, min(N_k, last_row + (N_k - N_q) + 1))
    b = e * (2.0 * N_q * d + 2.0 * kv_rows * d)
    if lse:
        b += 4.0 * N_q
    return b


def decode_bytes(B, H_q, H_kv, T, N_k, d, pages_per_seq=0, e=2) -> float:
    kv = 2.0 * B * H_kv * N_k * d * e
    qo = 2.0 * B * H_q * T * d * e
    lse = 4.0 * B * H_q * T
    table = 4.0 * B * pages_per_seq
    return kv + qo + lse + table


def decode_flops(B, H_q, T, N_k, d) -> float:
    return 4.0 * B * H_q * T * N_k * d
