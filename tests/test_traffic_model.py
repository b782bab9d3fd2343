"""The byte and FLOP accounting of the measurements, pinned to the numbers the pages print:
the table "One head, forward pass" of "Softmax and FlashAttention" (standard attention,
FlashAttention with no K/V reuse at blocks of 128 rows, and the every-value-once floor, at
three head shapes) and the chain "What FlashAttention removes from HBM" of "Attention kernel
chains" (one 8192 x 128 head: 34.4 GFLOP, 8 MiB compulsory, 128 MiB of scores, about 4096
FLOP per byte).  The causal variant of the no-reuse model is pinned to a brute-force count
of the keys every query row's block reads."""

import json
import os

import pytest

from online_softmax_07_amd import roofline as rl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def printed(value, as_printed):
    """`value` rounded to the digits the page prints equals the printed number."""
    text = repr(as_printed)
    decimals = len(text.split(".")[1]) if "." in text else 0
    return round(value, decimals) == as_printed


@pytest.mark.parametrize("row", golden("hbm_traffic_one_head.json")["rows"], ids=lambda r: f"N{r['N']}_d{r['d']}")
def test_one_head_table(row):
    g = golden("hbm_traffic_one_head.json")
    e, br, N, d = g["bytes_per_value"], g["block_rows"], row["N"], row["d"]
    std = rl.standard_attention_bytes(N, d, e) / 1e6
    fl = rl.flash_bytes_no_reuse(N, d, br, e) / 1e6
    floor = rl.flash_bytes_floor(N, d, e) / 1e6
    assert printed(std, row["standard_MB"]), std
    assert printed(fl, row["flash_no_l2_MB"]), fl
    assert printed(floor, row["floor_MB"]), floor
    # the exact per-block count agrees with the closed form without the mask (no LSE)
    assert rl.flash_bytes_model(N, N, d, br, causal=False, e=e, lse=False) == pytest.approx(fl * 1e6, rel=1e-12)


def test_one_head_8192x128_chain():
    g = golden("one_head_8192x128.json")
    N, d, e = g["N"], g["d"], g["bytes_per_value"]
    flops = rl.prefill_flops(1, 1, N, N, d, causal=False)
    assert round(flops / 1e9, 1) == g["flops_G"]
    compulsory = rl.flash_bytes_floor(N, d, e)
    assert compulsory == g["compulsory_MiB"] * 2 ** 20
    assert N * N * e == g["scores_MiB"] * 2 ** 20
    assert flops / compulsory == g["flop_per_byte_about"]
    # the floor of a whole launch is that of its heads (LSE aside)
    assert rl.prefill_bytes_floor(1, 32, 32, N, N, d, e, lse=False) == 32 * compulsory


def brute_force_kv_rows(N_q, N_k, Br, causal):
    """Keys each block of Br query rows reads: the largest key any of its rows sees, + 1."""
    total = 0
    for b0 in range(0, N_q, Br):
        reach = 0
        for i in range(b0, min(b0 + Br, N_q)):
            visible = [j for j in range(N_k) if not causal or j <= i + (N_k - N_q)]
            reach = max(reach, (max(visible) + 1) if visible else 0)
        total += reach
    return total


@pytest.mark.parametrize("N_q,N_k,Br", [(64, 64, 16), (100, 77, 32), (40, 130, 16), (130, 40, 32), (256, 256, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_causal_model_against_brute_force(N_q, N_k, Br, causal):
    d, e = 8, 2
    kv = brute_force_kv_rows(N_q, N_k, Br, causal)
    assert rl.flash_bytes_model(N_q, N_k, d, Br, causal, e, lse=False) == e * (2 * N_q * d + 2 * kv * d)
    assert rl.flash_bytes_model(N_q, N_k, d, Br, causal, e, lse=True) == e * (2 * N_q * d + 2 * kv * d) + 4 * N_q


def test_causal_model_is_about_half():
    # 4096 x 128 at Br = 256: (16 * 17 / 2) of 16 * 16 key-tile reads
    full = rl.flash_bytes_model(4096, 4096, 128, 256, False, lse=False) - 2 * 2 * 4096 * 128
    half = rl.flash_bytes_model(4096, 4096, 128, 256, True, lse=False) - 2 * 2 * 4096 * 128
    assert half / full == pytest.approx(136 / 256)
