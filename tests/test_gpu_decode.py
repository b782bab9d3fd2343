"""fa_decode_splitkv and fa_lse_merge on the GPU against the fp64 oracle, through the
C ABI.  The full-size decode workloads are small enough in rows that every output row
is compared, for every split count swept."""

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


def run_decode(w, ns, out_dtype=torch.bfloat16, q=None, k=None, v=None, bt=None):
    q = w.q.to(DEV) if q is None else q
    k = w.k.to(DEV) if k is None else k
    v = w.v.to(DEV) if v is None else v
    if w.block_table is not None and bt is None:
        bt = w.block_table.to(DEV)
    o = torch.full(q.shape, float("nan"), dtype=out_dtype, device=DEV)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_decode_splitkv(q, k, v, o, lse, causal=w.causal, scale=w.scale, num_splits=ns, block_table=bt,
                         n_k=w.n_k)
    torch.cuda.synchronize()
    return o, lse


def oracle_of(w):
    bt = None if w.block_table is None else w.block_table.numpy()
    return orc.decode(host(w.q), host(w.k), host(w.v), w.scale, w.causal, block_table=bt,
                      page_size=w.page_size or None, n_k=w.n_k)


@pytest.fixture(scope="module")
def c4():
    w = workloads.decode_splitkv_128k()
    say(w.name, "oracle")
    return w, oracle_of(w), (w.q.to(DEV), w.k.to(DEV), w.v.to(DEV))


@pytest.mark.parametrize("ns", [1, 8, 16, 32, 64, 0])
def test_decode_splitkv_128k(c4, ns):
    w, (O, L), (q, k, v) = c4
    say(w.name, "num_splits", ns)
    o, lse = run_decode(w, ns, q=q, k=k, v=v)
    check_o(o, O, "bf16")
    check_lse(lse, L)
    o32, lse32 = run_decode(w, ns, torch.float32, q=q, k=k, v=v)
    check_o(o32, O, "fp32out")
    check_lse(lse32, L)


@pytest.fixture(scope="module")
def c5():
    w = workloads.decode_paged_b64()
    say(w.name, "oracle")
    return w, oracle_of(w), (w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), w.block_table.to(DEV))


@pytest.mark.parametrize("ns", [1, 2, 4, 8, 0])
def test_decode_paged_b64(c5, ns):
    w, (O, L), (q, k, v, bt) = c5
    say(w.name, "num_splits", ns)
    o, lse = run_decode(w, ns, q=q, k=k, v=v, bt=bt)
    check_o(o, O, "bf16")
    check_lse(lse, L)
    o32, lse32 = run_decode(w, ns, torch.float32, q=q, k=k, v=v, bt=bt)
    check_o(o32, O, "fp32out")
    check_lse(lse32, L)


# B, H_q, H_kv, T, N_k, d, causal, page_size, ns
SMALL = [
    (1, 4, 1, 1, 64, 128, True, 0, 1),
    (2, 8, 2, 1, 1000, 128, True, 0, 3),
    (1, 4, 4, 4, 333, 128, True, 0, 2),      # T > 1, bottom-right mask, g = 1
    (2, 8, 2, 3, 77, 64, True, 0, 8),        # splits beyond the keys are empty
    (1, 16, 2, 3, 500, 128, True, 0, 4),     # 24 stacked rows: two row chunks
    (1, 32, 1, 1, 200, 64, False, 0, 2),     # 32 heads in one group
    (3, 8, 1, 2, 129, 128, False, 0, 5),
    (1, 4, 2, 5, 3, 128, True, 0, 1),        # T > N_k: rows that see no key
    (2, 8, 1, 1, 300, 128, True, 16, 4),     # paged
    (2, 4, 2, 2, 101, 128, True, 5, 3),      # odd page size, ragged last page
    (1, 8, 8, 1, 1024, 64, True, 64, 0),
    (4, 8, 1, 1, 8192, 128, True, 16, 0),
    (8, 32, 8, 4, 4096, 128, True, 16, 0),   # multi-token decode over pages: 16 stacked rows
    (2, 8, 1, 16, 2000, 64, True, 16, 0),    # 128 stacked rows, ragged last page
    (256, 8, 1, 1, 1024, 128, True, 16, 8),  # 2048 workgroups: several splits of a group per CU in turn
]


@pytest.fixture(params=["in_kernel", "merge_kernel"])
def merge(request):
    """Both ways of combining the splits, each for every split count: inside the decode
    kernel and the separate merge kernel."""
    prev = fa.fa_decode_set_merge(fa.FA_MERGE_IN_KERNEL if request.param == "in_kernel" else fa.FA_MERGE_KERNEL)
    yield request.param
    fa.fa_decode_set_merge(prev)


def test_decode_merge_in_kernel_is_available():
    # the MI355X deals workgroups to its XCDs round-robin: the probe must find that period
    assert fa.fa_decode_set_merge(fa.FA_MERGE_AUTO) == fa.FA_MERGE_AUTO
    p = fa.fa_decode_merge_period(DEV)
    say("placement period", p)
    assert p > 0 and p & (p - 1) == 0
    assert fa.fa_decode_set_merge(fa.FA_MERGE_KERNEL) == fa.FA_MERGE_AUTO
    assert fa.fa_decode_merge_period(DEV) == 0
    assert fa.fa_decode_set_merge(fa.FA_MERGE_AUTO) == fa.FA_MERGE_KERNEL
    assert fa.fa_decode_merge_period(DEV) == p
    with pytest.raises(fa.FAError):
        fa.fa_decode_set_merge(7)
    assert fa.lib().fa_decode_set_merge(7) == fa.FA_ERR_BAD_SHAPE   # through the C ABI: unchanged
    assert fa.fa_decode_set_merge(fa.FA_MERGE_IN_KERNEL) == fa.FA_MERGE_AUTO
    assert fa.fa_decode_merge_period(DEV) == p
    assert fa.fa_decode_merge_in_kernel(64, 8, 1, 1, 8192, 128, 16, DEV)      # forced: any split count
    assert fa.fa_decode_set_merge(fa.FA_MERGE_AUTO) == fa.FA_MERGE_IN_KERNEL
    # automatic: inside while every workgroup is resident and one round per share covers the splits
    assert fa.fa_decode_merge_in_kernel(64, 8, 1, 1, 8192, 128, 0, DEV)       # 4 splits, 256 workgroups
    assert fa.fa_decode_merge_in_kernel(1, 32, 8, 1, 131072, 128, 0, DEV)     # 32 splits, 4 shares of 8
    assert not fa.fa_decode_merge_in_kernel(64, 8, 1, 1, 8192, 128, 16, DEV)  # 1024 workgroups
    assert not fa.fa_decode_merge_in_kernel(1, 32, 8, 1, 131072, 128, 64, DEV)  # 64 splits > 4 x 8
    assert not fa.fa_decode_merge_in_kernel(1, 32, 8, 1, 131072, 128, 1, DEV)   # one split: no merge


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_decode_small(case, merge):
    B, Hq, Hkv, T, Nk, d, causal, ps, ns = case
    w = workloads.decode(B, Hq, Hkv, T, Nk, d, seed=sum(case), causal=causal, page_size=ps,
                         num_pages=None if ps == 0 else B * (-(-Nk // ps)) + 3)
    say("decode", case, merge)
    O, L = oracle_of(w)
    o, lse = run_decode(w, ns)
    check_o(o, O, "bf16")
    check_lse(lse, L)
    o32, lse32 = run_decode(w, ns, torch.float32)
    check_o(o32, O, "fp32out")
    check_lse(lse32, L)


def test_decode_workspace_needs_no_initialization():
    """The workspace is scratch: one buffer, first filled with 0xA5 and later with 0xFF
    bytes, serves calls of different shapes in turn, each checked against the oracle (no
    result may depend on what a previous call or anything else left there)."""
    cases = [(2, 8, 2, 1, 1000, 128, True, 0, 3), (1, 16, 2, 3, 500, 128, True, 0, 4),
             (2, 8, 1, 1, 300, 128, True, 16, 4), (1, 4, 2, 1, 700, 64, False, 0, 7)]
    ws = torch.full((1 << 22,), 0xA5, dtype=torch.uint8, device=DEV)
    for fill in (0xA5, 0xFF):
        ws.fill_(fill)
        for rep in range(2):
            for case in cases:
                B, Hq, Hkv, T, Nk, d, causal, ps, ns = case
                say("decode, shared workspace", hex(fill), rep, case)
                w = workloads.decode(B, Hq, Hkv, T, Nk, d, seed=sum(case), causal=causal, page_size=ps,
                                     num_pages=None if ps == 0 else B * (-(-Nk // ps)) + 3)
                assert fa.fa_decode_workspace_bytes(B, Hq, Hkv, T, Nk, d, ns) <= ws.numel()
                O, L = oracle_of(w)
                q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
                bt = None if w.block_table is None else w.block_table.to(DEV)
                o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
                lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
                fa.fa_decode_splitkv(q, k, v, o, lse, causal=causal, scale=w.scale, num_splits=ns,
                                     block_table=bt, n_k=w.n_k, workspace=ws)
                torch.cuda.synchronize()
                check_o(o, O, "bf16")
                check_lse(lse, L)


@pytest.mark.parametrize("ns", [255, 300])
def test_decode_many_splits(ns, merge):
    """Hundreds of splits, each holding one 64-key piece, merged into one row per head."""
    w = workloads.decode(1, 4, 2, 1, 64 * ns, 64, seed=4700 + ns, causal=True)
    say("decode, many splits", ns, merge)
    O, L = oracle_of(w)
    o, lse = run_decode(w, ns)
    check_o(o, O, "bf16")
    check_lse(lse, L)


def test_decode_groups_past_16_bits():
    """More workgroup groups than a 16-bit grid dimension holds (70000 sequences of one KV head
    with two query heads each): the one-dimensional grid reaches every one.  Sampled sequences,
    at both ends and around 2^16, are compared with the oracle; every row must be finite."""
    B, Hq, Hkv, T, Nk, d = 70000, 2, 1, 1, 40, 64
    w = workloads.decode(B, Hq, Hkv, T, Nk, d, seed=4900, causal=True)
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    idx = [0, 1, 4095, 65534, 65535, 65536, 65537, B - 1]
    O, L = orc.decode(host(w.q[idx]), host(w.k[idx]), host(w.v[idx]), w.scale, True)
    for ns in (1, 2):
        say("decode, 70000 groups, num_splits", ns)
        o, lse = run_decode(w, ns, q=q, k=k, v=v)
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        check_o(o[idx], O, "bf16")
        check_lse(lse[idx], L)


def test_decode_merge_paths_agree(c5):
    """The in-kernel merge and the merge kernel weigh the same partials: their outputs agree
    to fp32 rounding (the two sum the splits in different orders), and the partials the
    in-kernel call leaves in the workspace merge, through fa_lse_merge, to the same rows."""
    w, (O, L), (q, k, v, bt) = c5
    ns = 8
    need = fa.fa_decode_workspace_bytes(64, 8, 1, 1, 8192, 128, ns)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    outs = {}
    for mode in (fa.FA_MERGE_AUTO, fa.FA_MERGE_KERNEL):
        prev = fa.fa_decode_set_merge(mode)
        o = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
        fa.fa_decode_splitkv(q, k, v, o, lse, causal=True, scale=w.scale, num_splits=ns, block_table=bt,
                             n_k=w.n_k, workspace=ws)
        torch.cuda.synchronize()
        fa.fa_decode_set_merge(prev)
        outs[mode] = (o, lse)
        if mode == fa.FA_MERGE_AUTO:
            rows = 64 * 8
            op = ws[: ns * rows * 128 * 4].view(torch.float32).view(ns, rows, 128)
            lp = ws[ns * rows * 128 * 4: ns * rows * 128 * 4 + ns * rows * 4].view(torch.float32).view(ns, rows)
            om, lm = fa.fa_lse_merge(op.clone(), lp.clone(), out_dtype=torch.float32)
            torch.cuda.synchronize()
            torch.testing.assert_close(om.view(o.shape), o, rtol=2e-6, atol=2e-6)
            torch.testing.assert_close(lm.view(lse.shape), lse, rtol=2e-6, atol=2e-6)
    (oa, la), (ok_, lk) = outs[fa.FA_MERGE_AUTO], outs[fa.FA_MERGE_KERNEL]
    torch.testing.assert_close(oa, ok_, rtol=2e-6, atol=2e-6)
    torch.testing.assert_close(la, lk, rtol=2e-6, atol=2e-6)
    check_o(oa, O, "fp32out")
    check_lse(la, L)


# ---------------------------------------------------------------------------
# fa_lse_merge on its own
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bounds", [[(0, 50)], [(0, 10), (10, 50)], [(0, 0), (0, 7), (7, 7), (7, 50)],
                                    [(i, i + 1) for i in range(50)] + [(50, 50)] * 20])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_lse_merge(bounds, out_dtype):
    rng = np.random.default_rng(len(bounds))
    B, Hq, Hkv, T, Nk, d = 2, 4, 2, 3, 50, 128
    Q = rng.standard_normal((B, Hq, T, d))
    K = rng.standard_normal((B, Hkv, Nk, d)) * 1.5
    V = rng.standard_normal((B, Hkv, Nk, d))
    Op, Lp = orc.split_partials(Q, K, V, 0.1, True, bounds)
    O, L = orc.attention(Q, K, V, 0.1, True)
    ns = len(bounds)
    rows = B * Hq * T
    op = torch.from_numpy(Op.reshape(ns, rows, d).astype(np.float32)).to(DEV)
    lp = torch.from_numpy(Lp.reshape(ns, rows).astype(np.float32)).to(DEV)
    say("merge", ns, out_dtype)
    o, lse = fa.fa_lse_merge(op, lp, out_dtype=out_dtype)
    torch.cuda.synchronize()
    check_o(o.reshape(B, Hq, T, d), O, "bf16" if out_dtype == torch.bfloat16 else "fp32out")
    check_lse(lse.reshape(B, Hq, T), L, tol=1e-5)


def test_lse_merge_all_empty():
    op = torch.zeros(3, 4, 64, device=DEV)
    lp = torch.full((3, 4), float("-inf"), device=DEV)
    o, lse = fa.fa_lse_merge(op, lp, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
