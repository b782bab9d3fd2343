"""The C-ABI library without a GPU: it loads, exports every function include/fa.h
declares, and rejects every invalid call with the documented status before any HIP
call (so these run on a CPU-only host).  No call here ever passes validation: pointers
are fake, and each case breaks at least one rule."""

import ctypes
import os
import re
import subprocess

import pytest
import torch

from online_softmax_07_amd import fa
from online_softmax_07_amd import build as fabuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

P = 0x10000  # a fake, 16-byte aligned "device pointer"; never dereferenced (validation fails first)


CALIB_HEADER = os.path.join(ROOT, "include", "fa_calib.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("fa_fwd", "fa_decode_splitkv", "fa_lse_merge"):
        assert required in names
    assert set(names) == set(fa.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = fa.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)


def test_every_header_is_covered():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["fa.h", "fa_calib.h"]


def test_calib_library_exports_every_declared_symbol():
    from online_softmax_07_amd import calib
    L = calib.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", fabuild.CALIB_LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)$", out, flags=re.M))
    names = declared_functions(CALIB_HEADER)
    assert names == ["fa_calib_clock", "fa_calib_mfma", "fa_calib_mfma_valu", "fa_calib_stream_read"]
    for name in names:
        assert name in exported, name
        assert hasattr(L, name)


def test_calib_rejects_before_any_launch():
    from online_softmax_07_amd import calib
    L = calib.lib()
    assert L.fa_calib_mfma(None, P, 1, 1, None) == 1
    assert L.fa_calib_mfma(P, P, 0, 1, None) == 2
    assert L.fa_calib_mfma(P, P, 1, 0, None) == 2
    assert L.fa_calib_mfma_valu(None, P, 1, 1, 1, 24, None) == 1
    assert L.fa_calib_mfma_valu(P, P, 0, 1, 1, 24, None) == 2
    assert L.fa_calib_mfma_valu(P, P, 1, 0, 1, 24, None) == 2
    assert L.fa_calib_mfma_valu(P, P, 1, 1, 2, 24, None) == 2    # mfma is 0 or 1
    assert L.fa_calib_mfma_valu(P, P, 1, 1, 1, 12, None) == 2    # fmas is 0, 24 or 48
    assert L.fa_calib_mfma_valu(P, P, 1, 1, 0, 0, None) == 2     # no work at all
    assert L.fa_calib_stream_read(None, 16, P, 1, None) == 1
    assert L.fa_calib_stream_read(P, 24, P, 1, None) == 2      # not a multiple of 16
    assert L.fa_calib_stream_read(P + 8, 16, P, 1, None) == 2   # not 16-byte aligned
    assert L.fa_calib_stream_read(P, 16, P, 0, None) == 2
    assert L.fa_calib_clock(None, 10, None) == 1
    assert L.fa_calib_clock(P, 0, None) == 2
    assert L.fa_calib_clock(P, 10000001, None) == 2


def test_build_is_current():
    assert not fabuild.is_stale(), "library is older than its sources: rebuild"


def test_stale_library_is_refused(tmp_path, monkeypatch):
    """A library whose recorded source hash does not match the tree (built from older
    sources) is refused by the loader, so no test or bench can run on it."""
    import shutil
    lib = tmp_path / "libfa_old.so"
    shutil.copy(fabuild.LIB, lib)
    (tmp_path / "libfa_old.so.srchash").write_text("0" * 64 + "\n")
    monkeypatch.setenv("FA_MI355X_LIB", str(lib))
    monkeypatch.setattr(fa, "_lib", None)
    with pytest.raises(RuntimeError, match="not built from the sources"):
        fa.lib()
    # the same file with the tree's hash (and the defines it was built with) is accepted
    (tmp_path / "libfa_old.so.srchash").write_text(fabuild.source_hash(["FA_TEST_DEFINE=1"]) + " FA_TEST_DEFINE=1\n")
    assert not fabuild.is_stale(str(lib))
    (tmp_path / "libfa_old.so.srchash").unlink()
    assert fabuild.is_stale(str(lib))


def test_version_and_status_strings():
    L = fa.lib()
    assert L.fa_version() == 102
    for s in range(7):
        assert fa.fa_status_string(s).startswith(
            ["FA_OK", "FA_ERR_NULL_PTR", "FA_ERR_BAD_SHAPE", "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE",
             "FA_ERR_ALIGNMENT", "FA_ERR_HIP"][s])
    assert fa.fa_status_string(99) == "unknown fa_status"


def fwd(**kw):
    a = dict(Q=P, K=P, V=P, O=P, LSE=P, B=1, H_q=2, H_kv=1, N_q=8, N_k=8, d=64, scale=0.125, causal=0,
             dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.lib().fa_fwd(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H_q"], a["H_kv"], a["N_q"],
                           a["N_k"], a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), fa.FA_ERR_NULL_PTR), (dict(K=None), fa.FA_ERR_NULL_PTR), (dict(V=None), fa.FA_ERR_NULL_PTR),
    (dict(O=None), fa.FA_ERR_NULL_PTR),
    (dict(B=0), fa.FA_ERR_BAD_SHAPE), (dict(H_q=0), fa.FA_ERR_BAD_SHAPE), (dict(H_kv=0), fa.FA_ERR_BAD_SHAPE),
    (dict(N_q=-1), fa.FA_ERR_BAD_SHAPE), (dict(N_k=-3), fa.FA_ERR_BAD_SHAPE), (dict(d=0), fa.FA_ERR_BAD_SHAPE),
    (dict(H_q=3, H_kv=2), fa.FA_ERR_BAD_SHAPE), (dict(scale=0.0), fa.FA_ERR_BAD_SHAPE),
    (dict(scale=-1.0), fa.FA_ERR_BAD_SHAPE), (dict(scale=float("nan")), fa.FA_ERR_BAD_SHAPE),
    (dict(scale=float("inf")), fa.FA_ERR_BAD_SHAPE), (dict(causal=2), fa.FA_ERR_BAD_SHAPE),
    (dict(B=70000, H_q=70000, H_kv=70000), fa.FA_ERR_BAD_SHAPE),
    # every size at its maximum: B * H * N must be rejected without the product overflowing
    (dict(B=2**31 - 1, H_q=2**31 - 1, H_kv=2**31 - 1, N_q=2**31 - 1, N_k=2**31 - 1), fa.FA_ERR_BAD_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(d=256), fa.FA_ERR_UNSUPPORTED), (dict(dtype=7), fa.FA_ERR_UNSUPPORTED),
    (dict(Q=P + 8), fa.FA_ERR_ALIGNMENT), (dict(O=P + 2), fa.FA_ERR_ALIGNMENT), (dict(LSE=P + 2), fa.FA_ERR_ALIGNMENT),
])
def test_fwd_rejects(kw, status):
    assert fwd(**kw) == status


def fwd_paged(**kw):
    a = dict(Q=P, K=P, V=P, O=P, LSE=P, B=2, H_q=4, H_kv=2, N_q=16, N_k=100, d=128, scale=0.1, causal=1,
             bt=P, ps=16, pps=7, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.lib().fa_fwd_paged(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H_q"], a["H_kv"],
                                 a["N_q"], a["N_k"], a["d"], a["scale"], a["causal"], a["bt"], a["ps"],
                                 a["pps"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), fa.FA_ERR_NULL_PTR), (dict(V=None), fa.FA_ERR_NULL_PTR), (dict(bt=None), fa.FA_ERR_NULL_PTR),
    (dict(N_q=-1), fa.FA_ERR_BAD_SHAPE), (dict(N_k=-1), fa.FA_ERR_BAD_SHAPE), (dict(H_q=3), fa.FA_ERR_BAD_SHAPE),
    (dict(scale=0.0), fa.FA_ERR_BAD_SHAPE), (dict(causal=3), fa.FA_ERR_BAD_SHAPE),
    (dict(ps=0), fa.FA_ERR_BAD_SHAPE), (dict(pps=0), fa.FA_ERR_BAD_SHAPE), (dict(pps=-1, N_k=0), fa.FA_ERR_BAD_SHAPE),
    (dict(pps=6), fa.FA_ERR_BAD_SHAPE),                       # 6 * 16 < 100 keys
    (dict(N_k=1 << 24, pps=1 << 20), fa.FA_ERR_BAD_SHAPE),    # beyond the exact page division
    (dict(B=1 << 16, pps=1 << 16, N_k=16), fa.FA_ERR_BAD_SHAPE),  # table entries beyond int32
    (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(dtype=fa.FA_FP32), fa.FA_ERR_UNSUPPORTED),
    (dict(K=P + 8), fa.FA_ERR_ALIGNMENT), (dict(O=P + 2), fa.FA_ERR_ALIGNMENT),
    (dict(bt=P + 2), fa.FA_ERR_ALIGNMENT), (dict(LSE=P + 1), fa.FA_ERR_ALIGNMENT),
])
def test_fwd_paged_rejects(kw, status):
    assert fwd_paged(**kw) == status


def bwd(**kw):
    a = dict(Q=P, K=P, V=P, O=P, dO=P, L=P, dQ=P, dK=P, dV=P, B=1, H_q=4, H_kv=2, N_q=100, N_k=90, d=128,
             scale=0.1, causal=1, ws=P, wsb=1 << 20, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.lib().fa_bwd(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["L"], a["dQ"], a["dK"], a["dV"], a["B"],
                           a["H_q"], a["H_kv"], a["N_q"], a["N_k"], a["d"], a["scale"], a["causal"], a["ws"],
                           a["wsb"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), fa.FA_ERR_NULL_PTR), (dict(O=None), fa.FA_ERR_NULL_PTR), (dict(dO=None), fa.FA_ERR_NULL_PTR),
    (dict(L=None), fa.FA_ERR_NULL_PTR), (dict(dK=None), fa.FA_ERR_NULL_PTR), (dict(dV=None), fa.FA_ERR_NULL_PTR),
    (dict(N_q=-2), fa.FA_ERR_BAD_SHAPE), (dict(N_k=-1), fa.FA_ERR_BAD_SHAPE), (dict(H_q=3), fa.FA_ERR_BAD_SHAPE),
    (dict(scale=-0.1), fa.FA_ERR_BAD_SHAPE), (dict(causal=2), fa.FA_ERR_BAD_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(dtype=fa.FA_FP32), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE), (dict(wsb=100), fa.FA_ERR_WORKSPACE),
    (dict(dO=P + 8), fa.FA_ERR_ALIGNMENT), (dict(dK=P + 2), fa.FA_ERR_ALIGNMENT), (dict(L=P + 2), fa.FA_ERR_ALIGNMENT),
    (dict(ws=P + 4), fa.FA_ERR_ALIGNMENT),
])
def test_bwd_rejects(kw, status):
    assert bwd(**kw) == status


def test_bwd_workspace_bytes():
    # one 64-float record per 32 rows of each (batch, query head), rows padded to 64
    assert fa.fa_bwd_workspace_bytes(4, 16, 4096) == 4 * 16 * 128 * 256
    assert fa.fa_bwd_workspace_bytes(1, 1, 1) == 2 * 256
    assert fa.fa_bwd_workspace_bytes(1, 3, 33) == 3 * 2 * 256
    assert fa.fa_bwd_workspace_bytes(2, 3, 65) == 2 * 3 * 4 * 256
    assert fa.fa_bwd_workspace_bytes(0, 1, 1) == 0


def dec(**kw):
    a = dict(Q=P, K=P, V=P, O=P, LSE=P, B=1, H_q=4, H_kv=2, T=1, N_k=100, d=128, scale=0.1, causal=1, ns=4,
             bt=None, ps=0, pps=0, ws=P, wsb=1 << 20, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.lib().fa_decode_splitkv(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H_q"], a["H_kv"],
                                      a["T"], a["N_k"], a["d"], a["scale"], a["causal"], a["ns"], a["bt"],
                                      a["ps"], a["pps"], a["ws"], a["wsb"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), fa.FA_ERR_NULL_PTR), (dict(O=None), fa.FA_ERR_NULL_PTR),
    (dict(T=-1), fa.FA_ERR_BAD_SHAPE), (dict(N_k=-1), fa.FA_ERR_BAD_SHAPE), (dict(H_q=5), fa.FA_ERR_BAD_SHAPE),
    (dict(ns=-1), fa.FA_ERR_BAD_SHAPE), (dict(scale=0.0), fa.FA_ERR_BAD_SHAPE), (dict(causal=-1), fa.FA_ERR_BAD_SHAPE),
    (dict(bt=P, ps=0, pps=7), fa.FA_ERR_BAD_SHAPE), (dict(bt=P, ps=16, pps=0), fa.FA_ERR_BAD_SHAPE),
    (dict(bt=P, ps=16, pps=6), fa.FA_ERR_BAD_SHAPE),   # 6 * 16 < 100 keys
    (dict(d=32), fa.FA_ERR_UNSUPPORTED), (dict(dtype=fa.FA_FP32), fa.FA_ERR_UNSUPPORTED),
    # the one-dimensional grid takes any B*H_kv: this call gets as far as the workspace check
    (dict(B=300, H_q=300, H_kv=300), fa.FA_ERR_WORKSPACE),
    # a split count whose workgroup count, groups rounded up to 64 times the splits, passes 2^31
    (dict(H_q=1, H_kv=1, ns=1 << 25, wsb=1 << 62), fa.FA_ERR_BAD_SHAPE),
    (dict(K=P + 4), fa.FA_ERR_ALIGNMENT), (dict(bt=P + 2, ps=16, pps=7), fa.FA_ERR_ALIGNMENT),
    (dict(ws=None), fa.FA_ERR_WORKSPACE), (dict(wsb=100), fa.FA_ERR_WORKSPACE), (dict(ns=0, N_k=100000, wsb=10), fa.FA_ERR_WORKSPACE),
    (dict(ws=P + 4), fa.FA_ERR_ALIGNMENT),
    # a split count whose partial rows (splits x B*H_q*T) pass 2^31: rejected before any
    # workspace size is computed (those offsets, and split * split_len, would wrap)
    (dict(ns=(1 << 29) + 1), fa.FA_ERR_BAD_SHAPE), (dict(ns=0x7fffffff, wsb=(1 << 63)), fa.FA_ERR_BAD_SHAPE),
])
def test_decode_rejects(kw, status):
    assert dec(**kw) == status


def dec_noalloc(**kw):
    a = dict(Q=P, K=P, V=P, O=P, LSE=P, B=1, H_q=4, H_kv=2, T=1, N_k=100, d=128, scale=0.1, causal=1, ns=4,
             bt=None, ps=0, pps=0, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.lib().fa_decode_splitkv_noalloc(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H_q"],
                                              a["H_kv"], a["T"], a["N_k"], a["d"], a["scale"], a["causal"],
                                              a["ns"], a["bt"], a["ps"], a["pps"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), fa.FA_ERR_NULL_PTR), (dict(T=-1), fa.FA_ERR_BAD_SHAPE), (dict(H_q=5), fa.FA_ERR_BAD_SHAPE),
    (dict(ns=-1), fa.FA_ERR_BAD_SHAPE), (dict(d=32), fa.FA_ERR_UNSUPPORTED), (dict(K=P + 4), fa.FA_ERR_ALIGNMENT),
    (dict(ns=(1 << 29) + 1), fa.FA_ERR_BAD_SHAPE),
    # partials beyond the 16 MiB scratch: 8193 splits x 4 rows x 129 floats
    (dict(ns=8193), fa.FA_ERR_WORKSPACE),
])
def test_decode_noalloc_rejects(kw, status):
    assert dec_noalloc(**kw) == status


def test_decode_noalloc_scratch_limit():
    rows, d = 4, 128
    assert fa.fa_decode_workspace_bytes(1, 4, 2, 1, 100, d, 8193) > fa.DECODE_NOALLOC_SCRATCH_BYTES
    assert fa.fa_decode_workspace_bytes(1, 4, 2, 1, 100, d, 8000) <= fa.DECODE_NOALLOC_SCRATCH_BYTES
    assert "FA_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)" in open(HEADER).read()
    assert dec_noalloc(T=0) == fa.FA_OK          # no query row: validated no-op, no HIP call


@pytest.mark.parametrize("kw,status", [
    (dict(Op=None), fa.FA_ERR_NULL_PTR), (dict(Lp=None), fa.FA_ERR_NULL_PTR), (dict(O=None), fa.FA_ERR_NULL_PTR),
    (dict(ns=0), fa.FA_ERR_BAD_SHAPE), (dict(rows=-1), fa.FA_ERR_BAD_SHAPE), (dict(d=0), fa.FA_ERR_BAD_SHAPE),
    (dict(d=513), fa.FA_ERR_BAD_SHAPE), (dict(dtype=fa.FA_BF16_IN_FP32_OUT), fa.FA_ERR_UNSUPPORTED),
    (dict(Op=P + 1), fa.FA_ERR_ALIGNMENT),
])
def test_merge_rejects(kw, status):
    a = dict(Op=P, Lp=P, O=P, L=P, ns=4, rows=8, d=128, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    assert fa.lib().fa_lse_merge(a["Op"], a["Lp"], a["O"], a["L"], a["ns"], a["rows"], a["d"], a["dtype"],
                                 a["stream"]) == status


def test_empty_calls_enqueue_nothing():
    """Zero query rows: every entry point validates and returns FA_OK without a HIP call (so
    this runs on a CPU-only host), and tensors of zero elements may be NULL."""
    assert fwd(N_q=0) == fa.FA_OK
    assert fwd(N_q=0, Q=None, O=None) == fa.FA_OK
    assert fwd(N_q=0, N_k=0, Q=None, O=None, K=None, V=None) == fa.FA_OK
    assert fwd(N_q=0, dtype=fa.FA_FP32) == fa.FA_OK
    assert fwd(N_q=1, Q=None) == fa.FA_ERR_NULL_PTR         # a non-empty tensor may not be NULL
    assert fwd(N_q=0, N_k=5, K=None) == fa.FA_ERR_NULL_PTR
    assert fwd_paged(N_q=0) == fa.FA_OK
    assert fwd_paged(N_q=0, N_k=0, bt=None, pps=0, K=None, V=None) == fa.FA_OK
    assert dec(T=0) == fa.FA_OK
    assert dec(T=0, Q=None, O=None, LSE=None) == fa.FA_OK
    assert dec(T=0, N_k=0, K=None, V=None, ns=1, ws=None, wsb=0) == fa.FA_OK
    assert bwd(N_q=0, N_k=0, Q=None, O=None, dO=None, L=None, dQ=None, K=None, V=None, dK=None, dV=None,
               ws=None, wsb=0) == fa.FA_OK
    assert fa.lib().fa_lse_merge(None, None, None, None, 4, 0, 128, fa.FA_BF16, None) == fa.FA_OK
    # the split heuristic and workspace sizes accept empty lengths
    assert fa.fa_decode_num_splits(1, 8, 1, 0, 100, 128) == 1
    assert fa.fa_decode_num_splits(1, 8, 1, 1, 0, 128) == 1
    assert fa.fa_decode_workspace_bytes(1, 8, 1, 1, 0, 128, 0) == 0
    assert fa.fa_bwd_workspace_bytes(1, 8, 0) == 0


def test_workspace_and_split_sizes():
    # one split needs no workspace
    assert fa.fa_decode_workspace_bytes(1, 32, 8, 1, 131072, 128, 1) == 0
    # ns partial rows of d fp32, then ns lse values per row, then one uint32 completion flag per
    # split and workgroup group (batch x KV head x 16 stacked rows), each part rounded to 256 bytes
    def r256(x):
        return (x + 255) // 256 * 256

    def ws(ns, rows, d, groups):
        return r256(ns * rows * d * 4) + r256(ns * rows * 4) + r256(ns * groups * 4)
    assert fa.fa_decode_workspace_bytes(1, 32, 8, 1, 131072, 128, 8) == ws(8, 32, 128, 8) == 131072 + 1024 + 256
    assert fa.fa_decode_workspace_bytes(1, 32, 8, 1, 131072, 128, (1 << 26) + 1) == 0   # 32 rows x splits > 2^31
    # one group: the grid (groups rounded up to 64, times the splits) passes 2^31 first
    assert fa.fa_decode_workspace_bytes(1, 1, 1, 1, 100, 128, 1 << 25) == 0         # 64 x 2^25 = 2^31
    assert fa.fa_decode_workspace_bytes(1, 1, 1, 1, 100, 128, (1 << 25) - 1) > 0
    assert fa.fa_decode_workspace_bytes(64, 8, 1, 1, 8192, 128, 4) == ws(4, 512, 128, 64) == 1048576 + 8192 + 1024
    assert fa.fa_decode_workspace_bytes(1, 32, 8, 1, 0, 128, 8) == ws(8, 32, 128, 8)      # empty cache, 8 splits
    # 2 x 40 query heads x 3 rows = 240 rows; 20 heads x 3 = 60 stacked rows per KV head -> 4 groups
    assert fa.fa_decode_workspace_bytes(2, 40, 2, 3, 500, 64, 5) == ws(5, 240, 64, 2 * 2 * 4) == 307200 + 4864 + 512
    assert fa.fa_decode_workspace_bytes(1, 32, 8, 1, -1, 128, 8) == 0                      # invalid length
    # the automatic split count aims at one wave of one workgroup on each of 256 CUs
    assert fa.fa_decode_num_splits(1, 32, 8, 1, 131072, 128) == 32
    assert fa.fa_decode_num_splits(64, 8, 1, 1, 8192, 128) == 4   # 64 groups x 4 splits
    assert fa.fa_decode_num_splits(256, 32, 8, 1, 4096, 128) == 1
    assert fa.fa_decode_num_splits(1, 32, 8, 1, 300, 128) == 2  # never more splits than 256-key pieces
    assert fa.fa_decode_workspace_bytes(1, 32, 8, 1, 131072, 128, 0) == fa.fa_decode_workspace_bytes(
        1, 32, 8, 1, 131072, 128, 32)


def test_binding_refuses_host_tensors():
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q, q, o=torch.zeros_like(q), lse=torch.zeros(1, 1, 4), stream=0)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q[:, :, :3], q)


def test_decode_merge_switch_host_side():
    """fa_decode_set_merge is host state only: it returns the previous choice and refuses
    anything but the three modes, leaving the choice unchanged."""
    L = fa.lib()
    assert L.fa_decode_set_merge(fa.FA_MERGE_KERNEL) == fa.FA_MERGE_AUTO
    assert L.fa_decode_set_merge(fa.FA_MERGE_IN_KERNEL) == fa.FA_MERGE_KERNEL
    for bad in (-1, 3, 1 << 30):
        assert L.fa_decode_set_merge(bad) == fa.FA_ERR_BAD_SHAPE
    assert L.fa_decode_set_merge(fa.FA_MERGE_AUTO) == fa.FA_MERGE_IN_KERNEL
    with pytest.raises(fa.FAError):
        fa.fa_decode_set_merge(5)
    assert fa.fa_decode_set_merge(fa.FA_MERGE_AUTO) == fa.FA_MERGE_AUTO


def test_decode_merge_in_kernel_rejects_bad_sizes_before_any_hip_call():
    L = fa.lib()
    assert L.fa_decode_merge_in_kernel(0, 8, 1, 1, 100, 128, 0, None) == -1     # B = 0
    assert L.fa_decode_merge_in_kernel(1, 6, 4, 1, 100, 128, 0, None) == -1     # H_q % H_kv != 0
    assert L.fa_decode_merge_in_kernel(1, 8, 1, 1, 100, 128, -3, None) == -1    # negative split count
