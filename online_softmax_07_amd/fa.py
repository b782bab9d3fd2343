"""Python binding of libfa_mi355x.so (include/fa.h) through ctypes.

Argument marshalling only: the functions below check that the torch tensors they are
given match the shapes, dtypes and device the C call will assume (the C ABI sees only
raw pointers and cannot check buffer sizes), allocate outputs when none are passed,
and call the library on the current HIP stream.  Every step of the computation runs in
the library's HIP kernels; there is no fallback path.  If the library is missing it is
built once (hipcc); if that fails, if the library was built from other sources than the
ones in the tree, or if it cannot be loaded, an error is raised.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

from . import build as _build

FA_OK, FA_ERR_NULL_PTR, FA_ERR_BAD_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_ALIGNMENT, FA_ERR_HIP = range(7)
FA_BF16, FA_FP32, FA_BF16_IN_FP32_OUT = 0, 1, 2

EXPORTED = ("fa_fwd", "fa_fwd_paged", "fa_bwd", "fa_bwd_workspace_bytes", "fa_decode_num_splits", "fa_decode_workspace_bytes", "fa_decode_splitkv",
            "fa_decode_splitkv_noalloc", "fa_decode_merge_period", "fa_decode_merge_in_kernel",
            "fa_decode_set_merge", "fa_lse_merge",
            "fa_status_string", "fa_version")
FA_MERGE_AUTO, FA_MERGE_KERNEL, FA_MERGE_IN_KERNEL = 0, 1, 2   # fa_decode_set_merge choices of include/fa.h
DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20   # FA_DECODE_NOALLOC_SCRATCH_BYTES of include/fa.h

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} (status {status})")


def library_path() -> str:
    """The in-tree build, or the file named by FA_MI355X_LIB (an alternative build)."""
    return os.environ.get("FA_MI355X_LIB") or _build.LIB


def lib() -> ctypes.CDLL:
    """Load (building first only if nothing is built) and declare the C ABI."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if path == _build.LIB and not os.path.exists(path):
        _build.build(verbose=False)
    if _build.is_stale(path):
        raise RuntimeError(f"{path} was not built from the sources in this tree (missing or mismatched "
                           f"{os.path.basename(path)}.srchash): run `python -m online_softmax_07_amd.build`")
    L = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    L.fa_fwd.restype = i
    L.fa_fwd_paged.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, i, i, vp]
    L.fa_fwd_paged.restype = i
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, i, vp]
    L.fa_bwd.restype = i
    L.fa_bwd_workspace_bytes.argtypes = [i, i, i]
    L.fa_bwd_workspace_bytes.restype = sz
    L.fa_decode_num_splits.argtypes = [i, i, i, i, i, i]
    L.fa_decode_num_splits.restype = i
    L.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.fa_decode_workspace_bytes.restype = sz
    L.fa_decode_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, i, i, vp, sz, i, vp]
    L.fa_decode_splitkv.restype = i
    L.fa_decode_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, i, i, i, vp]
    L.fa_decode_splitkv_noalloc.restype = i
    L.fa_decode_merge_period.argtypes = [vp]
    L.fa_decode_merge_period.restype = i
    L.fa_decode_merge_in_kernel.argtypes = [i, i, i, i, i, i, i, vp]
    L.fa_decode_merge_in_kernel.restype = i
    L.fa_decode_set_merge.argtypes = [i]
    L.fa_decode_set_merge.restype = i
    L.fa_lse_merge.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
    L.fa_lse_merge.restype = i
    L.fa_status_string.argtypes = [i]
    L.fa_status_string.restype = ctypes.c_char_p
    L.fa_version.argtypes = []
    L.fa_version.restype = i
    _lib = L
    return L


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_dev(device, **tensors):
    for name, t in tensors.items():
        if t is None:
            continue
        _need(t.is_cuda, f"{name} must be a GPU tensor")
        _need(t.device == device, f"{name} is on {t.device}, expected {device}")
        _need(t.is_contiguous(), f"{name} must be contiguous")


def _raise(status: int, where: str):
    if status != FA_OK:
        raise FAError(status, where)


# ---------------------------------------------------------------------------
# fa_fwd
# ---------------------------------------------------------------------------

def fa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, *, causal: bool = False, scale: Optional[float] = None,
           out_dtype: Optional[torch.dtype] = None, want_lse: bool = True, stream=None):
    """O, LSE = attention(Q, K, V).  q [B,H_q,N_q,d]; k, v [B,H_kv,N_k,d]; bf16 or fp32.
    bf16 inputs give bf16 O unless ``out_dtype=torch.float32`` (or an fp32 ``o``)."""
    _need(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be 4-D")
    B, H_q, N_q, d = q.shape
    _, H_kv, N_k, _ = k.shape
    _need(k.shape == (B, H_kv, N_k, d) and v.shape == k.shape, "k/v shape mismatch")
    _need(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    if q.dtype == torch.float32:
        dtype, odt = FA_FP32, torch.float32
        _need(out_dtype in (None, torch.float32), "fp32 inputs give fp32 output")
    elif q.dtype == torch.bfloat16:
        odt = out_dtype or (o.dtype if o is not None else torch.bfloat16)
        _need(odt in (torch.bfloat16, torch.float32), "bf16 inputs give bf16 or fp32 output")
        dtype = FA_BF16 if odt == torch.bfloat16 else FA_BF16_IN_FP32_OUT
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if o is None:
        o = torch.empty((B, H_q, N_q, d), dtype=odt, device=q.device)
    _need(o.shape == (B, H_q, N_q, d) and o.dtype == odt, "o has the wrong shape or dtype")
    if lse is None and want_lse:
        lse = torch.empty((B, H_q, N_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse.shape == (B, H_q, N_q) and lse.dtype == torch.float32, "lse must be fp32 [B,H_q,N_q]")
    _check_dev(q.device, q=q, k=k, v=v, o=o, lse=lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H_q, H_kv, N_q, N_k, d,
                      float(scale), int(bool(causal)), dtype, _stream(stream, q.device))
    _raise(st, "fa_fwd")
    return o, lse


def _paged_sizes(q, k, block_table, n_k, check_table):
    """(H_kv, N_k, page_size, pages_per_seq) of a paged cache: k is a pool
    [num_pages, page_size, H_kv, d], block_table int32 [B, pages_per_seq]."""
    B, d = q.shape[0], q.shape[3]
    num_pages, page_size, H_kv, dk = k.shape
    _need(dk == d, "pool head dimension must match q")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.shape[0] == B,
          "block_table must be int32 [B, pages_per_seq]")
    _need(block_table.is_contiguous(), "block_table must be contiguous")
    pages_per_seq = block_table.shape[1]
    N_k = pages_per_seq * page_size if n_k is None else int(n_k)
    _need(0 <= N_k <= pages_per_seq * page_size, "n_k exceeds the block table")
    _check_dev(q.device, block_table=block_table)
    if check_table and block_table.numel() > 0:
        lo, hi = int(block_table.min()), int(block_table.max())
        _need(0 <= lo and hi < num_pages, f"block_table entries must lie in [0, {num_pages})")
    return H_kv, N_k, page_size, pages_per_seq


def fa_fwd_paged(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_table: torch.Tensor,
                 n_k: Optional[int] = None, o: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, *, causal: bool = True, scale: Optional[float] = None,
                 out_dtype: Optional[torch.dtype] = None, want_lse: bool = True, check_table: bool = True,
                 stream=None):
    """Chunked prefill over a paged cache.  q [B,H_q,N_q,d] bf16 (the last N_q of the
    ``n_k`` positions of each sequence); k, v pools [num_pages,page_size,H_kv,d] bf16;
    block_table [B,pages_per_seq] int32; ``n_k`` defaults to pages_per_seq*page_size.
    With ``check_table`` the table entries are checked to lie inside the pool."""
    _need(q.dim() == 4 and q.dtype == torch.bfloat16, "q must be bf16 [B,H_q,N_q,d]")
    B, H_q, N_q, d = q.shape
    _need(k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16 and k.shape == v.shape and k.dim() == 4,
          "k, v must be bf16 pools of the same shape")
    H_kv, N_k, page_size, pages_per_seq = _paged_sizes(q, k, block_table, n_k, check_table)
    odt = out_dtype or (o.dtype if o is not None else torch.bfloat16)
    _need(odt in (torch.bfloat16, torch.float32), "output must be bf16 or fp32")
    dtype = FA_BF16 if odt == torch.bfloat16 else FA_BF16_IN_FP32_OUT
    if o is None:
        o = torch.empty((B, H_q, N_q, d), dtype=odt, device=q.device)
    _need(o.shape == (B, H_q, N_q, d) and o.dtype == odt, "o has the wrong shape or dtype")
    if lse is None and want_lse:
        lse = torch.empty((B, H_q, N_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse.shape == (B, H_q, N_q) and lse.dtype == torch.float32, "lse must be fp32 [B,H_q,N_q]")
    _check_dev(q.device, q=q, k=k, v=v, o=o, lse=lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_paged(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H_q, H_kv, N_q, N_k, d,
                            float(scale), int(bool(causal)), _ptr(block_table), int(page_size),
                            int(pages_per_seq), dtype, _stream(stream, q.device))
    _raise(st, "fa_fwd_paged")
    return o, lse


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def fa_bwd_workspace_bytes(B, H_q, N_q) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, H_q, N_q))


def fa_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, do: torch.Tensor,
           lse: torch.Tensor, dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
           dv: Optional[torch.Tensor] = None, *, causal: bool = False, scale: Optional[float] = None,
           out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """dQ, dK, dV of attention for the upstream gradient ``do``.  q, o, do [B,H_q,N_q,d] and
    k, v [B,H_kv,N_k,d] bf16; lse [B,H_q,N_q] fp32 from fa_fwd on the same inputs.
    Gradients are bf16 unless ``out_dtype=torch.float32`` (or fp32 ``dq``)."""
    _need(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be 4-D")
    B, H_q, N_q, d = q.shape
    _, H_kv, N_k, _ = k.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _need(t.dtype == torch.bfloat16, f"{name} must be bf16")
    _need(k.shape == (B, H_kv, N_k, d) and v.shape == k.shape, "k/v shape mismatch")
    _need(o.shape == q.shape and do.shape == q.shape, "o and do must have q's shape")
    _need(lse.shape == (B, H_q, N_q) and lse.dtype == torch.float32, "lse must be fp32 [B,H_q,N_q]")
    odt = out_dtype or (dq.dtype if dq is not None else torch.bfloat16)
    _need(odt in (torch.bfloat16, torch.float32), "gradients must be bf16 or fp32")
    if dq is None:
        dq = torch.empty(q.shape, dtype=odt, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=odt, device=q.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=odt, device=q.device)
    _need(dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape, "gradient shapes")
    _need(dq.dtype == odt and dk.dtype == odt and dv.dtype == odt, "gradients must share one dtype")
    need = fa_bwd_workspace_bytes(B, H_q, N_q)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check_dev(q.device, q=q, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv, workspace=workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                      B, H_q, H_kv, N_q, N_k, d, float(scale), int(bool(causal)), _ptr(workspace), ws_bytes,
                      FA_BF16 if odt == torch.bfloat16 else FA_BF16_IN_FP32_OUT, _stream(stream, q.device))
    _raise(st, "fa_bwd")
    return dq, dk, dv


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def fa_decode_num_splits(B, H_q, H_kv, T, N_k, d) -> int:
    return int(lib().fa_decode_num_splits(B, H_q, H_kv, T, N_k, d))


def fa_decode_workspace_bytes(B, H_q, H_kv, T, N_k, d, num_splits) -> int:
    return int(lib().fa_decode_workspace_bytes(B, H_q, H_kv, T, N_k, d, num_splits))


def _decode_prelude(q, k, v, o, lse, block_table, n_k, out_dtype, want_lse, check_table):
    """Shapes and outputs shared by both decode entry points."""
    _need(q.dim() == 4 and q.dtype == torch.bfloat16, "q must be bf16 [B,H_q,T,d]")
    B, H_q, T, d = q.shape
    _need(k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16 and k.shape == v.shape and k.dim() == 4,
          "k, v must be bf16 4-D tensors of the same shape")
    if block_table is None:
        _, H_kv, N_k, _ = k.shape
        _need(k.shape == (B, H_kv, N_k, d), "contiguous k/v must be [B,H_kv,N_k,d]")
        page_size = pages_per_seq = 0
        _need(n_k in (None, N_k), "n_k must equal k.shape[2] for a contiguous cache")
    else:
        H_kv, N_k, page_size, pages_per_seq = _paged_sizes(q, k, block_table, n_k, check_table)
    odt = out_dtype or (o.dtype if o is not None else torch.bfloat16)
    _need(odt in (torch.bfloat16, torch.float32), "output must be bf16 or fp32")
    dtype = FA_BF16 if odt == torch.bfloat16 else FA_BF16_IN_FP32_OUT
    if o is None:
        o = torch.empty((B, H_q, T, d), dtype=odt, device=q.device)
    _need(o.shape == (B, H_q, T, d) and o.dtype == odt, "o has the wrong shape or dtype")
    if lse is None and want_lse:
        lse = torch.empty((B, H_q, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse.shape == (B, H_q, T) and lse.dtype == torch.float32, "lse must be fp32 [B,H_q,T]")
    return B, H_q, H_kv, T, N_k, d, page_size, pages_per_seq, dtype, o, lse


def fa_decode_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None, *, causal: bool = True,
                      scale: Optional[float] = None, num_splits: int = 0,
                      block_table: Optional[torch.Tensor] = None, n_k: Optional[int] = None,
                      workspace: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                      want_lse: bool = True, check_table: bool = True, stream=None):
    """Split-KV decode.  q [B,H_q,T,d] bf16.  Contiguous: k, v [B,H_kv,N_k,d].  Paged:
    k, v pools [num_pages,page_size,H_kv,d] with block_table [B,pages_per_seq] int32 and
    ``n_k`` tokens per sequence (default pages_per_seq*page_size).  With ``check_table``
    the table entries are checked to lie inside the pool (one device reduction)."""
    B, H_q, H_kv, T, N_k, d, page_size, pages_per_seq, dtype, o, lse = _decode_prelude(
        q, k, v, o, lse, block_table, n_k, out_dtype, want_lse, check_table)
    need = fa_decode_workspace_bytes(B, H_q, H_kv, T, N_k, d, num_splits)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace.numel() * workspace.element_size() >= need, "workspace too small")
    _check_dev(q.device, q=q, k=k, v=v, o=o, lse=lse, workspace=workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fa_decode_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H_q, H_kv, T, N_k, d,
                                 float(scale), int(bool(causal)), int(num_splits), _ptr(block_table),
                                 int(page_size), int(pages_per_seq), _ptr(workspace), ws_bytes, dtype,
                                 _stream(stream, q.device))
    _raise(st, "fa_decode_splitkv")
    return o, lse


def fa_decode_splitkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                              lse: Optional[torch.Tensor] = None, *, causal: bool = True,
                              scale: Optional[float] = None, num_splits: int = 0,
                              block_table: Optional[torch.Tensor] = None, n_k: Optional[int] = None,
                              check_table: bool = False, stream=None):
    """fa_decode_splitkv with the partials in the library's per-GPU scratch: the caller
    passes every output (``o``, and ``lse`` or None) and nothing is allocated on the way."""
    _need(o is not None, "o must be given (this entry point allocates nothing)")
    B, H_q, H_kv, T, N_k, d, page_size, pages_per_seq, dtype, o, lse = _decode_prelude(
        q, k, v, o, lse, block_table, n_k, None, False, check_table)
    _check_dev(q.device, q=q, k=k, v=v, o=o, lse=lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_decode_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H_q, H_kv, T, N_k, d,
                                         float(scale), int(bool(causal)), int(num_splits), _ptr(block_table),
                                         int(page_size), int(pages_per_seq), dtype, _stream(stream, q.device))
    _raise(st, "fa_decode_splitkv_noalloc")
    return o, lse


def fa_decode_merge_period(device=None, stream=None) -> int:
    """Placement period the in-kernel decode merge uses on `device` (0: the merge kernel runs);
    probes the GPU on first use."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    return int(lib().fa_decode_merge_period(_stream(stream, dev)))


def fa_decode_merge_in_kernel(B, H_q, H_kv, T, N_k, d, num_splits=0, device=None, stream=None) -> bool:
    """Whether a decode call of these sizes merges inside the split kernel on `device`."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    r = int(lib().fa_decode_merge_in_kernel(B, H_q, H_kv, T, N_k, d, int(num_splits), _stream(stream, dev)))
    _need(r >= 0, "invalid decode sizes")
    return r == 1


def fa_decode_set_merge(mode: int) -> int:
    """FA_MERGE_AUTO, FA_MERGE_KERNEL or FA_MERGE_IN_KERNEL, process-wide; returns the
    previous choice."""
    if int(mode) not in (FA_MERGE_AUTO, FA_MERGE_KERNEL, FA_MERGE_IN_KERNEL):
        raise FAError(FA_ERR_BAD_SHAPE, "fa_decode_set_merge")
    st = int(lib().fa_decode_set_merge(int(mode)))
    if st not in (FA_MERGE_AUTO, FA_MERGE_KERNEL, FA_MERGE_IN_KERNEL):
        _raise(st, "fa_decode_set_merge")
    return st


def fa_lse_merge(o_part: torch.Tensor, lse_part: torch.Tensor, o: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, *, out_dtype: torch.dtype = torch.bfloat16, stream=None):
    """o_part [ns, rows, d] fp32, lse_part [ns, rows] fp32 -> o [rows, d], lse [rows]."""
    _need(o_part.dim() == 3 and o_part.dtype == torch.float32, "o_part must be fp32 [ns, rows, d]")
    ns, rows, d = o_part.shape
    _need(lse_part.shape == (ns, rows) and lse_part.dtype == torch.float32, "lse_part must be fp32 [ns, rows]")
    odt = o.dtype if o is not None else out_dtype
    _need(odt in (torch.bfloat16, torch.float32), "output must be bf16 or fp32")
    if o is None:
        o = torch.empty((rows, d), dtype=odt, device=o_part.device)
    _need(o.shape == (rows, d), "o must be [rows, d]")
    if lse is None:
        lse = torch.empty((rows,), dtype=torch.float32, device=o_part.device)
    _need(lse.shape == (rows,) and lse.dtype == torch.float32, "lse must be fp32 [rows]")
    _check_dev(o_part.device, o_part=o_part, lse_part=lse_part, o=o, lse=lse)
    st = lib().fa_lse_merge(_ptr(o_part), _ptr(lse_part), _ptr(o), _ptr(lse), ns, rows, d,
                            FA_BF16 if odt == torch.bfloat16 else FA_FP32, _stream(stream, o_part.device))
    _raise(st, "fa_lse_merge")
    return o, lse
