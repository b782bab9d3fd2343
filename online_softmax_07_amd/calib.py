"""Python binding of libfa_calib.so (include/fa_calib.h) through ctypes, and the
measurements bench.py reports next to the published MI355X peaks: the sustained
matrix-core rate of an MFMA-only loop, how much fp32 vector work hides under that loop when
the same waves issue both, the one-pass HBM read rate in the decode kernel's access
pattern, and the shader clock.

Argument marshalling and timing only; the work runs in the library's kernels.
"""

from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

_lib = None

MFMA_FLOP = 2 * 32 * 32 * 16      # one 32x32x16 MFMA
MFMA_WAVES = 8                    # waves per workgroup of the MFMA loop
STREAM_THREADS = 256


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.CALIB_LIB):
        _build.build(verbose=False)
    if _build.is_stale():
        raise RuntimeError(f"{_build.CALIB_LIB} was not built from the sources in this tree: "
                           "run `python -m online_softmax_07_amd.build`")
    L = ctypes.CDLL(_build.CALIB_LIB)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.fa_calib_mfma.argtypes = [vp, vp, i, i, vp]
    L.fa_calib_mfma_valu.argtypes = [vp, vp, i, i, i, i, vp]
    L.fa_calib_stream_read.argtypes = [vp, sz, vp, i, vp]
    L.fa_calib_clock.argtypes = [vp, i, vp]
    for f in (L.fa_calib_mfma, L.fa_calib_mfma_valu, L.fa_calib_stream_read, L.fa_calib_clock):
        f.restype = i
    _lib = L
    return L


def _check(status: int, where: str):
    if status != 0:
        raise RuntimeError(f"{where} failed with status {status}")


def _sptr(stream) -> ctypes.c_void_p:
    return ctypes.c_void_p(stream.cuda_stream)


def shader_clock_mhz(device, stream, spin_ticks: int = 2000) -> float:
    """Shader clock over `spin_ticks` 100 MHz ticks (20 us by default), measured by one
    wave on `stream` (synchronises the stream)."""
    out = torch.zeros(2, dtype=torch.int64, device=device)
    _check(lib().fa_calib_clock(ctypes.c_void_p(out.data_ptr()), spin_ticks, _sptr(stream)), "fa_calib_clock")
    stream.synchronize()
    cyc, ticks = (int(x) for x in out.cpu())
    return 100.0 * cyc / ticks if ticks > 0 else float("nan")


def mfma_ceiling(device, stream, blocks: int = 256, iters: int = 60000) -> dict:
    """TFLOP/s of the MFMA-only loop (one 8-wave workgroup per CU, two waves per SIMD), and
    over each workgroup's loop the shader clock (s_memtime ticks per microsecond of the
    100 MHz real-time counter) and the bf16 FLOP per shader clock per CU (4096 at the
    published peak)."""
    sink = torch.empty(blocks * 64 * MFMA_WAVES, dtype=torch.float32, device=device)
    cyc = torch.zeros(2 * blocks, dtype=torch.int64, device=device)
    L = lib()
    args = (ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(cyc.data_ptr()), blocks)
    _check(L.fa_calib_mfma(*args, max(1, iters // 20), _sptr(stream)), "fa_calib_mfma")   # short warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    _check(L.fa_calib_mfma(*args, iters, _sptr(stream)), "fa_calib_mfma")
    e1.record(stream)
    stream.synchronize()
    ms = e0.elapsed_time(e1)
    flops = float(blocks) * MFMA_WAVES * iters * 4 * MFMA_FLOP
    c = cyc.view(blocks, 2).double()
    memtime, realtime = float(c[:, 0].mean()), float(c[:, 1].mean())
    per_wg = MFMA_WAVES * iters * 4 * MFMA_FLOP
    return {"tflops": round(flops / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 3),
            "memtime_mhz": round(100.0 * memtime / realtime, 0) if realtime > 0 else None,
            "loop_us_realtime": round(realtime / 100.0, 1),
            "flop_per_clock_per_cu": round(per_wg / memtime, 1) if memtime > 0 else None,
            "kernel": f"{blocks} workgroups x {MFMA_WAVES} waves, {iters} x 4 independent 32x32x16 bf16 MFMAs per wave"}


def mfma_valu_mix(device, stream, blocks: int = 256, iters: int = 20000, fmas=(24, 48)) -> dict:
    """For each count of fp32 FMAs per round of four 32x32x16 MFMAs (eight waves per CU, two
    per SIMD, as the prefill kernels run): the times of the MFMA-only, FMA-only and mixed
    loops, the share of the FMA-only time that disappears in the mixed loop (1: the vector
    work hides completely under the matrix work; 0: the two add up), and the matrix core's
    busy share in the mixed loop (MFMA-only time / mixed time).  The attention forward
    issues about 4.7 vector instructions per MFMA (d = 128, two issue slots per exponential
    counted once)."""
    sink = torch.empty(blocks * 64 * MFMA_WAVES, dtype=torch.float32, device=device)
    cyc = torch.zeros(2 * blocks, dtype=torch.int64, device=device)
    L = lib()

    def run(mfma: int, n: int) -> float:
        args = (ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(cyc.data_ptr()), blocks)
        _check(L.fa_calib_mfma_valu(*args, max(1, iters // 20), mfma, n, _sptr(stream)), "fa_calib_mfma_valu")
        best = None
        for _ in range(2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            _check(L.fa_calib_mfma_valu(*args, iters, mfma, n, _sptr(stream)), "fa_calib_mfma_valu")
            e1.record(stream)
            stream.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best

    out = {"kernel": f"{blocks} workgroups x {MFMA_WAVES} waves, {iters} rounds of 4 independent 32x32x16 bf16 "
                     "MFMAs and/or n fp32 FMAs in 8 independent chains per wave"}
    t_mfma = run(1, 0)
    for n in fmas:
        t_fma, t_mix = run(0, n), run(1, n)
        out[f"fma_per_round_{n}"] = {
            "mfma_only_ms": round(t_mfma, 3), "fma_only_ms": round(t_fma, 3), "mixed_ms": round(t_mix, 3),
            "fma_time_hidden": round((t_mfma + t_fma - t_mix) / t_fma, 3),
            "mfma_busy_in_mixed": round(t_mfma / t_mix, 3)}
    return out


def stream_read_ceiling(device, stream, nbytes: int = 512 << 20, flush=None, blocks_list=(256, 512, 1024, 2048)) -> dict:
    """Best GB/s over a few grid sizes of the nontemporal one-pass read of `nbytes`; `flush`
    (a callable) evicts the caches before each timed read."""
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=device)
    best = None
    L = lib()
    for blocks in blocks_list:
        sink = torch.empty(blocks * STREAM_THREADS, dtype=torch.float32, device=device)
        times = []
        for _ in range(3):
            if flush is not None:
                flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            _check(L.fa_calib_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                          blocks, _sptr(stream)), "fa_calib_stream_read")
            e1.record(stream)
            stream.synchronize()
            times.append(e0.elapsed_time(e1))
        gbs = nbytes / (min(times) * 1e-3) / 1e9
        if best is None or gbs > best["GB/s"]:
            best = {"GB/s": round(gbs, 1), "blocks": blocks, "bytes": nbytes}
    del buf
    return best
