#!/usr/bin/env python3
"""Benchmark of the FlashAttention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra] [--no-cpu]

Default step: one fa_fwd call on the long causal prefill B=1, H_q=H_kv=32, N=8192, d=128
(1% of key rows scaled x8), bf16 in, bf16 O and fp32 LSE out, inputs resident in HBM: the
largest of the prefill configurations that fit one GPU.  The headline ``value`` is its
attention throughput in TFLOP/s (4 N^2 d per head, halved for causal) over the bracketed K
timed calls.  ``roofline`` prices the dominant kernel's average launch (HIP events
recorded on the stream the library launches on, created with hipEventDisableSystemFence so
that recording them adds no system-scope cache writeback) against the dense bf16 MFMA peak
(prefill) or the HBM peak (decode), with ``traffic`` taken from the committed rocprofv3
counter summary when it was measured on the current kernel source.  ``gpu_clock_mhz`` is
the shader clock measured by one wave right before and right after the timed region;
``calib`` the ceilings of the committed calibration kernels (an MFMA-only loop, the same
loop with fp32 FMAs issued by the same waves, and a
one-pass streaming read) measured after everything else; ``host`` the CPU model.
``breakdown`` adds the other prefill variants (including B=4, H=16, N=4096 at d=128 and
d=64), the chunked prefill over a paged cache (FLOPs: 4 d per visible query-key pair,
exact), the backward pass at the B=4 prefill shape (FLOPs: 2.5x the forward's) and the two
decode workloads (decode timed with L2 and the Infinity Cache flushed by a 1 GiB read
before every call).  ``cpu_baseline`` times the fp64 oracle on a bounded sample of the
headline workload.  Prints exactly one JSON line.

Warm-up: by default the timed workload runs back to back for 1 s before the K timed calls
(each breakdown entry for 0.3 s): this GPU raises its clock over the first few hundred
milliseconds of load, and a handful of warm-up calls times the ramp as well as the kernel.
``--warmup W`` runs exactly W untimed calls instead; the JSON reports the count made and
the clock.

``--workload`` makes another workload the timed one (for profiling); ``--calib-copy``
adds a plain 1 GiB device copy (torch's copy kernel), the reference that scales the
HBM byte counters.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence of hip_runtime_api.h


class HipEvent:
    """A HIP timing event created with hipEventDisableSystemFence, the flag HIP documents for
    timing: recording it does not write back and invalidate the caches at system scope, a
    cost (about 2.4 us per bracket on the paged decode) that is part of the event, not of the
    work between two events.  Recorded on an explicit stream."""
    _hip = None

    def __init__(self):
        if HipEvent._hip is None:
            h = ctypes.CDLL("libamdhip64.so")   # the HIP runtime torch has loaded
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipEvent._hip = h
        self.e = ctypes.c_void_p()
        if HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if HipEvent._hip.hipEventRecord(self.e, ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (waits for `end`)."""
        h = HipEvent._hip
        ms = ctypes.c_float()
        if h.hipEventSynchronize(end.e) != 0 or h.hipEventElapsedTime(ctypes.byref(ms), self.e, end.e) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        if HipEvent._hip is not None and self.e:
            HipEvent._hip.hipEventDestroy(self.e)


METRIC = "attention TFLOP/s + % MFMA peak (prefill); HBM GB/s + % peak (decode), 1 GPU"
HERE = os.path.dirname(os.path.abspath(__file__))
PREFILL = {
    "prefill_d128_causal": (128, True), "prefill_d128_full": (128, False),
    "prefill_d64_causal": (64, True), "prefill_d64_full": (64, False),
}
DECODE = ("decode_splitkv_128k", "decode_paged_b64")
PAGED_PREFILL = ("chunked_prefill_paged",)
BACKWARD = ("backward",)
WORKLOADS = tuple(PREFILL) + ("long_prefill_8192",) + PAGED_PREFILL + BACKWARD + DECODE


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=-1,
                   help="untimed calls before the timed ones; -1 (default): as many as fill %.1f s, "
                        "the time this GPU takes to reach its steady clock under the load" % WARM_S)
    p.add_argument("--workload", default="long_prefill_8192", choices=WORKLOADS)
    p.add_argument("--num-splits", type=int, default=0, help="decode split count for --workload (0 = auto)")
    p.add_argument("--no-extra", action="store_true", help="time the --workload only")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--calib-copy", action="store_true", help="also run a plain 1 GiB copy (counter calibration)")
    p.add_argument("--no-flush", action="store_true", help="decode --workload: time without the cache flush")
    p.add_argument("--no-calib", action="store_true", help="skip the calibration ceilings")
    p.add_argument("--out", default=None, help="also write the JSON line to this file")
    return p.parse_args()


WARM_S = 1.0          # default warm-up of the timed workload, seconds of back-to-back calls
WARM_S_EXTRA = 0.3    # warm-up of each breakdown entry (the GPU is already at its clock)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this library is single-GPU: run bench.py with --gpus 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    sys.path.insert(0, HERE)
    from online_softmax_07_amd import build as fabuild, calib, fa, roofline as rl, workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def warm(fn, warmup, pre=None, seconds=WARM_S):
        """warmup >= 0: exactly that many untimed calls; < 0: calls until `seconds` of wall
        time have passed (at least 10).  Returns the number of calls made."""
        n = 0
        t_end = time.perf_counter() + seconds
        while (warmup >= 0 and n < warmup) or (warmup < 0 and (n < 10 or time.perf_counter() < t_end)):
            if pre:
                pre()
            fn()
            n += 1
            if warmup < 0 and n % 16 == 0:
                torch.cuda.synchronize()   # keep the queue short so the wall clock tracks the GPU
        torch.cuda.synchronize()
        return n

    def timed(fn, steps, warmup, pre=None, seconds=WARM_S, clocks=None):
        """Per-call durations (ms) from HIP events recorded on the launch stream, the
        bracketed total of the K calls (pre(), e.g. a cache flush, sits outside each call's
        bracket but inside the total), and the number of warm-up calls made first.  With
        `clocks` (a dict), the shader clock is measured right before and right after the
        bracket, outside it."""
        n_warm = warm(fn, warmup, pre, seconds)
        st = [HipEvent() for _ in range(steps)]
        en = [HipEvent() for _ in range(steps)]
        t0, t1 = HipEvent(), HipEvent()
        torch.cuda.synchronize()
        if clocks is not None:
            clocks["before_timed"] = round(calib.shader_clock_mhz(dev, stream), 0)
        t0.record(stream)
        for i in range(steps):
            if pre:
                pre()
            st[i].record(stream)
            fn()
            en[i].record(stream)
        t1.record(stream)
        torch.cuda.synchronize()
        if clocks is not None:
            clocks["after_timed"] = round(calib.shader_clock_mhz(dev, stream), 0)
        return t0.elapsed_time(t1), [a.elapsed_time(b) for a, b in zip(st, en)], n_warm

    def make(name):
        if name in PREFILL:
            return workloads.prefill_4x16x4096(*PREFILL[name])
        if name == "long_prefill_8192":
            return workloads.long_prefill_8192()
        if name == "chunked_prefill_paged":
            return workloads.chunked_prefill_paged()
        if name == "backward":
            return workloads.backward_4x16x4096()
        if name == "decode_splitkv_128k":
            return workloads.decode_splitkv_128k()
        return workloads.decode_paged_b64()

    def prefill_case(w):
        q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        s = w.shape
        flops = rl.prefill_flops(s["B"], s["H_q"], s["N_q"], s["N_k"], s["d"], w.causal)

        def fn():
            fa.fa_fwd(q, k, v, o, lse, causal=w.causal, scale=w.scale, stream=stream)
        return fn, flops, (q, k, v, o, lse)

    def paged_prefill_case(w):
        q, k, v, bt = (t.to(dev) for t in (w.q, w.k, w.v, w.block_table))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        s = w.shape
        flops = rl.chunked_prefill_flops(s["B"], s["H_q"], s["T"], s["N_k"], s["d"], w.causal)
        assert 0 <= int(bt.min()) and int(bt.max()) < w.k.shape[0]   # once, outside any timing

        def fn():
            fa.fa_fwd_paged(q, k, v, bt, w.n_k, o, lse, causal=w.causal, scale=w.scale, check_table=False,
                            stream=stream)
        return fn, flops, (q, k, v, bt, o, lse)

    def backward_case(wd):
        """fa_bwd (D prep + dQ + dK/dV kernels) on the forward's own O and LSE; FLOPs are
        2.5x the forward's (five products of 2 N_q N_k d each, halved for causal), the
        usual count, although the dQ kernel recomputes two of them."""
        w, do = wd
        q, k, v, g = (t.to(dev) for t in (w.q, w.k, w.v, do))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        fa.fa_fwd(q, k, v, o, lse, causal=w.causal, scale=w.scale, stream=stream)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        s = w.shape
        ws = torch.empty(fa.fa_bwd_workspace_bytes(s["B"], s["H_q"], s["N_q"]), dtype=torch.uint8, device=dev)
        flops = 2.5 * rl.prefill_flops(s["B"], s["H_q"], s["N_q"], s["N_k"], s["d"], w.causal)

        def fn():
            fa.fa_bwd(q, k, v, o, g, lse, dq, dk, dv, causal=w.causal, scale=w.scale, workspace=ws, stream=stream)
        return fn, flops, (q, k, v, g, o, lse, dq, dk, dv, ws)

    def any_prefill_case(w):
        if isinstance(w, tuple):
            return backward_case(w)
        return paged_prefill_case(w) if w.name.startswith("chunked_prefill") else prefill_case(w)

    def decode_case(w, ns):
        q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
        bt = None if w.block_table is None else w.block_table.to(dev)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        sh = w.shape
        pps = 0 if bt is None else bt.shape[1]
        nbytes = rl.decode_bytes(sh["B"], sh["H_q"], sh["H_kv"], sh["T"], sh["N_k"], sh["d"], pps)
        wsb = fa.fa_decode_workspace_bytes(sh["B"], sh["H_q"], sh["H_kv"], sh["T"], sh["N_k"], sh["d"], ns)
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
        if bt is not None:   # validate the table once, outside any timing
            assert 0 <= int(bt.min()) and int(bt.max()) < w.k.shape[0]

        def fn():
            fa.fa_decode_splitkv(q, k, v, o, lse, causal=w.causal, scale=w.scale, num_splits=ns,
                                 block_table=bt, n_k=w.n_k, workspace=ws, check_table=False, stream=stream)
        return fn, nbytes, (q, k, v, bt, o, lse, ws)

    flush = None

    def flush_caches():
        # Read (not write) 1 GiB: evicts L2 and the 256 MB Infinity Cache with clean lines,
        # so no write-back of dirty flush data competes with the timed call.
        flush_sink.copy_(flush.view(torch.int64).sum(dtype=torch.int64))

    # ---- the timed workload ----
    head = args.workload
    w = make(head)
    w_inputs = w
    if head in BACKWARD:
        w = w[0]
    s = w.shape
    flush_sink = torch.zeros((), dtype=torch.int64, device=dev)
    clocks = {}
    if head in DECODE:
        flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)   # 1 GiB: evicts L2 and MALL
        fn, nbytes, bufs = decode_case(w, args.num_splits)
        total_ms, per, n_warm = timed(fn, args.steps, args.warmup, pre=None if args.no_flush else flush_caches,
                                      clocks=clocks)
        avg = statistics.mean(per)
        ms_per_step = avg   # the flush between calls is not part of the step
        value = nbytes / (ms_per_step * 1e-3) / 1e9
        unit, bound, peak, achieved = "GB/s", "hbm", rl.PEAK_HBM_GBPS, nbytes / (avg * 1e-3) / 1e9
        ns = args.num_splits or fa.fa_decode_num_splits(s["B"], s["H_q"], s["H_kv"], s["T"], s["N_k"], s["d"])
        in_kernel = fa.fa_decode_merge_in_kernel(s["B"], s["H_q"], s["H_kv"], s["T"], s["N_k"], s["d"], ns,
                                                 dev, stream)
        kernel = ("fa::decode_split_kernel (LSE merge inside)" if in_kernel or ns == 1
                  else "fa::decode_split_kernel + fa::lse_merge_kernel")
        extra_cfg = {"T": s["T"], "num_splits": ns, "bytes_per_step": nbytes, "paged": w.block_table is not None}
    else:
        paged = head in PAGED_PREFILL
        fn, flops, bufs = any_prefill_case(w_inputs)
        total_ms, per, n_warm = timed(fn, args.steps, args.warmup, clocks=clocks)
        avg = statistics.mean(per)
        ms_per_step = total_ms / args.steps
        value = flops / (ms_per_step * 1e-3) / 1e12
        unit, bound, peak, achieved = "TFLOP/s", "mfma", rl.PEAK_BF16_MFMA_TFLOPS, flops / (avg * 1e-3) / 1e12
        bc = 128 if (s["d"] == 128 and not paged) else 64   # the launch's key tile,
        nw, rh = (8, 1) if s["d"] == 128 else (4, 2)          # waves and 32-row halves per wave
        kernel = (f"fa::fwd_bf16_kernel<{s['d']}, {bc}, {nw}, {rh}, {str(w.causal).lower()}, "
                  f"{str(paged).lower()}, bf16>")
        if head in BACKWARD:
            kernel = "fa::bwd_prep_kernel + fa::bwd_dq_kernel + fa::bwd_dkdv_kernel (whole fa_bwd call)"
        extra_cfg = {"N_q": s["T"] if paged else s["N_q"], "N_k": s["N_k"], "causal": w.causal,
                     "flops_per_step": flops}
        if paged:
            extra_cfg.update({"paged": True, "page_size": w.page_size,
                              "flops": "4 d per visible (query, key) pair, exact"})
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: iid N(0,1) rounded to bf16 (seeded)",
        "config": {"workload": w.name, "B": s["B"], "H_q": s["H_q"], "H_kv": s["H_kv"], "d": s["d"], **extra_cfg},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": None, "kernel": kernel,
                     "avg_launch_us": round(avg * 1e3, 2)},
        "gpu_clock_mhz": clocks,
        "host": host_info(),
        "timing": "HIP events on the launch stream, created with hipEventDisableSystemFence",
    }
    traffic = load_traffic(w.name, fabuild)
    if traffic is not None:
        result["roofline"]["traffic"] = traffic
    del bufs

    # ---- breakdown ----
    if not args.no_extra:
        breakdown = {}
        for name in WORKLOADS:
            if name == head or name in DECODE:
                continue
            ww = make(name)
            fn, fl, bufs = any_prefill_case(ww)
            _, per, _ = timed(fn, max(10, args.steps // 2), -1, seconds=WARM_S_EXTRA)
            med = statistics.median(per)
            if isinstance(ww, tuple):
                ww = ww[0]
            breakdown[ww.name] = {"us": round(med * 1e3, 2), "TFLOP/s": round(fl / med / 1e9, 2),
                                  "frac_mfma": round(fl / med / 1e9 / rl.PEAK_BF16_MFMA_TFLOPS, 4)}
            del bufs
        if flush is None:
            flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        for name in DECODE:
            ww = make(name)
            entry, best = {"by_num_splits": {}}, None
            for ns in list(ww.num_splits) + [0]:
                fn, nbytes, bufs = decode_case(ww, ns)
                _, per, _ = timed(fn, 100, -1, pre=flush_caches, seconds=WARM_S_EXTRA)
                med = statistics.median(per)
                gbs = nbytes / (med * 1e-3) / 1e9
                key = "auto" if ns == 0 else str(ns)
                entry["by_num_splits"][key] = {"us": round(med * 1e3, 2), "min_us": round(min(per) * 1e3, 2),
                                               "GB/s": round(gbs, 1), "frac_hbm": round(gbs / rl.PEAK_HBM_GBPS, 4)}
                if best is None or gbs > best[1]:
                    best = (key, gbs)
                del bufs
            entry["bytes"] = nbytes
            entry["best"] = {"num_splits": best[0], "GB/s": round(best[1], 1),
                             "frac_hbm": round(best[1] / rl.PEAK_HBM_GBPS, 4)}
            breakdown[ww.name] = entry
        result["breakdown"] = breakdown
    del flush

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(3)
        torch.cuda.synchronize()
        _, per, _ = timed(lambda: b.copy_(a), 5, 2)
        result["calib_copy"] = {"bytes_read": 1 << 30, "bytes_written": 1 << 30,
                                "us": round(statistics.median(per) * 1e3, 2)}
        del a, b

    # ---- calibrated ceilings (context for the fractions of the published peaks) ----
    if not args.no_calib:
        flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        mf = calib.mfma_ceiling(dev, stream)
        mix = calib.mfma_valu_mix(dev, stream)
        sr = calib.stream_read_ceiling(dev, stream, flush=flush_caches)
        del flush
        result["calib"] = {
            "mfma_loop": {**mf, "frac_of_peak": round(mf["tflops"] / rl.PEAK_BF16_MFMA_TFLOPS, 4)},
            "mfma_valu_mix": mix,
            "stream_read": {**sr, "frac_of_peak": round(sr["GB/s"] / rl.PEAK_HBM_GBPS, 4)},
        }
        ceiling = mf["tflops"] if unit == "TFLOP/s" else sr["GB/s"]
        result["roofline"]["frac_of_calibrated"] = round(achieved / ceiling, 4)

    # ---- CPU baseline: the fp64 oracle on a bounded sample of the timed workload ----
    if not args.no_cpu and head not in DECODE and head not in BACKWARD:
        result["cpu_baseline"] = cpu_baseline(w, rl)

    line = json.dumps(result)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


def host_info():
    """CPU model and the cores this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cores_available": len(os.sched_getaffinity(0))}


def cpu_baseline(w, rl):
    """The fp64 numpy oracle, untuned, on whole (batch, head) pairs of the workload until
    about 10 s of CPU time have been spent; reported in the metric's unit."""
    import oracle.fa_oracle as orc
    from threadpoolctl import threadpool_info
    q, k, v = (t.float().numpy() for t in (w.q, w.k, w.v))
    paged = getattr(w, "block_table", None) is not None
    B, H = q.shape[:2]
    g = H // k.shape[1]
    heads = 0
    t0 = time.perf_counter()
    if paged:   # the oracle's own gather, one sequence at a time, inside the timing
        g = H // k.shape[2]
    kb = None
    for bh in range(B * H):
        b, h = divmod(bh, H)
        if paged:
            if h == 0:
                bt = w.block_table.numpy()[b:b + 1]
                kb = orc.gather_pages(k, bt, w.n_k, w.page_size)[0]
                vb = orc.gather_pages(v, bt, w.n_k, w.page_size)[0]
            orc.attention_head(q[b, h], kb[h // g], vb[h // g], w.scale, w.causal)
        else:
            orc.attention_head(q[b, h], k[b, h // g], v[b, h // g], w.scale, w.causal)
        heads += 1
        if time.perf_counter() - t0 > 10.0:
            break
    el = time.perf_counter() - t0
    s = w.shape
    if paged:
        fl = rl.chunked_prefill_flops(1, heads, s["T"], s["N_k"], s["d"], w.causal)
    else:
        fl = rl.prefill_flops(1, heads, s["N_q"], s["N_k"], s["d"], w.causal)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(fl / el / 1e12, 6), "unit": "TFLOP/s",
            "cores": min(threads, len(os.sched_getaffinity(0))), "kind": "oracle",
            "sample": f"fp64 numpy oracle on {heads} of {B * H} (batch, head) pairs of {w.name}, "
                      f"all rows each, {el:.1f} s; same FLOP convention"}


def load_traffic(workload_name, fabuild):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current sources of that kernel (else None)."""
    path = os.path.join(HERE, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    kind = t.get("kernel_family")
    if kind is None or t.get("kernel_hash") != fabuild.kernel_hash(kind):
        return None
    return t.get("traffic_bytes_per_launch")


if __name__ == "__main__":
    main()
