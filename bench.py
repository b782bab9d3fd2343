#!/usr/bin/env python3
"""Benchmark of the FlashAttention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

One step is one fa_fwd call on the prefill workload B=4, H_q=H_kv=16, N=4096, d=128,
causal (bottom-right), bf16 in / bf16 O + fp32 LSE out, inputs resident in HBM.  The
headline ``value`` is its attention throughput in TFLOP/s (4 N^2 d per head, halved for
causal).  ``roofline`` prices the prefill kernel's average launch (HIP events on the
launch stream) against the dense bf16 MFMA peak.  ``breakdown`` adds the other prefill
variants, the long causal prefill, and the two decode workloads (HBM GB/s against the
HBM peak, with L2 and the Infinity Cache flushed between timed calls).
``cpu_baseline`` times the fp64 oracle on a bounded sample of the headline workload.
Prints exactly one JSON line.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

METRIC = "attention TFLOP/s + % MFMA peak (prefill); HBM GB/s + % peak (decode), 1 GPU"
HERE = os.path.dirname(os.path.abspath(__file__))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-extra", action="store_true", help="headline workload only (for profiling)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--only", default=None, help="run one breakdown entry as the only timed work")
    p.add_argument("--out", default=None, help="also write the JSON to this file")
    return p.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    sys.path.insert(0, HERE)
    from online_softmax_07_amd import fa, roofline as rl, workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def timed(fn, steps, warmup, pre=None):
        """Per-call durations (ms) from HIP events recorded on the launch stream, and the
        total bracketed time of the K calls."""
        for _ in range(warmup):
            if pre:
                pre()
            fn()
        torch.cuda.synchronize()
        st = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        en = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(steps):
            if pre:
                pre()
            st[i].record(stream)
            fn()
            en[i].record(stream)
        t1.record(stream)
        torch.cuda.synchronize()
        per = [a.elapsed_time(b) for a, b in zip(st, en)]
        return t0.elapsed_time(t1), per

    # ---- prefill workloads ----
    def prefill_case(w):
        q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        s = w.shape
        flops = rl.prefill_flops(s["B"], s["H_q"], s["N_q"], s["N_k"], s["d"], w.causal)

        def fn():
            fa.fa_fwd(q, k, v, o, lse, causal=w.causal, scale=w.scale, stream=stream)
        return fn, flops, (q, k, v, o, lse)

    # ---- headline: prefill B=4 H=16 N=4096 d=128 causal ----
    head_w = workloads.prefill_4x16x4096(128, True)
    fn, flops, bufs = prefill_case(head_w)
    total_ms, per = timed(fn, args.steps, args.warmup)
    ms_per_step = total_ms / args.steps
    avg_launch_ms = statistics.mean(per)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    s = head_w.shape
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: iid N(0,1) rounded to bf16, seed 201",
        "config": {"workload": head_w.name, "B": s["B"], "H_q": s["H_q"], "H_kv": s["H_kv"],
                   "N_q": s["N_q"], "N_k": s["N_k"], "d": s["d"], "causal": True,
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": rl.PEAK_BF16_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / rl.PEAK_BF16_MFMA_TFLOPS, 4),
                     "traffic": None, "kernel": "fa::fwd_bf16_kernel<128, 64, true, bf16>",
                     "avg_launch_us": round(avg_launch_ms * 1e3, 2)},
    }
    del bufs

    # ---- breakdown ----
    breakdown = {}
    if not args.no_extra:
        for d, causal in [(64, False), (64, True), (128, False)]:
            w = workloads.prefill_4x16x4096(d, causal)
            fn, fl, bufs = prefill_case(w)
            _, per = timed(fn, max(10, args.steps // 2), 3)
            med = statistics.median(per)
            breakdown[w.name] = {"us": round(med * 1e3, 2), "TFLOP/s": round(fl / med / 1e9, 2),
                                 "frac_mfma": round(fl / med / 1e9 / rl.PEAK_BF16_MFMA_TFLOPS, 4)}
            del bufs
        w = workloads.long_prefill_8192()
        fn, fl, bufs = prefill_case(w)
        _, per = timed(fn, max(10, args.steps // 2), 3)
        med = statistics.median(per)
        breakdown[w.name] = {"us": round(med * 1e3, 2), "TFLOP/s": round(fl / med / 1e9, 2),
                             "frac_mfma": round(fl / med / 1e9 / rl.PEAK_BF16_MFMA_TFLOPS, 4)}
        del bufs

        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)   # 1 GiB: evicts L2 and MALL

        def pre():
            flush.fill_(1)

        for w in (workloads.decode_splitkv_128k(), workloads.decode_paged_b64()):
            q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
            bt = None if w.block_table is None else w.block_table.to(dev)
            o = torch.empty_like(q)
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
            sh = w.shape
            pps = 0 if bt is None else bt.shape[1]
            nbytes = rl.decode_bytes(sh["B"], sh["H_q"], sh["H_kv"], sh["T"], sh["N_k"], sh["d"], pps)
            entry = {"bytes": nbytes, "by_num_splits": {}}
            best = None
            for ns in list(w.num_splits) + [0]:
                wsb = fa.fa_decode_workspace_bytes(sh["B"], sh["H_q"], sh["H_kv"], sh["T"], sh["N_k"], sh["d"], ns)
                ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

                def fn(ns=ns, ws=ws):
                    fa.fa_decode_splitkv(q, k, v, o, lse, causal=w.causal, scale=w.scale, num_splits=ns,
                                         block_table=bt, n_k=w.n_k, workspace=ws, check_table=False,
                                         stream=stream)
                _, per = timed(fn, 30, 3, pre=pre)
                med = statistics.median(per)
                gbs = nbytes / (med * 1e-3) / 1e9
                key = "auto" if ns == 0 else str(ns)
                entry["by_num_splits"][key] = {"us": round(med * 1e3, 2), "min_us": round(min(per) * 1e3, 2),
                                               "GB/s": round(gbs, 1),
                                               "frac_hbm": round(gbs / rl.PEAK_HBM_GBPS, 4)}
                if best is None or gbs > best[1]:
                    best = (key, gbs)
            entry["best"] = {"num_splits": best[0], "GB/s": round(best[1], 1),
                             "frac_hbm": round(best[1] / rl.PEAK_HBM_GBPS, 4)}
            breakdown[w.name] = entry
            del q, k, v, bt, o, lse
        del flush
        result["breakdown"] = breakdown

    # ---- CPU baseline: the fp64 oracle on a bounded sample of the headline workload ----
    if not args.no_cpu:
        import oracle.fa_oracle as orc
        from threadpoolctl import threadpool_info
        q = head_w.q.float().numpy()
        k = head_w.k.float().numpy()
        v = head_w.v.float().numpy()
        heads = 0
        t0 = time.perf_counter()
        B, H = q.shape[:2]
        for bh in range(B * H):
            b, h = divmod(bh, H)
            orc.attention_head(q[b, h], k[b, h], v[b, h], head_w.scale, True)
            heads += 1
            if time.perf_counter() - t0 > 10.0:
                break
        el = time.perf_counter() - t0
        fl = rl.prefill_flops(1, heads, s["N_q"], s["N_k"], s["d"], True)
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        result["cpu_baseline"] = {
            "value": round(fl / el / 1e12, 6), "unit": "TFLOP/s",
            "cores": min(threads, len(os.sched_getaffinity(0))), "kind": "oracle",
            "sample": f"fp64 numpy oracle on {heads} of {B * H} (batch, head) pairs, all 4096 rows each, "
                      f"{el:.1f} s; same FLOP convention",
        }

    line = json.dumps(result)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
