"""rocprofv3 passes over bench.py and the summaries kept under profiles/.

    python -m online_softmax_07_amd.profiling --workload long_prefill_8192 [--workload ...]
        [--raw gpurun_out/prof] [--summaries gpurun_out/prof/summaries] [--steps 20] [--warmup 5]
        [--variant br128 --passes trace,fetch,write]
    python -m online_softmax_07_amd.profiling --next3-table      # measured vs modelled bytes

For each workload this runs bench.py (timing that workload only) as a child process under
rocprofv3, once per pass:

* ``trace``: ``--kernel-trace --stats`` with the given steps and warm-up calls (by default
  the driver's: 5 warm-up calls, 20 timed ones) -- per-kernel durations, whose mean over
  the timed dispatches must agree with bench.py's own HIP-event mean of the same process;
* ``fetch`` / ``write``: ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` (KiB per dispatch)
  with a plain 1 GiB device copy in the same process (``--calib-copy``), whose readings
  scale the counters to bytes;
* ``mfma`` (prefill and backward only): ``--pmc MfmaUtil MfmaFlopsBF16
  SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE`` -- the fraction of cycles the matrix cores
  are busy and the bf16 MFMA operations actually executed (units of 512 FLOP, converted),
  to compare with the algorithmic FLOPs.

Each pass runs under its own time limit; the first failing pass stops everything.  This
process never touches the GPU itself (rocprofv3 must start the profiled program directly).
The summaries written are ``<workload name>.txt`` (trace and MFMA counters) and
``traffic_<workload name>.json`` (HBM bytes, with the hash of the kernel sources they were
measured on, which bench.py checks before reporting them).
"""

from __future__ import annotations

import argparse
import collections
import glob
import json
import os
import sqlite3
import subprocess
import sys

from . import build as fb
from . import roofline as rl

ROOT = fb.ROOT

# workload (bench.py name) -> (summary name, title, kernel-name prefixes, family, algorithmic bytes, FLOPs)
def _cases():
    c = {}
    n8, d = 8192, 128
    c["long_prefill_8192"] = (
        "long_prefill_b1_h32_n8192_d128_causal_heavy1pct",
        "fa_fwd, bf16, B=1 H=32 N=8192 d=128 causal, 1% of key rows x8",
        ["_ZN2fa15fwd_bf16_kernel"], "prefill",
        rl.prefill_bytes_floor(1, 32, 32, n8, n8, d), rl.prefill_flops(1, 32, n8, n8, d, True))
    for dd in (128, 64):
        for causal in (True, False):
            key = f"prefill_d{dd}_{'causal' if causal else 'full'}"
            c[key] = (f"prefill_b4_h16_n4096_d{dd}_{'causal' if causal else 'full'}",
                      f"fa_fwd, bf16, B=4 H=16 N=4096 d={dd} {'causal' if causal else 'non-causal'}",
                      ["_ZN2fa15fwd_bf16_kernel"], "prefill",
                      rl.prefill_bytes_floor(4, 16, 16, 4096, 4096, dd), rl.prefill_flops(4, 16, 4096, 4096, dd, causal))
    c["chunked_prefill_paged"] = (
        "chunked_prefill_paged_b4_hq32_hkv8_q2048_ctx8192_p16",
        "fa_fwd_paged, bf16, B=4 H_q=32 H_kv=8, 2048-token chunk over 8192 positions, d=128, 16-token pages, causal",
        ["_ZN2fa15fwd_bf16_kernel"], "prefill",
        rl.prefill_bytes_floor(4, 32, 8, 2048, 8192, d) + 4 * 4 * 512,
        rl.chunked_prefill_flops(4, 32, 2048, 8192, d, True))
    c["backward"] = (
        "backward_b4_h16_n4096_d128_causal",
        "fa_bwd, bf16, B=4 H=16 N=4096 d=128 causal (dQ, dK, dV from the saved O and LSE)",
        ["void fa::bwd_prep_kernel", "_ZN2fa13bwd_dq_kernel", "_ZN2fa15bwd_dkdv_kernel"], "backward",
        8 * (4 * 16 * 4096 * 128 * 2) + 4 * 16 * 4096 * 4, 2.5 * rl.prefill_flops(4, 16, 4096, 4096, d, True))
    c["decode_splitkv_128k"] = (
        "decode_splitkv_b1_hq32_hkv8_s131072",
        "fa_decode_splitkv, B=1 H_q=32 H_kv=8 S=131072 d=128, automatic split count",
        ["_ZN2fa19decode_split_kernel", "_ZN2fa16lse_merge_kernel"], "decode",
        rl.decode_bytes(1, 32, 8, 1, 131072, d), rl.decode_flops(1, 32, 1, 131072, d))
    c["decode_paged_b64"] = (
        "decode_paged_b64_hq8_hkv1_ctx8192_p16",
        "fa_decode_splitkv paged, B=64 H_q=8 H_kv=1 ctx 8192, 16-token pages, automatic split count",
        ["_ZN2fa19decode_split_kernel", "_ZN2fa16lse_merge_kernel"], "decode",
        rl.decode_bytes(64, 8, 1, 1, 8192, d, 512), rl.decode_flops(64, 8, 1, 8192, d))
    return c


CASES = _cases()
MFMA_COUNTERS = ["MfmaUtil", "MfmaFlopsBF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]


def _db(path_prefix):
    hits = sorted(glob.glob(os.path.join(path_prefix, "**", "*results.db"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no rocprofv3 database under {path_prefix}")
    return sqlite3.connect(hits[-1])


def dispatches(db_dir, prefixes):
    """[(name, start, end, duration_ns, vgpr, agpr, sgpr, lds)] of the matching kernels, in dispatch order."""
    con = _db(db_dir)
    rows = con.execute("select name, start, end, duration, vgpr_count, accum_vgpr_count, sgpr_count, lds_size "
                       "from kernels order by start").fetchall()
    return [r for r in rows if any(r[0].startswith(p) for p in prefixes)]


def top_kernels(db_dir):
    con = _db(db_dir)
    return con.execute("select name, total_calls, total_duration, average, percentage from top_kernels").fetchall()


def counters_per_dispatch(db_dir):
    """{(kernel name, counter): [value summed over the dimension instances, per dispatch]}"""
    con = _db(db_dir)
    acc = collections.defaultdict(float)
    names = {}
    for disp, name, cn, v in con.execute("select dispatch_id, kernel_name, counter_name, value from counters_collection"):
        acc[(disp, cn)] += float(v)
        names[disp] = name
    out = collections.defaultdict(list)
    for (disp, cn), v in sorted(acc.items()):
        out[(names[disp], cn)].append(v)
    return out


def copy_reference(db_dir, counter):
    """The counter's mean over the 1 GiB copies of --calib-copy: the copy dispatches with
    the largest grid (small copies, such as reading a result back, also run as copy kernels)."""
    con = _db(db_dir)
    acc = collections.defaultdict(float)
    grid = {}
    for disp, name, cn, v, g in con.execute(
            "select dispatch_id, kernel_name, counter_name, value, grid_size from counters_collection"):
        if name.startswith("__amd_rocclr_copyBuffer") and cn == counter:
            acc[disp] += float(v)
            grid[disp] = int(g)
    gmax = max(grid.values())
    vals = [v for d, v in acc.items() if grid[d] == gmax]
    return sum(vals) / len(vals)


def mean_counter(per, prefixes, counter):
    vals = [v for (n, c), vs in per.items() if c == counter and any(n.startswith(p) for p in prefixes) for v in vs]
    return sum(vals) / len(vals) if vals else None


def sum_of_means(per, prefixes, counter):
    """Per call: the mean over dispatches of each kernel family member, summed over the members."""
    tot = 0.0
    for p in prefixes:
        m = mean_counter(per, [p], counter)
        if m is None:
            return None
        tot += m
    return tot


def _bench_cmd(workload, steps, warmup, extra=()):
    return ["python3", os.path.join(ROOT, "bench.py"), "--workload", workload, "--no-extra", "--no-cpu", "--no-calib",
            "--steps", str(steps), "--warmup", str(warmup), *extra]


def _run(cmd, log, limit, env=None):
    print("+", " ".join(cmd), flush=True)
    with open(log, "w") as f:
        r = subprocess.run(["timeout", "-s", "KILL", str(limit), *cmd], stdout=f, stderr=subprocess.STDOUT,
                           cwd="/tmp", env={**(env or os.environ), "TMPDIR": "/tmp"})
    if r.returncode != 0:
        with open(log) as f:
            tail = f.read()[-3000:]
        print(tail, flush=True)
        # rocprofv3 may end with a segmentation fault after a complete run; accept that only
        # when the profiled program printed its JSON line
        if not (r.returncode in (139, -11) and '"metric"' in tail):
            raise SystemExit(f"pass failed (exit {r.returncode}): {' '.join(cmd)}")
    print(f"  done: {log}", flush=True)


def _last_json(path):
    line = None
    with open(path) as f:
        for l in f:
            if l.startswith("{"):
                line = l
    return json.loads(line) if line else None


def profile(workload, raw, summaries, steps, warmup, limit=240, run=True, variant=None,
            passes=("trace", "fetch", "write", "mfma")):
    name, title, prefixes, family, alg_bytes, flops = CASES[workload]
    env = None
    defines = []
    if variant is not None:
        lib = fb.variant_lib(variant)
        defines = fb.VARIANTS[variant]
        env = {**os.environ, "FA_MI355X_LIB": lib}
        name = f"next3_{variant}_{name}"
        title = f"{title}; build variant {variant} ({' '.join('-D' + d for d in defines)})"
        workload_dir = f"{variant}_{workload}"
    else:
        workload_dir = workload
    base = os.path.join(raw, workload_dir)
    os.makedirs(base, exist_ok=True)
    os.makedirs(summaries, exist_ok=True)
    rel = os.path.relpath
    cmds = {}

    # trace
    tdir = os.path.join(base, "trace")
    tjson = os.path.join(base, "trace.json")
    cmds["trace"] = ["rocprofv3", "--kernel-trace", "--stats", "-d", tdir, "-o", "t", "--",
                     *_bench_cmd(workload, steps, warmup, ["--out", tjson])]
    if run:
        _run(cmds["trace"], os.path.join(base, "trace.log"), limit, env)
    # counters
    for key, pmc in (("fetch", ["FETCH_SIZE"]), ("write", ["WRITE_SIZE"]),
                     *((("mfma", MFMA_COUNTERS),) if family in ("prefill", "backward") and "mfma" in passes else ())):
        cmds[key] = ["rocprofv3", "--pmc", *pmc, "-d", os.path.join(base, key), "-o", "t", "--",
                     *_bench_cmd(workload, 3, 1, ["--calib-copy"] if key in ("fetch", "write") else [])]
        if run:
            _run(cmds[key], os.path.join(base, key + ".log"), limit, env)

    def show(cmd):
        text = " ".join(rel(c, ROOT) if c.startswith(ROOT) else c for c in cmd)
        return (f"FA_MI355X_LIB={rel(fb.variant_lib(variant), ROOT)} " + text) if variant else text

    # ---- trace summary ----
    bench = _last_json(tjson)
    disp = dispatches(tdir, prefixes)
    # the members of the family this call path launched (the decode's merge kernel runs only
    # when the split kernel does not merge by itself)
    prefixes = [p for p in prefixes if any(r[0].startswith(p) for r in disp)]
    n_timed = bench["steps"]
    per_call = len(prefixes)
    timed = disp[-n_timed * per_call:]
    timed_us = sum(r[3] for r in timed) / 1e3 / n_timed
    all_us = sum(r[3] for r in disp) / 1e3 / (len(disp) / per_call)
    peak = rl.PEAK_HBM_GBPS if family == "decode" else rl.PEAK_BF16_MFMA_TFLOPS
    unit = "GB/s" if family == "decode" else "TFLOP/s"
    work = alg_bytes if family == "decode" else flops
    scale = 1e9 if family == "decode" else 1e12
    lines = [f"# {title}", "",
             "Produced by (from the repository root, one MI355X):", "",
             f"    python -m online_softmax_07_amd.profiling --workload {workload} --steps {steps} --warmup {warmup}"
             + (f" --variant {variant} --passes {','.join(passes)}" if variant else ""),
             "", "which runs, each as its own process:", ""]
    lines += [f"    {show(c)}" for c in cmds.values()]
    lines += ["", f"## Kernel trace ({bench['warmup']} warm-up calls, then {n_timed} timed calls)", "",
              "rocprofv3 --stats (every dispatch of the process; microseconds):", "",
              "| kernel | calls | total_us | average_us | % |", "|---|---|---|---|---|"]
    for n, c, t, a, p in top_kernels(tdir):
        lines.append(f"| `{n[:110]}` | {c} | {float(t):.1f} | {float(a):.2f} | {float(p):.1f} |")
    r0 = disp[-1]
    # rocprofv3's kernel record lists half the vector registers a wave is given on this chip
    # (arch_vgpr_count = (VGPR + AGPR allocation) / 2, accum_vgpr_count 0): e.g. 128 for the
    # d=128 forward, which the compiler gives 256 VGPRs
    lines += ["", f"Registers of `{r0[0][:60]}...`: {2 * int(r0[4]) + int(r0[5])} vector registers per lane "
              f"(VGPR and AGPR together; rocprofv3's kernel record: arch_vgpr_count {r0[4]}, accum_vgpr_count "
              f"{r0[5]}), {r0[6]} SGPR; LDS {r0[7]} B.", "",
              f"- Mean duration per call over the {n_timed} timed calls (the last {n_timed * per_call} matching "
              f"dispatches): **{timed_us:.2f} us** -> {work / (timed_us * 1e-6) / scale:.1f} {unit}, "
              f"frac {work / (timed_us * 1e-6) / scale / peak:.4f} of {peak:g}.",
              f"- Mean over all {len(disp) // per_call} calls (warm-up included): {all_us:.2f} us.",
              f"- bench.py in the same process (HIP events on the launch stream): mean launch "
              f"{bench['roofline']['avg_launch_us']} us, roofline frac {bench['roofline']['frac']}, value "
              f"{bench['value']} {bench['unit']} over the bracketed timed calls; shader clock "
              f"{bench.get('gpu_clock_mhz')} MHz."]
    if family != "decode":
        lines.append(f"- Work per call: {flops:.6g} FLOP (4 N_q N_k d per head, halved for causal"
                     f"{'; backward 2.5x the forward' if family == 'backward' else ''}).")
    # ---- traffic ----
    pf = counters_per_dispatch(os.path.join(base, "fetch"))
    pw = counters_per_dispatch(os.path.join(base, "write"))
    cf = copy_reference(os.path.join(base, "fetch"), "FETCH_SIZE")
    cw = copy_reference(os.path.join(base, "write"), "WRITE_SIZE")
    kf = sum_of_means(pf, prefixes, "FETCH_SIZE")
    kw = sum_of_means(pw, prefixes, "WRITE_SIZE")
    ff, wf = (1 << 20) / cf, (1 << 20) / cw
    traffic = kf * ff * 1024 + kw * wf * 1024
    t = {"workload": name, "kernels": prefixes, "kernel_family": family, "kernel_hash": fb.kernel_hash(family),
         "kernel_sources": fb.KERNEL_SOURCES[family],
         "fetch_kib_per_call_raw": round(kf, 1), "write_kib_per_call_raw": round(kw, 1),
         "copy_reference": {"bytes_read": 1 << 30, "bytes_written": 1 << 30, "fetch_kib_raw": round(cf, 1),
                            "write_kib_raw": round(cw, 1)},
         "fetch_scale": ff, "write_scale": wf,
         "traffic_bytes_per_launch": round(traffic), "algorithmic_bytes_per_launch": round(alg_bytes),
         "traffic_over_algorithmic": round(traffic / alg_bytes, 4),
         "variant": variant, "defines": defines, "mean_launch_us": round(timed_us, 2),
         "commands": [show(cmds["fetch"]), show(cmds["write"])]}
    with open(os.path.join(summaries, f"traffic_{name}.json"), "w") as f:
        json.dump(t, f, indent=1)
    lines += ["", "## HBM traffic (rocprofv3 --pmc, copy-calibrated)", "",
              f"- FETCH_SIZE {kf:.1f} KiB and WRITE_SIZE {kw:.1f} KiB per call; a 1 GiB device copy in the same "
              f"process reads FETCH {cf:.1f} KiB, WRITE {cw:.1f} KiB, so the scale factors are {ff:.4f} and {wf:.4f}.",
              f"- Traffic {traffic / 1e6:.1f} MB per call against {alg_bytes / 1e6:.1f} MB algorithmic "
              f"({traffic / alg_bytes:.3f} x).  Stored in `traffic_{name}.json`."]
    # ---- MFMA counters ----
    if "mfma" in cmds:
        pm = counters_per_dispatch(os.path.join(base, "mfma"))
        lines += ["", "## Matrix cores (rocprofv3 --pmc " + " ".join(MFMA_COUNTERS) + ")", "",
                  "| kernel | MfmaUtil % | executed bf16 MFMA FLOP | SQ_VALU_MFMA_BUSY_CYCLES | GRBM_GUI_ACTIVE |",
                  "|---|---|---|---|---|"]
        exe_total = 0.0
        for p in prefixes:
            util = mean_counter(pm, [p], "MfmaUtil")
            fl = mean_counter(pm, [p], "MfmaFlopsBF16")
            busy = mean_counter(pm, [p], "SQ_VALU_MFMA_BUSY_CYCLES")
            gui = mean_counter(pm, [p], "GRBM_GUI_ACTIVE")
            exe_total += fl or 0.0
            lines.append(f"| `{p}` | {util:.1f} | {fl:.6g} | {busy:.6g} | {gui:.6g} |")
        lines += ["", f"- Executed bf16 MFMA work per call {exe_total:.6g} FLOP against {flops:.6g} algorithmic: "
                      f"{exe_total / flops:.3f} x (the excess is masked work on the causal diagonal tiles, padding "
                      f"and, in the backward, the recomputed products)."]
    with open(os.path.join(summaries, f"{name}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {name}.txt and traffic_{name}.json: {timed_us:.2f} us/call, traffic {traffic / alg_bytes:.3f} x",
          flush=True)


NEXT3_WORKLOADS = {   # bench name -> (B, H, N, d, causal)
    "prefill_d128_causal": (4, 16, 4096, 128, True),
    "prefill_d128_full": (4, 16, 4096, 128, False),
    "long_prefill_8192": (1, 32, 8192, 128, True),
}
NEXT3_BR = {None: 256, "br256_plain": 256, "br128": 128, "br64": 64}


def next3_table(profiles_dir) -> str:
    """Markdown table of measured against modelled HBM bytes per prefill launch, from the
    committed traffic summaries of the shipped build and its variants: the no-reuse model of
    page "Softmax and FlashAttention" ("Maths"), counted per query block (exact under the
    causal mask), and the every-value-once floor."""
    rows = ["| variant | Br | workload | model, no reuse (MB) | measured (MB) | floor (MB) | measured / floor | "
            "mean launch (us) | TFLOP/s |", "|---|---|---|---|---|---|---|---|---|"]
    for variant, br in NEXT3_BR.items():
        for wl, (B, H, N, d, causal) in NEXT3_WORKLOADS.items():
            name = CASES[wl][0] if variant is None else f"next3_{variant}_{CASES[wl][0]}"
            path = os.path.join(profiles_dir, f"traffic_{name}.json")
            if not os.path.exists(path):
                continue
            with open(path) as f:
                t = json.load(f)
            model = B * H * rl.flash_bytes_model(N, N, d, br, causal)
            floor = rl.prefill_bytes_floor(B, H, H, N, N, d)
            meas = t["traffic_bytes_per_launch"]
            us = t.get("mean_launch_us")
            tf = f"{rl.prefill_flops(B, H, N, N, d, causal) / (us * 1e-6) / 1e12:.0f}" if us else "-"
            label = "shipped (XCD order)" if variant is None else (
                "plain blockIdx order" if variant.endswith("plain") else "XCD order")
            rows.append(f"| {variant or 'br256'}: {label} | {br} | {CASES[wl][0]} | {model / 1e6:.1f} | "
                        f"{meas / 1e6:.1f} | {floor / 1e6:.1f} | {meas / floor:.2f} | {us if us else '-'} | {tf} |")
    return "\n".join(rows)


def main():
    if "--next3-table" in sys.argv:
        print(next3_table(os.path.join(ROOT, "profiles")))
        return 0
    p = argparse.ArgumentParser()
    p.add_argument("--workload", action="append", required=True, choices=sorted(CASES))
    p.add_argument("--raw", default=os.path.join(ROOT, "gpurun_out", "prof"))
    p.add_argument("--summaries", default=os.path.join(ROOT, "gpurun_out", "prof", "summaries"))
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--summarize-only", action="store_true",
                   help="write the summaries from the results already under --raw (no profiling run)")
    p.add_argument("--variant", choices=sorted(fb.VARIANTS), default=None,
                   help="profile a build variant (python -m online_softmax_07_amd.build --variants)")
    p.add_argument("--passes", default="trace,fetch,write,mfma")
    a = p.parse_args()
    for w in a.workload:
        profile(w, a.raw, a.summaries, a.steps, a.warmup, run=not a.summarize_only, variant=a.variant,
                passes=tuple(a.passes.split(",")))
    print("profiling done", flush=True)


if __name__ == "__main__":
    sys.exit(main())
