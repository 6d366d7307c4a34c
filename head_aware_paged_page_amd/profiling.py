"""rocprofv3 helpers for the committed kernel summaries.

Two uses:

  python -m head_aware_paged_page_amd.profiling copy --mib 1024
      runs one plain device-to-device copy of a known size (warm-up + 4 timed
      copies), the calibration kernel for the FETCH_SIZE / WRITE_SIZE counters;

  python -m head_aware_paged_page_amd.profiling summarize --workload 32k \\
      --trace DIR --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \\
      --copy-mib 1024 --out profiles
      turns rocprofv3 CSV output (kernel trace + stats, and the counter runs)
      into the text summaries and the per-kernel HBM-traffic records that
      bench.py reports as roofline.traffic.

Counters: FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch.  Each is
divided by what the same counter reads for the calibration copy per byte it
actually moves, so the scaled figure is in true bytes.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# kernel-name fragment -> (call it belongs to, short name)
KERNELS = [
    ("relocate_kernel", "rope_relocate", "relocate_kernel"),
    ("prefill_bf16_kernel", "segpaged_prefill", "prefill_bf16_kernel"),
    ("prefill_merge_kernel", "segpaged_prefill", "prefill_merge_kernel"),
    ("plan_kernel", "segpaged_prefill", "plan_kernel"),
    ("decode_bf16_kernel", "segpaged_decode", "decode_bf16_kernel"),
    ("decode_merge_kernel", "segpaged_decode", "decode_merge_kernel"),
    ("prefill_f32_kernel", "segpaged_prefill", "prefill_f32_kernel"),
    ("decode_f32_kernel", "segpaged_decode", "decode_f32_kernel"),
    ("page_copy_kernel", "segpaged_pack_pages", "page_copy_kernel"),
    ("importance_bf16_kernel", "segpaged_token_importance", "importance_bf16_kernel"),
    ("importance_reduce_kernel", "segpaged_token_importance", "importance_reduce_kernel"),
    ("importance_plan_kernel", "segpaged_token_importance", "importance_plan_kernel"),
    ("fill_zero_kernel", "segpaged_token_importance", "fill_zero_kernel"),
    ("importance_f32_kernel", "segpaged_token_importance", "importance_f32_kernel"),
    ("layer_score_kernel", "segpaged_select_tokens", "layer_score_kernel"),
    ("select_kernel", "segpaged_select_tokens", "select_kernel"),
]
# The sources a call's kernel timings and traffic depend on: its kernels and the
# host runtime, whose planner sets split counts and launch shapes.
KERNEL_SOURCES = {
    "rope_relocate": ["relocate.hip", "device_common.hpp", "runtime.cpp", "internal.hpp"],
    "segpaged_prefill": ["prefill.hip", "device_common.hpp", "runtime.cpp", "internal.hpp"],
    "segpaged_decode": ["decode.hip", "device_common.hpp", "runtime.cpp", "internal.hpp"],
    "segpaged_pack_pages": ["pack.hip", "device_common.hpp", "runtime.cpp", "internal.hpp"],
    "segpaged_token_importance": ["importance.hip", "device_common.hpp", "runtime.cpp", "internal.hpp"],
    "segpaged_select_tokens": ["importance.hip", "device_common.hpp", "runtime.cpp", "internal.hpp"],
}


def source_hash(call: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[call]:
        with open(os.path.join(ROOT, "head_aware_paged_page_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(name: str):
    # the longest matching fragment wins (importance_plan_kernel also contains plan_kernel)
    best = None
    for frag, call, short in KERNELS:
        if frag in name and (best is None or len(frag) > len(best[0])):
            best = (frag, call, short)
    return (best[1], best[2]) if best else (None, None)


def copy_main(mib: int) -> None:
    import torch
    n = mib * (1 << 20) // 2
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_()
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n * 2, "copies": 5}), flush=True)


def read_counters(d: str):
    """Average counter value per dispatch, per kernel name."""
    path = os.path.join(d, "run_counter_collection.csv")
    acc = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(path)):
        acc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = {}
    for k, cs in acc.items():
        out[k] = {c: sum(v) / len(v) for c, v in cs.items()}
    return out


def calib_factor(d: str, counter: str, copy_bytes: int) -> float:
    """Counter KiB per true KiB for the biggest dispatch of the calibration run."""
    vals = [v[counter] for v in read_counters(d).values() if counter in v]
    best = max(vals)
    return best / (copy_bytes / 1024.0)


def summarize(a) -> None:
    copy_bytes = a.copy_mib * (1 << 20)
    f_fetch = calib_factor(a.copy_fetch, "FETCH_SIZE", copy_bytes)
    f_write = calib_factor(a.copy_write, "WRITE_SIZE", copy_bytes)
    fetch = read_counters(a.fetch)
    write = read_counters(a.write)
    stats = list(csv.DictReader(open(os.path.join(a.trace, "run_kernel_stats.csv"))))
    bench_cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
                 f"python3 bench.py --config {a.workload} --steps 10 --warmup 2 --no-cpu-baseline --no-128k --no-window --no-layers")
    pmc_cmd = ("rocprofv3 --pmc {c} --output-format csv -d <dir> -o run -- "
               f"python3 bench.py --config {a.workload} --steps 2 --warmup 1 --no-cpu-baseline --no-128k --no-window --no-layers")
    copy_cmd = ("rocprofv3 --pmc {c} --output-format csv -d <dir> -o run -- "
                f"python3 -m head_aware_paged_page_amd.profiling copy --mib {a.copy_mib}")
    lines = [f"# Kernel time, workload {a.workload} (rocprofv3 kernel trace, --stats)", "",
             "command (from the repository root, on one MI355X):", f"  {bench_cmd}", "",
             "The run holds the warm-up (2 steps, then untimed steps until 0.3 s have passed), the zero-query", "pass that counts visible keys, and 10 timed steps; the averages cover every call.", "",
             f"{'kernel':28s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}"]
    by_short = {}
    for r in stats:
        call, short = short_name(r["Name"])
        if not short:
            continue
        by_short[short] = dict(call=call, calls=int(r["Calls"]), avg_us=float(r["AverageNs"]) / 1e3,
                               min_us=float(r["MinNs"]) / 1e3, max_us=float(r["MaxNs"]) / 1e3)
        lines.append(f"{short:28s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f}")
    lines += ["", f"# HBM traffic per dispatch (FETCH_SIZE, WRITE_SIZE; separate runs)", "",
              "commands:", "  " + pmc_cmd.format(c="FETCH_SIZE"), "  " + pmc_cmd.format(c="WRITE_SIZE"),
              "  calibration: " + copy_cmd.format(c="FETCH_SIZE"), "  calibration: " + copy_cmd.format(c="WRITE_SIZE"),
              "",
              f"calibration copy of {a.copy_mib} MiB each way: FETCH_SIZE reads {f_fetch:.4f} KiB per KiB moved, "
              f"WRITE_SIZE {f_write:.4f}; the figures below are divided by these factors.", "",
              f"{'kernel':28s} {'fetch_MB':>10s} {'write_MB':>10s} {'total_MB':>10s}"]
    traffic = {}
    for name in set(fetch) | set(write):
        call, short = short_name(name)
        if not short:
            continue
        fb = fetch.get(name, {}).get("FETCH_SIZE", 0.0) * 1024 / f_fetch
        wb = write.get(name, {}).get("WRITE_SIZE", 0.0) * 1024 / f_write
        traffic[short] = dict(call=call, fetch_bytes=fb, write_bytes=wb)
    for short in sorted(traffic):
        t = traffic[short]
        lines.append(f"{short:28s} {t['fetch_bytes'] / 1e6:10.2f} {t['write_bytes'] / 1e6:10.2f} "
                     f"{(t['fetch_bytes'] + t['write_bytes']) / 1e6:10.2f}")
    os.makedirs(a.out, exist_ok=True)
    txt = os.path.join(a.out, f"kernels_{a.workload}.txt")
    open(txt, "w").write("\n".join(lines) + "\n")
    # one traffic record per call's dominant kernel, keyed by the call's source hash
    main_kernel = {"rope_relocate": "relocate_kernel", "segpaged_prefill": "prefill_bf16_kernel",
                   "segpaged_decode": "decode_bf16_kernel", "segpaged_pack_pages": "page_copy_kernel",
                   "segpaged_token_importance": "importance_bf16_kernel"}
    for call, short in main_kernel.items():
        if short not in traffic:
            continue
        t = traffic[short]
        rec = {"call": call, "kernel": short, "workload": a.workload, "source_hash": source_hash(call),
               "hbm_bytes_per_launch": round(t["fetch_bytes"] + t["write_bytes"]),
               "fetch_bytes_per_launch": round(t["fetch_bytes"]), "write_bytes_per_launch": round(t["write_bytes"]),
               "calibration": {"copy_mib": a.copy_mib, "fetch_factor": f_fetch, "write_factor": f_write},
               "avg_us": by_short.get(short, {}).get("avg_us"),
               "commands": [pmc_cmd.format(c="FETCH_SIZE"), pmc_cmd.format(c="WRITE_SIZE"),
                            copy_cmd.format(c="FETCH_SIZE"), copy_cmd.format(c="WRITE_SIZE")]}
        json.dump(rec, open(os.path.join(a.out, f"{call}_{a.workload}_pmc.json"), "w"), indent=1)
    print(open(txt).read())


# Hardware counter passes for the instruction mix and pipe activity of the
# step's kernels (one rocprofv3 --pmc run each: at most 8 SQ counters a pass).
COUNTER_PASSES = [
    "GRBM_GUI_ACTIVE SQ_WAVE_CYCLES SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU "
    "SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_SCA SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_ANY",
    "GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_VALU_TRANS_F32 "
    "SQ_WAIT_INST_LDS SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_SMEM",
]


def counters(a) -> None:
    """Per-dispatch averages of the counter passes for the step's main kernels,
    with the kernel durations of the same runs (--kernel-trace), into
    profiles/counters_<workload>.txt."""
    cmd = ("timeout -s KILL 120 rocprofv3 --kernel-trace --pmc {c} --output-format csv -d <dir> -o run -- "
           f"python3 bench.py --config {a.workload} --steps 2 --warmup 1 --no-cpu-baseline --no-128k --no-window --no-layers")
    vals, durs = defaultdict(dict), defaultdict(list)
    for d in a.passes:
        for name, cs in read_counters(d).items():
            _, short = short_name(name)
            if short:
                vals[short].update(cs)
        kt = os.path.join(d, "run_kernel_trace.csv")
        if os.path.exists(kt):
            for r in csv.DictReader(open(kt)):
                _, short = short_name(r["Kernel_Name"])
                if short:
                    durs[short].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# Hardware counters per dispatch, workload {a.workload}", "",
             "commands (from the repository root, on one MI355X; one pass each):"]
    lines += ["  " + cmd.format(c=f'"{c}"') for c in COUNTER_PASSES]
    lines += ["", "Averages over every dispatch of the runs (warm-up, settle and timed calls).  SQ counters",
              "aggregate all SIMDs, GRBM_GUI_ACTIVE sums the 8 XCDs (divided by a dispatch's duration",
              "it gives 8 times the clock).  Derived, per dispatch, with cycles = GRBM_GUI_ACTIVE / 8:",
              "  clock = cycles / duration (median duration of the same runs' kernel trace);",
              "  mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles * 1024 SIMDs);",
              "  cu_busy = SQ_BUSY_CU_CYCLES / (cycles * 256 CUs);",
              "  valu / lds / salu share = SQ_ACTIVE_INST_{VALU,LDS,SCA} / SQ_WAVE_CYCLES (wave time",
              "  spent issuing or executing each kind); wait share = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES;",
              "  coexec = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES (matrix-busy cycles with",
              "  vector work alongside); per MFMA = instruction counts divided by SQ_INSTS_MFMA.",
              "The counting window of a dispatch is somewhat longer than the kernel: for dispatches of",
              "under about 100 us the clock reads high and the busy fractions low; the instruction",
              "counts and ratios are exact.", ""]
    for short in ("prefill_bf16_kernel", "decode_bf16_kernel", "relocate_kernel", "importance_bf16_kernel"):
        if short not in vals:
            continue
        v = vals[short]
        lines.append(f"## {short}")
        for k in sorted(v):
            lines.append(f"  {k:32s} {v[k]:18.1f}")
        g = v.get("GRBM_GUI_ACTIVE", 0.0) / 8           # one XCD's cycles
        wc = v.get("SQ_WAVE_CYCLES", 0.0)
        mf = v.get("SQ_INSTS_MFMA", 0.0)
        dur = sorted(durs[short])[len(durs[short]) // 2] if durs.get(short) else None
        der = []
        if dur and g:
            der.append(f"clock {g / dur / 1e3:.2f} GHz (median duration {dur:.1f} us)")
        if g:
            der.append(f"mfma_busy {v.get('SQ_VALU_MFMA_BUSY_CYCLES', 0.0) / (g * 1024):.3f}")
            der.append(f"cu_busy {v.get('SQ_BUSY_CU_CYCLES', 0.0) / (g * 256):.3f}")
        if v.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            der.append(f"coexec {v.get('SQ_VALU_MFMA_COEXEC_CYCLES', 0.0) / v['SQ_VALU_MFMA_BUSY_CYCLES']:.3f}")
        if wc:
            for name, key in (("valu", "SQ_ACTIVE_INST_VALU"), ("lds", "SQ_ACTIVE_INST_LDS"),
                              ("salu", "SQ_ACTIVE_INST_SCA"), ("wait", "SQ_WAIT_INST_ANY")):
                if key in v:
                    der.append(f"{name} share {v[key] / wc:.3f}")
        if mf:
            for name, key in (("valu", "SQ_INSTS_VALU"), ("trans", "SQ_INSTS_VALU_TRANS_F32"),
                              ("salu", "SQ_INSTS_SALU"), ("lds", "SQ_INSTS_LDS"), ("smem", "SQ_INSTS_SMEM")):
                if key in v:
                    der.append(f"{name} per MFMA {v[key] / mf:.2f}")
        lines += ["  derived: " + "; ".join(der), ""]
    os.makedirs(a.out, exist_ok=True)
    txt = os.path.join(a.out, f"counters_{a.workload}.txt")
    open(txt, "w").write("\n".join(lines) + "\n")
    print(open(txt).read())


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    s = sub.add_parser("summarize")
    s.add_argument("--workload", required=True)
    for k in ("trace", "fetch", "write", "copy-fetch", "copy-write"):
        s.add_argument(f"--{k}", required=True)
    s.add_argument("--copy-mib", type=int, default=1024)
    s.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    k = sub.add_parser("counters")
    k.add_argument("--workload", required=True)
    k.add_argument("--passes", nargs="+", required=True, help="one rocprofv3 output directory per counter pass")
    k.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args(argv)
    if a.cmd == "copy":
        copy_main(a.mib)
    elif a.cmd == "counters":
        counters(a)
    else:
        summarize(a)


if __name__ == "__main__":
    main(sys.argv[1:])
