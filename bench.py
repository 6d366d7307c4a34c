#!/usr/bin/env python3
"""Benchmark of the SegPaged hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input, all inputs
resident in HBM before the timed region:
  rope_relocate    every reused segment key, offline -> online position
                   (out of place, so every step does identical work)
  segpaged_prefill the new-token chunk of every (layer, KV head) slot, one call
  segpaged_decode  one decode token per sequence over every slot
The page tables are built once beforehand by segpaged_build_tables on the
host; its time is reported separately (build_tables_ms).

Work counted is algorithmic only:
  prefill FLOPs = 4 * head_dim per (query row, visible key) pair;
  prefill bytes = K and V of every page in each head's table, read once
                  (the chunk's queries share them) + q/out;
  relocate bytes = 2 * (valid segment-key elements) * elem + 16 B per list item;
  decode bytes  = per slot, visible keys * 2 * head_dim * elem (K and V read
                  once, shared by the group's heads) + q/out + table entries.
Visible counts are read back from the HIP path itself with zero queries
(every weight is then exactly 1, so exp(LSE) is the count).

The reported value is the whole step's share of the MI355X roofline:
100 * (max(prefill FLOPs / 2.5 PFLOP/s, prefill bytes / 8 TB/s)
       + (relocate + decode bytes) / 8 TB/s) / step time.
(A 64-token chunk over a shared KV page does 4 * 256 rows FLOPs per 4 bytes
of K and V: about 256 FLOP/B, below the chip's 312 FLOP/B ridge, so the
prefill of such a chunk is bound by HBM, not by the matrix cores.)
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "segpaged prefill TFLOP/s + decode/relocate GB/s at 32K & 128K, % of roofline"
PEAK_BF16_FLOPS = 2.5e15
PEAK_FP32_FLOPS = 157.3e12
PEAK_HBM = 8.0e12
WORKLOAD_TEXT = {
    "32k": "32K RAG: 8 layers x 8 KV heads (64 slots), 32 q-heads/8 KV (G=4), head_dim 128, bf16, page 16; "
           "6 reused segments x 5000 tokens (offline base 0) + 64-token question + 1 decode token; "
           "10 global / 54 local (window 256) slots; K scaled 0.5",
    "128k": "128K microbench: 64 slots, G=4, head_dim 128, bf16, page 32; one 129024-token reused segment shifted "
            "+4096, 2048-token prefill chunk + 1 decode token; 58 local (window 1024) / 6 global",
    "16k": "16K 4x4K: 64 slots, G=8, head_dim 128, bf16, page 16; 4 x 4096 segments + 128-token suffix + 1 decode; "
           "58 local (512) / 3 global / 2 retrieval (64 pages) / 1 dense",
    "batch": "serving mix: 32 sequences 8K-64K, 64 slots, G=8, head_dim 128, bf16, page 16; 256 new tokens + 1 "
             "decode per sequence; 55 local (256) / 6 global / 3 retrieval (32 pages)",
    "tiny": "tiny fp32 layer: 4 slots (MHA), head_dim 64, page 16, 2 x 256 segments + 32-token suffix + 1 decode",
    "recovery32k": "head-level recovery prefill: the 10 global slots of the 32K workload (G=4, head_dim 128, bf16, "
                   "page 16) recomputed in full, 30000 context tokens as one causal query chunk + 1 decode token",
}
from head_aware_paged_page_amd.profiling import source_hash  # noqa: E402


def committed_traffic(call: str, workload: str):
    """HBM bytes per launch from a committed PMC summary, if it was taken on the current kernel source."""
    for path in glob.glob(os.path.join(ROOT, "profiles", f"*{call}*{workload}*pmc*.json")):
        try:
            d = json.load(open(path))
        except (OSError, ValueError):
            continue
        if d.get("source_hash") == source_hash(call) and d.get("workload") == workload:
            return d.get("hbm_bytes_per_launch")
    return None


def algorithmic_work(w, torch):
    """Visible counts from the HIP path with zero queries, then FLOPs / bytes."""
    import numpy as np
    lay = w.lay
    esz = 4 if lay.dtype == "f32" else 2
    zq = torch.zeros_like(w.q_prefill)
    zd = torch.zeros_like(w.q_decode)
    _, lp = w.prefill(q=zq, out=torch.empty_like(zq), lse=torch.empty_like(w.lse_prefill))
    _, ld = w.decode(q=zd, out=torch.empty_like(zd), lse=torch.empty_like(w.lse_decode))
    torch.cuda.synchronize()
    cnt_p = np.rint(np.exp(lp.double().cpu().numpy())).astype(np.int64)
    cnt_d = np.rint(np.exp(ld.double().cpu().numpy())).astype(np.int64)
    D = lay.head_dim
    prefill_flops = int(cnt_p.sum()) * 4 * D
    per_slot = cnt_d[:, ::lay.group]                       # one head per slot: K/V read once per slot
    decode_bytes = int(per_slot.sum()) * 2 * D * esz + 2 * w.q_decode.numel() * esz + 16 * len(w.td["entries"])
    ent_p, rp = w.tp["entries"], w.tp["row_ptr"]
    table_keys = int(ent_p[:, 2].sum())
    prefill_bytes = table_keys * 2 * D * esz + 2 * w.q_prefill.numel() * esz + 16 * len(ent_p)
    reloc = w.tp["reloc"]
    reloc_bytes = 2 * int(reloc[:, 2].sum()) * D * esz + 16 * len(reloc)
    return dict(prefill_flops=prefill_flops, prefill_bytes=prefill_bytes, decode_bytes=decode_bytes,
                relocate_bytes=reloc_bytes,
                prefill_pairs=int(cnt_p.sum()), decode_keys=int(per_slot.sum()))


def cpu_baseline(w, work_budget_s: float):
    """The fp64 oracle on a bounded sample of the same workload, one core."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attention as oatt
    from oracle import rope as orope

    lay = w.lay
    D, G = lay.head_dim, lay.group
    rows_g = [s * lay.n_seq for s in range(lay.n_slot) if lay.cls[s] != 1]
    rows_l = [s * lay.n_seq for s in range(lay.n_slot) if lay.cls[s] == 1]
    order = [r for pair in zip(rows_g, rows_l) for r in pair] + rows_g[len(rows_l):] + rows_l[len(rows_g):]
    flops = 0
    pbytes = 0
    rbytes = 0
    dbytes = 0
    t_used = 0.0
    ent_p, rp = w.tp["entries"], w.tp["row_ptr"]
    n_rows = 0
    esz = 4 if lay.dtype == "f32" else 2
    with threadpool_limits(1):
        for r in order:
            slot, seq = divmod(r, lay.n_seq)
            K, V = w.unit_host(slot, seq)
            heads = slice(slot * G, (slot + 1) * G)
            qp = w.q_prefill[w.h_tok_ptr[seq]:w.h_tok_ptr[seq + 1], heads].double().cpu().numpy()
            qd = w.q_decode[seq:seq + 1, heads].double().cpu().numpy()
            ctx = lay.ctx_len(seq)
            on = np.concatenate([np.arange(o, o + l) for o, l in zip(lay.seg_online[seq], lay.seg_len[seq])])
            off = np.concatenate([np.arange(o, o + l) for o, l in zip(lay.seg_offline[seq], lay.seg_len[seq])])
            t0 = time.perf_counter()
            K[:ctx] = orope.relocate(K[:ctx], off, on, lay.theta)
            q_pos = lay.new_base[seq] + np.arange(lay.n_prefill)
            _, _, cnt = oatt.row_attention(lay, slot, seq, K, V, qp, q_pos)
            _, _, cd = oatt.row_attention(lay, slot, seq, K, V, qd, [lay.new_base[seq] + lay.n_prefill])
            t_used += time.perf_counter() - t0
            n_rows += 1
            flops += int(cnt.sum()) * G * 4 * D
            pbytes += int(ent_p[rp[r]:rp[r + 1], 2].sum()) * 2 * D * esz
            rbytes += 2 * ctx * D * esz
            dbytes += int(cd.sum()) * 2 * D * esz
            if t_used >= work_budget_s:
                break
    t_roof = max(flops / PEAK_BF16_FLOPS, pbytes / PEAK_HBM) + (rbytes + dbytes) / PEAK_HBM
    return {"value": 100.0 * t_roof / t_used, "unit": "% of roofline", "cores": 1, "kind": "oracle",
            "sample": f"{n_rows} of {lay.n_slot * lay.n_seq} (slot, seq) rows of the same workload, alternating "
                      f"global/local: fp64 relocation of their segment keys, prefill of all {lay.n_prefill} "
                      f"query tokens and the decode token; {t_used:.1f} s on 1 core; oracle prefill "
                      f"{flops / t_used / 1e9:.2f} GFLOP/s, relocation {rbytes / t_used / 1e9:.3f} GB/s",
            "seconds": round(t_used, 2)}


class HipEvent:
    """A HIP timing event recorded on a given stream.

    Created with hipEventDisableSystemFence: recording it then adds no
    system-scope memory fence between the kernels it separates.  torch's
    events keep that fence, which on this step added about 13 us (5 %) of
    stall per step across its four records; these add about 5 us.
    """
    _hip = None
    FLAGS = 0x20000000    # hipEventDisableSystemFence (hip_runtime_api.h); timing stays on

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            HipEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._ct = ctypes
        self.e = ctypes.c_void_p()
        rc = HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.e), ctypes.c_uint(self.FLAGS))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = HipEvent._hip.hipEventRecord(self.e, self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    @staticmethod
    def elapsed_ms(a: "HipEvent", b: "HipEvent") -> float:
        f = a._ct.c_float()
        rc = HipEvent._hip.hipEventElapsedTime(a._ct.byref(f), a.e, b.e)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def __del__(self):
        if HipEvent._hip is not None and self.e:
            HipEvent._hip.hipEventDestroy(self.e)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="32k", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the hot path runs on a single MI355X and has no "
              "multi-GPU mode (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from head_aware_paged_page_amd.workload import Workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lay = synth.make_layout(args.config, seed=args.seed)
    print(f"[bench] building workload {args.config} ...", file=sys.stderr, flush=True)
    w = Workload(lay, device="cuda")
    t0 = time.perf_counter()
    reps = 5
    for _ in range(reps):
        import head_aware_paged_page_amd.segpaged as sp
        sp.build_tables(**w.arr_p, page_size=w.ps, free_list=w.free)
    build_ms = (time.perf_counter() - t0) / reps * 1e3
    work = algorithmic_work(w, torch)
    print(f"[bench] work: {work}", file=sys.stderr, flush=True)

    def step():
        w.relocate()
        w.prefill(k=w.k_reloc)
        w.decode(k=w.k_reloc)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[HipEvent() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        e = ev[i]
        e[0].record(stream)
        w.relocate()
        e[1].record(stream)
        w.prefill(k=w.k_reloc)
        e[2].record(stream)
        w.decode(k=w.k_reloc)
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms = lambda a, b: sum(HipEvent.elapsed_ms(ev[i][a], ev[i][b]) for i in range(args.steps)) / args.steps
    t_reloc, t_pref, t_dec = (max(ms(a, a + 1), 1e-6) for a in range(3))   # an empty call may time as 0
    ms_per_step = wall / args.steps * 1e3

    peak_flops = PEAK_FP32_FLOPS if lay.dtype == "f32" else PEAK_BF16_FLOPS
    t_pref_roof = max(work["prefill_flops"] / peak_flops, work["prefill_bytes"] / PEAK_HBM)
    pref_bound = "mfma" if work["prefill_flops"] / peak_flops >= work["prefill_bytes"] / PEAK_HBM else "hbm"
    calls = {
        "rope_relocate": {"ms": round(t_reloc, 4), "GB/s": round(work["relocate_bytes"] / t_reloc / 1e6, 1),
                          "frac_hbm": round(work["relocate_bytes"] / t_reloc / 1e-3 / PEAK_HBM, 4),
                          "bytes": work["relocate_bytes"]},
        "segpaged_prefill": {"ms": round(t_pref, 4), "TFLOP/s": round(work["prefill_flops"] / t_pref / 1e9, 2),
                             "frac_mfma": round(work["prefill_flops"] / t_pref / 1e-3 / peak_flops, 4),
                             "GB/s": round(work["prefill_bytes"] / t_pref / 1e6, 1),
                             "frac_hbm": round(work["prefill_bytes"] / t_pref / 1e-3 / PEAK_HBM, 4),
                             "flops": work["prefill_flops"], "bytes": work["prefill_bytes"],
                             "bound": pref_bound},
        "segpaged_decode": {"ms": round(t_dec, 4), "GB/s": round(work["decode_bytes"] / t_dec / 1e6, 1),
                            "frac_hbm": round(work["decode_bytes"] / t_dec / 1e-3 / PEAK_HBM, 4),
                            "bytes": work["decode_bytes"]},
        "segpaged_build_tables": {"host_ms": round(build_ms, 3), "outside_timed_step": True},
    }
    t_roof = t_pref_roof + (work["relocate_bytes"] + work["decode_bytes"]) / PEAK_HBM
    value = 100.0 * t_roof / (ms_per_step * 1e-3)

    times = {"rope_relocate": t_reloc, "segpaged_prefill": t_pref, "segpaged_decode": t_dec}
    dom = max(times, key=times.get)
    if dom == "segpaged_prefill" and pref_bound == "mfma":
        ach = work["prefill_flops"] / (t_pref * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_flops / 1e12, "unit": "TFLOP/s",
                "frac": round(ach * 1e12 / peak_flops, 4)}
    else:
        b = {"rope_relocate": work["relocate_bytes"], "segpaged_decode": work["decode_bytes"],
             "segpaged_prefill": work["prefill_bytes"]}[dom]
        ach = b / (times[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "frac": round(ach * 1e9 / PEAK_HBM, 4)}
    roof["kernel"] = dom
    roof["traffic"] = committed_traffic(dom, args.config)

    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "% of roofline", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if lay.dtype == "f32" else "bf16", "data": "synthetic",
        "config": {"workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}", "seed": args.seed,
                   "slots": lay.n_slot, "sequences": lay.n_seq, "prefill_tokens": int(w.h_tok_ptr[-1]),
                   "decode_tokens": lay.n_seq},
        "roofline": roof,
        "calls": calls,
    }
    # A row beyond the step, measured on its own: the per-head visible-page
    # pack (the pages the decode tables list, gathered in table order), not
    # part of the step or its value.  Bytes: every listed K and V page read
    # once and written once.
    import head_aware_paged_page_amd.segpaged as sp
    n_ent = int(w.td["row_ptr"][-1])
    k_pk = torch.empty((n_ent,) + tuple(w.k_pool.shape[1:]), dtype=w.k_pool.dtype, device="cuda")
    v_pk = torch.empty((n_ent,) + tuple(w.v_pool.shape[1:]), dtype=w.v_pool.dtype, device="cuda")
    for _ in range(3):
        sp.pack_pages(w.k_pool, w.v_pool, w.d_entries, n_ent, k_pk, v_pk)
    torch.cuda.synchronize()
    pe = [HipEvent() for _ in range(2)]
    reps = 20
    pe[0].record(stream)
    for _ in range(reps):
        sp.pack_pages(w.k_pool, w.v_pool, w.d_entries, n_ent, k_pk, v_pk)
    pe[1].record(stream)
    torch.cuda.synchronize()
    t_pack = HipEvent.elapsed_ms(pe[0], pe[1]) / reps
    pack_bytes = 2 * (k_pk.numel() + v_pk.numel()) * k_pk.element_size()
    res["beyond_step"] = {"pack_pages": {"ms": round(t_pack, 4), "GB/s": round(pack_bytes / t_pack / 1e6, 1),
                                         "frac_hbm": round(pack_bytes / t_pack / 1e-3 / PEAK_HBM, 4),
                                         "bytes": pack_bytes, "pages": n_ent}}
    if not args.no_cpu_baseline and lay.n_prefill > 4096:
        # one row of the fp64 oracle over every query of such a chunk runs for minutes
        res["cpu_baseline"] = None
        res["cpu_baseline_note"] = "skipped: the oracle cannot finish one row of this chunk in a bounded sample"
    elif not args.no_cpu_baseline:
        print("[bench] timing the oracle on a CPU sample ...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
