#!/usr/bin/env python3
"""Benchmark of the SegPaged hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input, all inputs
resident in HBM before the timed region:
  rope_relocate    every reused segment key, offline -> online position, in
                   place in the pool (as a server rotates the cached keys it
                   reuses); a replica's successive uses rotate by +delta and
                   -delta in turn, so its keys keep their values and every
                   step does identical work
  segpaged_prefill the new-token chunk of every (layer, KV head) slot, one call
  segpaged_decode  one decode token per sequence over every slot
The page tables are built once beforehand by segpaged_build_tables on the
host; its time is reported separately (build_tables), as is the host-side
launch planning inside each prefill and decode call (plan_host_ms).  Before
the K timed steps: W warm-up steps, then untimed steps until 0.3 s have
passed (settle_steps), so that timing starts from a busy GPU's clocks; the
timed steps follow the last settle step without a pause.  Each timed step
records three HIP events on the call stream (after relocate, prefill and
decode; the step before it ends where it starts), which time the calls.

Cache-clean timing.  The chip's last-level cache (256 MB) could serve a call
data that the previous call just read (decode reads the global slots' pages
prefill read a moment before).  So the pools exist in R identical replicas and
step i runs relocate on replica i mod R, prefill on replica (i+1) mod R and
decode on replica (i+2) mod R: with R >= 3 and R replicas of at least 1 GB
together, the prefill and decode of other replicas (allocating reads of some
300 MB at 32K) and a relocation pass lie between two calls that touch the
same replica.  (The relocation's non-temporal traffic alone does not evict the
cache: a decode that rereads one replica with only relocations in between
runs about 12 % faster.)  A workload whose pools are too large for three copies runs
with R = 1; its calls each move several GB.

Work counted is algorithmic only, from the host tables (never from the GPU):
  prefill FLOPs = 4 * head_dim per (query row, visible key) pair;
  prefill bytes = K and V of every page in each head's table, read once
                  (the chunk's queries share them) + q/out + table entries;
  relocate bytes = 2 * (valid segment-key elements) * elem + 16 B per list item;
  decode bytes  = per slot, visible keys * 2 * head_dim * elem (K and V read
                  once, shared by the group's heads) + q/out + table entries.
A key of a table entry (pos_start, n_valid) is visible to a query at position
p when its position is <= p and, for a local slot of window W, > p - W.

The reported value is the whole step's share of the MI355X roofline:
100 * (max(prefill FLOPs / 2.5 PFLOP/s, prefill bytes / 8 TB/s)
       + (relocate + decode bytes) / 8 TB/s) / step time.
(A 64-token chunk over a shared KV page does 4 * 256 rows FLOPs per 4 bytes
of K and V: about 256 FLOP/B, below the chip's 312 FLOP/B ridge, so the
prefill of such a chunk is bound by HBM, not by the matrix cores.)

With the default workload (32K) the same line also carries the 128K
microbenchmark, measured the same way, under "config_128k", the same
workload with window-only storage (every head stores only the pages its
queries can read) under "window_only", with the KV bytes one session holds,
and its prefill and decode issued as one call per layer (8 calls of the
layer's 8 KV heads each, as a model runs them) under "per_layer".
"""
from __future__ import annotations

import argparse
import gc
import glob
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "segpaged prefill TFLOP/s + decode/relocate GB/s at 32K & 128K, % of roofline"
PEAK_BF16_FLOPS = 2.5e15
PEAK_FP32_FLOPS = 157.3e12
PEAK_HBM = 8.0e12
LOCAL = 1
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
MAX_REPLICA_BYTES = 24 << 30     # pools of all replicas together
MIN_ROTATION_BYTES = 1 << 30     # replicas together at least this large (4x the last-level cache)
MAX_REPLICAS = 16                # (a workload of a few MB, the tiny one, stops here)
MAX_CPU_QUERIES = 128            # query tokens per row the oracle baseline runs (evenly spaced)
# After the W warm-up steps, untimed steps go on until this much wall time has
# passed: an idle MI355X runs its first tens of milliseconds of matrix work at
# a lower engine clock (about 1.9 GHz against 2.4 for matrix work alone), so
# the timed steps start from the clocks of a GPU that has been busy.
CLOCK_SETTLE_S = 0.3
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


# ----------------------------------------------------------------------------- algorithmic work

def table_visible_counts(row_ptr, entries, cls, window, n_seq, q_pos_of_seq):
    """Visible keys of each query of each row, from the row's table alone.

    Row r = slot * n_seq + seq; entries[:, 1:3] = (pos_start, n_valid) in
    ascending position.  Returns a list over rows of int64 arrays, one count per
    position in q_pos_of_seq[seq]: the table's keys at positions <= p, less
    (local slots) those at positions <= p - W."""
    out = []
    for r in range(len(row_ptr) - 1):
        slot, seq = divmod(r, n_seq)
        e = np.asarray(entries[row_ptr[r]:row_ptr[r + 1]], np.int64)
        s, n = e[:, 1], e[:, 2]
        before = np.concatenate([[0], np.cumsum(n)])

        def upto(x):
            i = np.searchsorted(s, x, side="right") - 1
            j = np.maximum(i, 0)
            return np.where(i >= 0, before[j] + np.minimum(n[j], x - s[j] + 1), 0)

        p = np.asarray(q_pos_of_seq[seq], np.int64)
        c = upto(p)
        if int(cls[slot]) == LOCAL:
            c = c - upto(p - int(window[slot]))
        out.append(c)
    return out


def algorithmic_work(w):
    lay = w.lay
    esz = 4 if lay.dtype == "f32" else 2
    D, G = lay.head_dim, lay.group
    q_pos = [lay.new_base[s] + np.arange(lay.n_prefill) for s in range(lay.n_seq)]
    d_pos = [np.asarray([lay.new_base[s] + lay.n_prefill]) for s in range(lay.n_seq)]
    cp = table_visible_counts(w.tp["row_ptr"], w.tp["entries"], lay.cls, lay.window, lay.n_seq, q_pos)
    cd = table_visible_counts(w.td["row_ptr"], w.td["entries"], lay.cls, lay.window, lay.n_seq, d_pos)
    pairs = int(sum(int(c.sum()) for c in cp)) * G
    dkeys = int(sum(int(c.sum()) for c in cd))
    ent_p = w.tp["entries"]
    prefill_bytes = int(ent_p[:, 2].sum()) * 2 * D * esz + 2 * w.q_prefill.numel() * esz + 16 * len(ent_p)
    decode_bytes = dkeys * 2 * D * esz + 2 * w.q_decode.numel() * esz + 16 * len(w.td["entries"])
    reloc = w.tp["reloc"]
    reloc_bytes = 2 * int(reloc[:, 2].sum()) * D * esz + 16 * len(reloc)
    return dict(prefill_flops=pairs * 4 * D, prefill_bytes=prefill_bytes, decode_bytes=decode_bytes,
                relocate_bytes=reloc_bytes, prefill_pairs=pairs, decode_keys=dkeys)


# ----------------------------------------------------------------------------- CPU baseline (the oracle)

_LAYOUTS = {}


def _cpu_task(args):
    """One (slot, seq) row of the workload through the fp64 oracle: relocation of
    its segment keys, prefill of every chunk token, the decode token.  Inputs are
    the row's seeded values drawn by the CPU generator (the same streams and
    distributions as the GPU's, other draws); only the oracle's work is timed."""
    import torch
    from threadpoolctl import threadpool_limits
    from oracle import attention as oatt
    from oracle import rope as orope
    import synth

    name, seed, r = args
    if name not in _LAYOUTS:
        _LAYOUTS[name] = synth.make_layout(name, seed=seed)
    lay = _LAYOUTS[name]
    slot, seq = divmod(r, lay.n_seq)
    G, D = lay.group, lay.head_dim
    u = synth.unit_values(lay, slot, seq, device="cpu")
    K = torch.cat([u["seg_k"], u["new_k"]]).double().numpy()
    V = torch.cat([u["seg_v"], u["new_v"]]).double().numpy()
    q = synth.seq_queries(lay, seq, device="cpu")[:, slot * G:(slot + 1) * G].double().numpy()
    ctx = lay.ctx_len(seq)
    on = np.concatenate([np.arange(o, o + l) for o, l in zip(lay.seg_online[seq], lay.seg_len[seq])] + [[]])
    off = np.concatenate([np.arange(o, o + l) for o, l in zip(lay.seg_offline[seq], lay.seg_len[seq])] + [[]])
    with threadpool_limits(1):
        t0 = time.perf_counter()
        K[:ctx] = orope.relocate(K[:ctx], off, on, lay.theta)
        toks = np.unique(np.linspace(0, lay.n_prefill - 1, min(lay.n_prefill, MAX_CPU_QUERIES)).astype(np.int64))
        qp = lay.new_base[seq] + toks
        _, _, cnt = oatt.row_attention(lay, slot, seq, K, V, q[toks], qp)
        _, _, cd = oatt.row_attention(lay, slot, seq, K, V, q[lay.n_prefill:lay.n_prefill + 1],
                                      [lay.new_base[seq] + lay.n_prefill])
        dt = time.perf_counter() - t0
    return dict(row=r, seconds=dt, pid=os.getpid(), pairs=int(cnt.sum()) * G, ctx=ctx, dkeys=int(cd.sum()),
                q_frac=len(toks) / lay.n_prefill)


def cpu_baseline(pool, n_workers, lay, tp, budget_s):
    """The fp64 oracle on a bounded sample of the same workload's rows, over
    n_workers host processes (one BLAS thread each); rows alternate between
    global-like and local slots and are handed out until the summed oracle time
    reaches budget_s per worker.  The value is the work done over the busiest
    worker's oracle time, against the same roofline formula as the GPU.  A
    chunk of more than MAX_CPU_QUERIES tokens runs that many of its queries,
    evenly spaced; its table bytes are charged in proportion."""
    D, G = lay.head_dim, lay.group
    esz = 4 if lay.dtype == "f32" else 2
    rows_g = [s * lay.n_seq + q for s in range(lay.n_slot) if lay.cls[s] != LOCAL for q in range(lay.n_seq)]
    rows_l = [s * lay.n_seq + q for s in range(lay.n_slot) if lay.cls[s] == LOCAL for q in range(lay.n_seq)]
    order = [r for pair in zip(rows_g, rows_l) for r in pair] + rows_g[len(rows_l):] + rows_l[len(rows_g):]
    per_worker, done = {}, []
    it = pool.imap_unordered(_cpu_task, [(lay.name, lay.seed, r) for r in order])
    for res in it:
        done.append(res)
        per_worker[res["pid"]] = per_worker.get(res["pid"], 0.0) + res["seconds"]
        if sum(per_worker.values()) >= budget_s * n_workers:
            break
    pool.terminate()
    span = max(per_worker.values())
    ent, rp = tp["entries"], tp["row_ptr"]
    flops = sum(d["pairs"] for d in done) * 4 * D
    pbytes = sum(int(ent[rp[d["row"]]:rp[d["row"] + 1], 2].sum()) * d["q_frac"] for d in done) * 2 * D * esz
    rbytes = sum(d["ctx"] for d in done) * 2 * D * esz
    dbytes = sum(d["dkeys"] for d in done) * 2 * D * esz
    t_roof = max(flops / PEAK_BF16_FLOPS, pbytes / PEAK_HBM) + (rbytes + dbytes) / PEAK_HBM
    return {"value": 100.0 * t_roof / span, "unit": "% of roofline", "cores": len(per_worker), "kind": "oracle",
            "sample": f"{len(done)} of {lay.n_slot * lay.n_seq} (slot, seq) rows of the same workload, alternating "
                      f"global/local, over {len(per_worker)} processes (one BLAS thread each): fp64 relocation of "
                      f"their segment keys, prefill of {min(lay.n_prefill, MAX_CPU_QUERIES)} of the {lay.n_prefill} query "
                      f"tokens (evenly spaced) and the decode token; "
                      f"row values drawn by the CPU generator from the same seeded streams; busiest process "
                      f"{span:.1f} s of oracle time; oracle prefill {flops / span / 1e9:.2f} GFLOP/s, "
                      f"relocation {rbytes / span / 1e9:.3f} GB/s",
            "seconds": round(span, 2)}


# ----------------------------------------------------------------------------- timing

class HipEvent:
    """A HIP timing event recorded on a given stream.

    Created with hipEventDisableSystemFence: recording it then adds no
    system-scope memory fence between the kernels it separates.  torch's
    events keep that fence, which on this step added about 13 us (5 %) of
    stall per step across four records; these add about 1-1.5 us each.
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
        try:
            if HipEvent._hip is not None and self.e:
                HipEvent._hip.hipEventDestroy(self.e)
        except (AttributeError, TypeError):   # interpreter shutdown: the module is being torn down
            pass


def _pct(xs, q):
    return float(np.percentile(np.asarray(xs), q))


def layer_calls(w, reps, n_rep, steps, warmup, work):
    """The same prefill and decode as one call per layer (the slots of one layer,
    its KV heads, per call), as a model would issue them: n_layers prefill calls,
    then n_layers decode calls, each on its own slice of the queries and tables,
    with its own plan and workspace.  The prefill calls of a step run on one pool
    replica and its decode calls on the next, so consecutive uses of one replica
    are separated by the traffic of two whole passes.  Returns the summed call
    times and the per-layer means, against the same algorithmic work (the sum
    over the layers is the whole call's)."""
    import torch
    import head_aware_paged_page_amd.segpaged as sp

    from synth.configs import CONFIGS

    lay = w.lay
    G, D, ns, ps = lay.group, lay.head_dim, lay.n_seq, w.ps
    spl = CONFIGS[lay.name]["n_kv"]          # a layer's KV heads: slots l * spl .. (l + 1) * spl - 1
    n_layers = lay.n_slot // spl
    code = sp.SP_F32 if lay.dtype == "f32" else sp.SP_BF16
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def sub(tab, l):   # the layer's rows (slots l*spl .. (l+1)*spl - 1, every sequence) of a table
        rp, ent = tab["row_ptr"], tab["entries"]
        r0, r1 = l * spl * ns, (l + 1) * spl * ns
        return (rp[r0:r1 + 1] - rp[r0]).astype(np.int32), np.ascontiguousarray(ent[rp[r0]:rp[r1]], dtype=np.int32)

    layers = []
    for l in range(n_layers):
        heads = slice(l * spl * G, (l + 1) * spl * G)
        rp_p, en_p = sub(w.tp, l)
        rp_d, en_d = sub(w.td, l)
        qp, qd = w.q_prefill[:, heads].contiguous(), w.q_decode[:, heads].contiguous()
        common = dict(page_size=ps, group=G, n_seq=ns, n_slot=spl,
                      d_cls=dev(lay.cls[l * spl:(l + 1) * spl].astype(np.int32)),
                      d_window=dev(lay.window[l * spl:(l + 1) * spl].astype(np.int32)), scale=w.scale)
        pre = dict(common, h_tok_ptr=w.h_tok_ptr, h_row_ptr=rp_p, d_tok_ptr=w.d_tok_ptr, d_q_pos0=w.d_q_pos0,
                   d_row_ptr=dev(rp_p), d_entries=dev(en_p), out=torch.empty_like(qp),
                   lse=torch.empty(qp.shape[:2], dtype=torch.float32, device="cuda"),
                   workspace=torch.empty(sp.workspace_bytes(sp.SP_WS_PREFILL, code, D, ps, G, ns, spl, w.h_tok_ptr,
                                                            rp_p), dtype=torch.uint8, device="cuda"))
        dec = dict(common, h_row_ptr=rp_d, d_q_pos=w.d_q_dec, d_row_ptr=dev(rp_d), d_entries=dev(en_d),
                   out=torch.empty_like(qd), lse=torch.empty(qd.shape[:2], dtype=torch.float32, device="cuda"),
                   workspace=torch.empty(sp.workspace_bytes(sp.SP_WS_DECODE, code, D, ps, G, ns, spl, None, rp_d),
                                         dtype=torch.uint8, device="cuda"))
        layers.append((qp, qd, pre, dec))

    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        b, c = reps[(2 * i) % n_rep], reps[(2 * i + 1) % n_rep]
        for j, (qp, _, pre, _) in enumerate(layers):
            sp.prefill(qp, b[2], b[1], **pre)
            if ev:
                ev[j].record(stream)
        for j, (_, qd, _, dec) in enumerate(layers):
            sp.decode(qd, c[2], c[1], **dec)
            if ev:
                ev[len(layers) + j].record(stream)

    n_l = len(layers)
    ev0 = HipEvent()
    ev = [[HipEvent() for _ in range(2 * n_l)] for _ in range(steps)]
    for i in range(max(warmup, n_rep)):
        step(i)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    marks = [ev0] + [e for row in ev for e in row]
    per_call = np.array([[HipEvent.elapsed_ms(marks[2 * n_l * i + k], marks[2 * n_l * i + k + 1])
                          for k in range(2 * n_l)] for i in range(steps)])     # [steps, 2 * n_layers]
    t_p = float(per_call[:, :n_l].sum(axis=1).mean())
    t_d = float(per_call[:, n_l:].sum(axis=1).mean())
    peak_flops = PEAK_FP32_FLOPS if lay.dtype == "f32" else PEAK_BF16_FLOPS
    n_glob = [int((lay.cls[l * spl:(l + 1) * spl] != LOCAL).sum()) for l in range(n_layers)]
    return {
        "calls_per_step": 2 * n_l, "slots_per_call": spl, "non_local_slots_per_layer": n_glob,
        "segpaged_prefill": {"ms": round(t_p, 4), "TFLOP/s": round(work["prefill_flops"] / t_p / 1e9, 2),
                             "frac_mfma": round(work["prefill_flops"] / t_p / 1e-3 / peak_flops, 4),
                             "per_layer_ms": [round(float(x), 4) for x in per_call[:, :n_l].mean(axis=0)]},
        "segpaged_decode": {"ms": round(t_d, 4), "GB/s": round(work["decode_bytes"] / t_d / 1e6, 1),
                            "frac_hbm": round(work["decode_bytes"] / t_d / 1e-3 / PEAK_HBM, 4),
                            "per_layer_ms": [round(float(x), 4) for x in per_call[:, n_l:].mean(axis=0)]},
        "note": "the step's prefill and decode as one call per layer (8 KV heads each); sums of the calls' times",
    }


def run_config(name, seed, steps, warmup, log, window_only=False, per_layer=False):
    """Build one workload on the GPU and time `steps` steps; returns (result dict, workload).
    window_only: each head stores only the pages its queries can read.
    per_layer: also time the prefill and decode as one call per layer."""
    import torch
    import synth
    import head_aware_paged_page_amd.segpaged as sp
    from head_aware_paged_page_amd.workload import Workload

    lay = synth.make_layout(name, seed=seed)
    t0 = time.perf_counter()
    log(f"building workload {name}{' (window-only storage)' if window_only else ''} ...")
    w = Workload(lay, device="cuda", window_only=window_only)
    # enough replicas that about 1 GB of other traffic separates two uses of one
    n_rep = min(MAX_REPLICAS, max(3, -(-MIN_ROTATION_BYTES // w.pool_bytes())))
    if n_rep * w.pool_bytes() > MAX_REPLICA_BYTES:
        n_rep = 1
    reps = w.replicas(n_rep)
    torch.cuda.synchronize()
    log(f"built in {time.perf_counter() - t0:.1f} s; {n_rep} pool replica(s) of {w.pool_bytes() / 1e9:.2f} GB")

    def host_ms(fn, reps_=5):
        fn()
        t = time.perf_counter()
        for _ in range(reps_):
            fn()
        return (time.perf_counter() - t) / reps_ * 1e3

    build_ms = host_ms(lambda: sp.build_tables_ex(**w.arr_p, page_size=w.ps, free_list=w.free,
                                                  keep_from=w.keep_from))
    code = sp.SP_F32 if lay.dtype == "f32" else sp.SP_BF16
    plan_p = host_ms(lambda: sp.workspace_bytes(sp.SP_WS_PREFILL, code, w.D, w.ps, w.G, w.n_seq, w.n_slot,
                                                w.h_tok_ptr, w.tp["row_ptr"]))
    plan_d = host_ms(lambda: sp.workspace_bytes(sp.SP_WS_DECODE, code, w.D, w.ps, w.G, w.n_seq, w.n_slot, None,
                                                w.td["row_ptr"]))
    work = algorithmic_work(w)
    log(f"work: {work}")

    def calls(i, ev=None):
        # ev: the step's three events, after relocate, prefill and decode; the
        # event before the relocation is the previous step's last (or ev0), so a
        # step records three markers, not four.
        a, b, c = reps[i % n_rep], reps[(i + 1) % n_rep], reps[(i + 2) % n_rep]
        # the replica's keys rotated in place, by +delta and -delta on its
        # successive uses, so its pool keeps its values
        w.relocate(k_in=a[0], k_out=a[0], back=bool(uses[i % n_rep] % 2))
        uses[i % n_rep] += 1
        if ev:
            ev[0].record(stream)
        w.prefill(k=b[2], v=b[1])
        if ev:
            ev[1].record(stream)
        w.decode(k=c[2], v=c[1])
        if ev:
            ev[2].record(stream)

    uses = [0] * n_rep
    stream = torch.cuda.current_stream()
    # Everything the timed loop needs is made, and the garbage collected, before
    # the warm-up: a pause between the settle phase and the timed steps (a full
    # collection takes tens of ms) lets the clocks drop again.
    ev0 = HipEvent()
    ev = [[HipEvent() for _ in range(3)] for _ in range(steps)]
    gc.collect()
    gc.disable()          # a collection inside the timed loop would stall the launches
    t_warm = time.perf_counter()
    for i in range(max(warmup, n_rep)):
        calls(i)
    torch.cuda.synchronize()
    n_settle = 0
    while time.perf_counter() - t_warm < CLOCK_SETTLE_S:
        for _ in range(8):
            calls(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        calls(i, ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gc.enable()
    log(f"warm-up: {max(warmup, n_rep)} steps, then {n_settle} more until {CLOCK_SETTLE_S} s had passed")
    marks = [ev0] + [e for step_ev in ev for e in step_ev]      # 3 * steps + 1, in stream order
    per = [[max(HipEvent.elapsed_ms(marks[3 * i + a], marks[3 * i + a + 1]), 1e-6) for i in range(steps)]
           for a in range(3)]
    t_reloc, t_pref, t_dec = (sum(x) / steps for x in per)
    ms_per_step = wall / steps * 1e3

    peak_flops = PEAK_FP32_FLOPS if lay.dtype == "f32" else PEAK_BF16_FLOPS
    t_pref_roof = max(work["prefill_flops"] / peak_flops, work["prefill_bytes"] / PEAK_HBM)
    pref_bound = "mfma" if work["prefill_flops"] / peak_flops >= work["prefill_bytes"] / PEAK_HBM else "hbm"

    def spread(x):
        return {"p10_ms": round(_pct(x, 10), 4), "p90_ms": round(_pct(x, 90), 4)}

    calls_out = {
        "rope_relocate": {"ms": round(t_reloc, 4), **spread(per[0]),
                          "GB/s": round(work["relocate_bytes"] / t_reloc / 1e6, 1),
                          "frac_hbm": round(work["relocate_bytes"] / t_reloc / 1e-3 / PEAK_HBM, 4),
                          "bytes": work["relocate_bytes"]},
        "segpaged_prefill": {"ms": round(t_pref, 4), **spread(per[1]),
                             "TFLOP/s": round(work["prefill_flops"] / t_pref / 1e9, 2),
                             "frac_mfma": round(work["prefill_flops"] / t_pref / 1e-3 / peak_flops, 4),
                             "GB/s": round(work["prefill_bytes"] / t_pref / 1e6, 1),
                             "frac_hbm": round(work["prefill_bytes"] / t_pref / 1e-3 / PEAK_HBM, 4),
                             "flops": work["prefill_flops"], "bytes": work["prefill_bytes"],
                             "bound": pref_bound, "plan_host_ms": round(plan_p, 3)},
        "segpaged_decode": {"ms": round(t_dec, 4), **spread(per[2]),
                            "GB/s": round(work["decode_bytes"] / t_dec / 1e6, 1),
                            "frac_hbm": round(work["decode_bytes"] / t_dec / 1e-3 / PEAK_HBM, 4),
                            "bytes": work["decode_bytes"], "plan_host_ms": round(plan_d, 3)},
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
    roof["traffic"] = committed_traffic(dom, name)

    # A row beyond the step, measured on its own: the per-head visible-page
    # pack (the pages the decode tables list, gathered in table order), not
    # part of the step or its value, cycled over the replicas like the step.
    n_ent = int(w.td["row_ptr"][-1])
    k_pk = torch.empty((n_ent,) + tuple(w.k_pool.shape[1:]), dtype=w.k_pool.dtype, device="cuda")
    v_pk = torch.empty((n_ent,) + tuple(w.v_pool.shape[1:]), dtype=w.v_pool.dtype, device="cuda")
    pack_bytes = 2 * (k_pk.numel() + v_pk.numel()) * k_pk.element_size()
    n_pack = max(n_rep, 1)
    for i in range(3):
        sp.pack_pages(reps[i % n_pack][0], reps[i % n_pack][1], w.d_entries, n_ent, k_pk, v_pk)
    torch.cuda.synchronize()
    pe = [HipEvent() for _ in range(2)]
    n_calls = 21
    pe[0].record(stream)
    for i in range(n_calls):
        sp.pack_pages(reps[i % n_pack][0], reps[i % n_pack][1], w.d_entries, n_ent, k_pk, v_pk)
    pe[1].record(stream)
    torch.cuda.synchronize()
    t_pack = HipEvent.elapsed_ms(pe[0], pe[1]) / n_calls
    del k_pk, v_pk

    per_layer_out = None
    if per_layer:
        log("timing the prefill and decode as one call per layer ...")
        per_layer_out = layer_calls(w, reps, n_rep, steps, warmup, work)

    # Rows beyond the step: attention importance of the reused segment
    # positions for the chunk's queries (against the prefill's lse), and the
    # selection of a quarter of them per layer for the FFN.  Importance work:
    # 2 * head_dim FLOPs per visible (query row, key) pair (the scores; one
    # exp each), K of every table page read once, q and lse read, one fp32
    # written per slot and position; selection reads the slots' importances and
    # writes the layer scores.
    beyond_imp = None
    if lay.dtype == "bf16" and lay.n_slot % 8 == 0:
        w.prefill(k=reps[0][2], v=reps[0][1])
        lse = w.lse_prefill.clone()
        imp, pos_ptr = w.importance(lse=lse, k=reps[0][2], span="segments")
        n_layers, spl = lay.n_slot // 8, 8
        n_pos = int(pos_ptr[-1])
        ks = [int(pos_ptr[q + 1] - pos_ptr[q]) // 4 for q in range(lay.n_seq)]
        sel_ptr = np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)
        score = torch.empty((n_layers, n_pos), dtype=torch.float32, device="cuda")
        sel = torch.empty((n_layers, max(1, int(sel_ptr[-1]))), dtype=torch.int32, device="cuda")
        d_pos, d_sel = torch.from_numpy(pos_ptr).cuda(), torch.from_numpy(sel_ptr).cuda()

        def select():
            sp.select_tokens(imp, n_layers=n_layers, slots_per_layer=spl, n_seq=lay.n_seq, h_pos_ptr=pos_ptr,
                             d_pos_ptr=d_pos, h_sel_ptr=sel_ptr, d_sel_ptr=d_sel, score=score, sel=sel)
        ie = [HipEvent() for _ in range(3)]
        n_imp = max(n_rep, 6)
        torch.cuda.synchronize()
        ie[0].record(stream)
        for i in range(n_imp):
            w.importance(lse=lse, k=reps[i % n_rep][2], out=(imp, pos_ptr))
        ie[1].record(stream)
        for i in range(n_imp):
            select()
        ie[2].record(stream)
        torch.cuda.synchronize()
        t_imp = HipEvent.elapsed_ms(ie[0], ie[1]) / n_imp
        t_sel = HipEvent.elapsed_ms(ie[1], ie[2]) / n_imp
        esz = 2
        imp_flops = work["prefill_pairs"] * 2 * lay.head_dim
        imp_bytes = (int(w.tp["entries"][:, 2].sum()) * lay.head_dim * esz + w.q_prefill.numel() * esz
                     + w.lse_prefill.numel() * 4 + imp.numel() * 4)
        sel_bytes = imp.numel() * 4 + score.numel() * 4 + int(sel_ptr[-1]) * n_layers * 4
        beyond_imp = {
            "token_importance": {"ms": round(t_imp, 4), "TFLOP/s": round(imp_flops / t_imp / 1e9, 2),
                                 "frac_mfma": round(imp_flops / t_imp / 1e-3 / PEAK_BF16_FLOPS, 4),
                                 "GB/s": round(imp_bytes / t_imp / 1e6, 1),
                                 "frac_hbm": round(imp_bytes / t_imp / 1e-3 / PEAK_HBM, 4),
                                 "flops": imp_flops, "bytes": imp_bytes},
            "select_tokens": {"ms": round(t_sel, 4), "GB/s": round(sel_bytes / t_sel / 1e6, 1),
                              "bytes": sel_bytes, "layers": n_layers, "k_per_layer_seq": ks[:4]},
        }
        del imp, score, sel

    page_bytes = w.k_pool[0].numel() * w.k_pool.element_size() * 2
    stored = int((w.tp["storage"] >= 0).sum())
    res = {
        "value": round(value, 3), "ms_per_step": round(ms_per_step, 4),
        "kv_bytes_per_session": stored * page_bytes, "stored_pages": stored,
        "chain_pages": int(len(w.tp["storage"])),
        "config": {"workload": f"{name}: {WORKLOAD_TEXT[name]}", "seed": seed, "slots": lay.n_slot,
                   "sequences": lay.n_seq, "prefill_tokens": int(w.h_tok_ptr[-1]), "decode_tokens": lay.n_seq,
                   "pool_replicas": n_rep, "settle_steps": n_settle},
        "roofline": roof, "calls": calls_out,
        "beyond_step": {"pack_pages": {"ms": round(t_pack, 4), "GB/s": round(pack_bytes / t_pack / 1e6, 1),
                                       "frac_hbm": round(pack_bytes / t_pack / 1e-3 / PEAK_HBM, 4),
                                       "bytes": pack_bytes, "pages": n_ent},
                        **(beyond_imp or {})},
        "dtype": "f32" if lay.dtype == "f32" else "bf16",
    }
    if per_layer_out is not None:
        res["per_layer"] = per_layer_out
    del reps
    return res, w


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="32k", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-128k", action="store_true", help="skip the 128K block of the default run")
    ap.add_argument("--no-window", action="store_true", help="skip the window-only storage block")
    ap.add_argument("--no-layers", action="store_true", help="skip the per-layer calls of the default run")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle seconds per CPU process")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the hot path runs on a single MI355X and has no "
              "multi-GPU mode (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # The oracle's worker processes are forked before anything touches the GPU,
    # so none of them holds the device.
    pool = n_workers = None
    if not args.no_cpu_baseline:
        n_workers = max(1, min(16, os.cpu_count() or 1))
        pool = mp.get_context("fork").Pool(n_workers)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    res0, w = run_config(args.config, args.seed, args.steps, args.warmup, log,
                         per_layer=args.config == "32k" and not args.no_layers)
    lay, tp = w.lay, w.tp
    del w
    res = {"metric": METRIC, "value": res0["value"], "unit": "% of roofline", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": res0["ms_per_step"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": res0["dtype"], "data": "synthetic",
           "config": res0["config"], "roofline": res0["roofline"], "calls": res0["calls"],
           "beyond_step": res0["beyond_step"]}
    if "per_layer" in res0:
        res["per_layer"] = res0["per_layer"]
    if args.config == "32k" and not args.no_128k:
        torch.cuda.empty_cache()
        r128, w128 = run_config("128k", args.seed, max(3, args.steps // 2), max(2, args.warmup // 2), log)
        del w128
        torch.cuda.empty_cache()
        res["config_128k"] = {k: r128[k] for k in ("value", "ms_per_step", "config", "roofline", "calls",
                                                    "beyond_step")}
    if args.config in ("32k", "16k", "128k", "batch") and not args.no_window:
        # Window-only storage of the same workload (every head stores only the
        # pages its queries can read): the same step, and the KV bytes one
        # session holds, against whole chains.
        torch.cuda.empty_cache()
        rw, ww = run_config(args.config, args.seed, args.steps, args.warmup, log, window_only=True)
        del ww
        torch.cuda.empty_cache()
        whole = res0["kv_bytes_per_session"]
        res["window_only"] = {
            "ms_per_step": rw["ms_per_step"], "value": rw["value"],
            "calls": {k: rw["calls"][k] for k in ("rope_relocate", "segpaged_prefill", "segpaged_decode")},
            "kv_bytes_per_session": rw["kv_bytes_per_session"], "whole_chain_kv_bytes_per_session": whole,
            "sessions_ratio": round(whole / rw["kv_bytes_per_session"], 3),
            "sessions_per_288GB": {"whole_chains": int(288e9 // whole),
                                   "window_only": int(288e9 // rw["kv_bytes_per_session"])},
            "note": "relocation moves only the stored segment keys; prefill and decode results are bit-identical "
                    "to whole-chain storage (value against the same roofline formula, now with fewer bytes)"}
    if pool is not None:
        log(f"timing the oracle on a CPU sample ({n_workers} processes) ...")
        res["cpu_baseline"] = cpu_baseline(pool, n_workers, lay, tp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
