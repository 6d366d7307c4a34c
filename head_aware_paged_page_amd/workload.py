"""A device-resident SegPaged workload: tables, pools and queries on one GPU.

Glue around the C ABI for tests, the smoke check and the benchmark: it builds
the prefill and decode tables with ``segpaged_build_tables``, fills the paged
K/V pools with the seeded synthetic values, uploads everything once, and then
issues ``rope_relocate`` / ``segpaged_prefill`` / ``segpaged_decode`` on
device-resident inputs.  Every step of the path runs in libsegpaged.
"""
from __future__ import annotations

import math
import time

import numpy as np

import synth
from . import segpaged as sp
from .kvpool import chain_token_index, place


class Workload:
    def __init__(self, lay, device="cuda", fill_nan: bool = True, pool_slack: int = 0, relocated_pool: bool = True,
                 free=None, window_only: bool = False):
        """window_only: store only the pages some query of the session can read
        (segpaged_build_tables_ex with keep_from = the prefill chunk's first
        position); the decode tables then come from segpaged_tables_from_chains
        over the same storage, and tokens on pages not stored are not placed."""
        import torch
        self.lay = lay
        self.device = device
        ps, D, G = lay.page_size, lay.head_dim, lay.group
        self.ps, self.D, self.G = ps, D, G
        self.n_seq, self.n_slot = lay.n_seq, lay.n_slot
        self.Hq = lay.n_slot * G
        self.dtype = torch.float32 if lay.dtype == "f32" else torch.bfloat16
        self.scale = 1.0 / math.sqrt(D)

        arr_p = lay.abi_arrays("prefill")
        arr_d = lay.abi_arrays("decode")
        self.window_only = window_only
        self.keep_from = arr_p["q_lo"] if window_only else None
        cnt = sp.build_tables_ex(**arr_p, page_size=ps, free_list=None, keep_from=self.keep_from,
                                 counts_only=True)["counts"]
        if free is None:
            self.n_phys = int(cnt[3]) + pool_slack
            self.free = synth.free_list(lay, self.n_phys)
        else:
            self.free = np.ascontiguousarray(free, dtype=np.int32)
            self.n_phys = int(self.free.max()) + 1
        t0 = time.perf_counter()
        self.tp = sp.build_tables_ex(**arr_p, page_size=ps, free_list=self.free, keep_from=self.keep_from)
        t1 = time.perf_counter()
        self.layout_args = {k: arr_p[k] for k in ("seg_ptr", "segs", "n_new", "cls", "window", "ret_ptr",
                                                  "ret_pages")}
        rp, ent = sp.tables_from_chains(**self.layout_args, q_lo=arr_d["q_lo"], q_hi=arr_d["q_hi"], page_size=ps,
                                        chain_ptr=self.tp["chain_ptr"], storage=self.tp["storage"])
        self.td = dict(row_ptr=rp, entries=ent)
        self.build_seconds = (t1 - t0)
        self.arr_p, self.arr_d = arr_p, arr_d

        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
        self.d_cls = dev(arr_p["cls"])
        self.d_window = dev(arr_p["window"])
        self.d_reloc = dev(self.tp["reloc"])
        self.p_row_ptr, self.p_entries = dev(self.tp["row_ptr"]), dev(self.tp["entries"])
        self.d_row_ptr, self.d_entries = dev(self.td["row_ptr"]), dev(self.td["entries"])
        self.h_tok_ptr = np.arange(self.n_seq + 1, dtype=np.int32) * lay.n_prefill
        self.d_tok_ptr = dev(self.h_tok_ptr)
        self.d_q_pos0 = dev(arr_p["q_lo"])
        self.d_q_dec = dev(arr_d["q_lo"])

        # pools: segment K as cached (offline rotation), new K/V at online positions
        fill = float("nan") if fill_nan else 0.0
        self.k_pool = torch.full((self.n_phys, ps, D), fill, dtype=self.dtype, device=device)
        self.v_pool = torch.full((self.n_phys, D, ps), fill, dtype=self.dtype, device=device)
        storage = torch.from_numpy(self.tp["storage"].astype(np.int64)).to(device)
        chain_ptr = self.tp["chain_ptr"]
        self.chain_phys = lambda slot, seq: storage[chain_ptr[slot * self.n_seq + seq]:
                                                    chain_ptr[slot * self.n_seq + seq + 1]]
        self._tok_index = {}
        for seq in range(self.n_seq):
            idx, off = chain_token_index(lay.seg_len[seq], lay.n_new, ps)
            self._tok_index[seq] = (torch.from_numpy(idx).to(device), torch.from_numpy(off).to(device))
        for slot in range(self.n_slot):
            for seq in range(self.n_seq):
                u = synth.unit_values(lay, slot, seq, device=device)
                K = torch.cat([u["seg_k"], u["new_k"]])
                V = torch.cat([u["seg_v"], u["new_v"]])
                idx, off = self._tok_index[seq]
                phys = self.chain_phys(slot, seq)
                stored = phys[idx] >= 0               # tokens on pages that are not stored stay out
                if not bool(stored.all()):
                    idx, off, K, V = idx[stored], off[stored], K[stored], V[stored]
                place(self.k_pool, self.v_pool, phys, idx, off, K, V)
                del u, K, V
        self.k_reloc = self.k_pool.clone() if relocated_pool else None

        qs = [synth.seq_queries(lay, seq, device=device) for seq in range(self.n_seq)]
        self.q_prefill = torch.cat([q[: lay.n_prefill] for q in qs]).contiguous()
        self.q_decode = torch.cat([q[lay.n_prefill: lay.n_prefill + 1] for q in qs]).contiguous()
        del qs

        code = sp.SP_F32 if lay.dtype == "f32" else sp.SP_BF16
        self.ws_prefill = sp.workspace_bytes(sp.SP_WS_PREFILL, code, D, ps, G, self.n_seq, self.n_slot,
                                             self.h_tok_ptr, self.tp["row_ptr"])
        self.ws_decode = sp.workspace_bytes(sp.SP_WS_DECODE, code, D, ps, G, self.n_seq, self.n_slot, None,
                                            self.td["row_ptr"])
        self.workspace = torch.empty(max(self.ws_prefill, self.ws_decode), dtype=torch.uint8, device=device)
        self.out_prefill = torch.empty_like(self.q_prefill)
        self.lse_prefill = torch.empty(self.q_prefill.shape[:2], dtype=torch.float32, device=device)
        self.out_decode = torch.empty_like(self.q_decode)
        self.lse_decode = torch.empty(self.q_decode.shape[:2], dtype=torch.float32, device=device)

    # ------------------------------------------------------------------ calls
    def relocate(self, k_in=None, k_out=None, stream=None, back=False):
        """rope_relocate of the workload's list, in place when k_in is k_out;
        back=True rotates by the negated deltas (undoes a relocation in place)."""
        k_in = self.k_pool if k_in is None else k_in
        k_out = self.k_reloc if k_out is None else k_out
        if back and getattr(self, "_d_reloc_back", None) is None:
            self._d_reloc_back = self.d_reloc.clone()
            self._d_reloc_back[:, 1] = -self._d_reloc_back[:, 1]
        lst = self._d_reloc_back if back else self.d_reloc
        sp.rope_relocate(k_in, k_out, self.ps, lst, self.lay.theta, stream=stream)
        return k_out

    def prefill(self, k=None, q=None, out=None, lse=None, stream=None, v=None):
        k = self.k_pool if k is None else k
        v = self.v_pool if v is None else v
        sp.prefill(self.q_prefill if q is None else q, k, v, page_size=self.ps, group=self.G,
                   n_seq=self.n_seq, n_slot=self.n_slot, h_tok_ptr=self.h_tok_ptr, h_row_ptr=self.tp["row_ptr"],
                   d_tok_ptr=self.d_tok_ptr, d_q_pos0=self.d_q_pos0, d_cls=self.d_cls, d_window=self.d_window,
                   d_row_ptr=self.p_row_ptr, d_entries=self.p_entries, scale=self.scale,
                   out=self.out_prefill if out is None else out, lse=self.lse_prefill if lse is None else lse,
                   workspace=self.workspace, stream=stream)
        return self.out_prefill if out is None else out, self.lse_prefill if lse is None else lse

    def decode(self, k=None, q=None, out=None, lse=None, stream=None, v=None):
        k = self.k_pool if k is None else k
        v = self.v_pool if v is None else v
        sp.decode(self.q_decode if q is None else q, k, v, page_size=self.ps, group=self.G,
                  n_seq=self.n_seq, n_slot=self.n_slot, h_row_ptr=self.td["row_ptr"], d_q_pos=self.d_q_dec,
                  d_cls=self.d_cls, d_window=self.d_window, d_row_ptr=self.d_row_ptr, d_entries=self.d_entries,
                  scale=self.scale, out=self.out_decode if out is None else out,
                  lse=self.lse_decode if lse is None else lse, workspace=self.workspace, stream=stream)
        return self.out_decode if out is None else out, self.lse_decode if lse is None else lse

    def importance(self, lse=None, k=None, span="all", out=None, stream=None):
        """segpaged_token_importance over the prefill call (its lse by default):
        returns (imp [n_slot, n_pos] fp32, pos_ptr); span "all" covers every
        position of a sequence (segments and new tokens), "segments" only the
        reused segment positions.  out: a previous call's (imp, pos_ptr) to
        write into again (no allocation)."""
        import torch
        if out is None:
            lens = [int(self.lay.new_base[s]) + (self.lay.n_new if span == "all" else 0) for s in range(self.n_seq)]
            pos_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            code = sp.SP_F32 if self.lay.dtype == "f32" else sp.SP_BF16
            nb = sp.workspace_bytes(sp.SP_WS_IMPORTANCE, code, self.D, self.ps, self.G, self.n_seq, self.n_slot,
                                    self.h_tok_ptr, self.tp["row_ptr"])
            self._imp_ws = torch.empty(nb, dtype=torch.uint8, device=self.device)
            self._imp_pos = torch.from_numpy(pos_ptr).to(self.device)
            imp = torch.empty((self.n_slot, int(pos_ptr[-1])), dtype=torch.float32, device=self.device)
        else:
            imp, pos_ptr = out
        sp.token_importance(self.q_prefill, k if k is not None else self.k_pool, page_size=self.ps, group=self.G,
                            n_seq=self.n_seq, n_slot=self.n_slot, h_tok_ptr=self.h_tok_ptr,
                            h_row_ptr=self.tp["row_ptr"], d_tok_ptr=self.d_tok_ptr, d_q_pos0=self.d_q_pos0,
                            d_cls=self.d_cls, d_window=self.d_window, d_row_ptr=self.p_row_ptr,
                            d_entries=self.p_entries, scale=self.scale,
                            lse=self.lse_prefill if lse is None else lse, h_pos_ptr=pos_ptr,
                            d_pos_ptr=self._imp_pos, imp=imp, workspace=self._imp_ws, stream=stream)
        return imp, pos_ptr

    def replicas(self, n: int):
        """n copies of the pools, [(k_pool, v_pool, k_reloc)], the first being the
        workload's own; the copies share every table (same physical ids)."""
        reps = [(self.k_pool, self.v_pool, self.k_reloc)]
        for _ in range(n - 1):
            reps.append((self.k_pool.clone(), self.v_pool.clone(), self.k_reloc.clone()))
        return reps

    def pool_bytes(self) -> int:
        """Bytes of one replica: the K and V pools and the relocated K pool."""
        b = self.k_pool.numel() * self.k_pool.element_size() * 2
        return b + (self.k_reloc.numel() * self.k_reloc.element_size() if self.k_reloc is not None else 0)

    # ------------------------------------------------------------------ host views for checking
    def unit_host(self, slot: int, seq: int):
        """fp64 copies of one unit's generated K/V (position order) for the checker."""
        u = synth.unit_values(self.lay, slot, seq, device=self.device)
        K = np.concatenate([u["seg_k"].double().cpu().numpy(), u["new_k"].double().cpu().numpy()])
        V = np.concatenate([u["seg_v"].double().cpu().numpy(), u["new_v"].double().cpu().numpy()])
        return K, V

    def gather_keys(self, pool, slot: int, seq: int):
        """Keys of one chain read back from a K pool, in position order (fp64
        host); NaN for tokens on pages that are not stored."""
        idx, off = self._tok_index[seq]
        phys = self.chain_phys(slot, seq)[idx]
        out = pool[phys.clamp(min=0), off].double()
        out[phys < 0] = float("nan")
        return out.cpu().numpy()
