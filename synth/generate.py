"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws numbers and lays out the workload (sequence lengths,
segment positions, head classes, retrieval page lists, the free list and the
Q/K/V values).  It holds none of the method's arithmetic: no page tables, no
visibility, no rotation, no attention.

Reading of the pages used here (the pages give no generator):
  * Online positions of a sequence's segments are contiguous in segment order,
    starting at 0; the new tokens (prefill chunk, then decode tokens) follow the
    last segment.
  * Q and K are drawn directly as the already-rotated vectors at their cached
    (offline, for segment keys) or online (new keys, queries) positions: an
    orthogonal rotation of i.i.d. N(0,1) coordinates is again i.i.d. N(0,1), so
    the draw has the distribution of rotated vectors without rotating anything.
  * Values are drawn in fp32 and rounded to nearest-even to the storage dtype;
    both sides consume the identical rounded values.
  * Head-class counts over the (layer, kv-head) slots use the largest
    remainder in integer arithmetic, ties broken by the order the mix is
    stated in; the labels are then placed by a seeded permutation.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .configs import CONFIGS, GLOBAL, LOCAL, RETRIEVAL, DENSE

# stream ids for SeedSequence spawn keys
_S_CLASS, _S_LENS, _S_RET, _S_FREE, _S_VAL, _S_Q, _S_SCORE = 1, 2, 3, 4, 5, 6, 7


def _rng(seed: int, cfg_idx: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(cfg_idx,) + key)))


def _torch_seed(seed: int, cfg_idx: int, *key: int) -> int:
    st = np.random.SeedSequence(seed, spawn_key=(cfg_idx,) + key).generate_state(2, dtype=np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


@dataclass
class Layout:
    """One workload instance: sequences, segments, slots and their classes."""
    name: str
    seed: int
    n_seq: int
    seg_len: list            # per seq: np.int64 array of segment lengths
    seg_online: list         # per seq: online base position of each segment
    seg_offline: list        # per seq: offline (cached) base position of each segment
    new_base: np.ndarray     # per seq: position of the first new token
    n_prefill: int
    n_decode: int
    n_slot: int
    cls: np.ndarray          # [n_slot] class code
    window: np.ndarray       # [n_slot] window (local) else 0
    ret_k: np.ndarray        # [n_slot] pages listed per retrieval row (0 otherwise)
    ret_pages: dict = field(default_factory=dict)   # (slot, seq) -> sorted segment-page ordinals
    page_size: int = 16
    head_dim: int = 128
    group: int = 1
    dtype: str = "bf16"
    theta: float = 10000.0
    k_scale: float = 1.0
    cfg_idx: int = 0

    @property
    def n_new(self) -> int:
        return self.n_prefill + self.n_decode

    def ctx_len(self, seq: int) -> int:
        return int(self.seg_len[seq].sum())

    # --- ABI marshalling (plain arrays in the layout the C header documents) ---
    def abi_arrays(self, call: str):
        """Arrays for segpaged_build_tables; ``call`` is "prefill" or "decode"."""
        seg_ptr = np.zeros(self.n_seq + 1, np.int32)
        segs = []
        for s in range(self.n_seq):
            seg_ptr[s + 1] = seg_ptr[s] + len(self.seg_len[s])
            for ln, on, off in zip(self.seg_len[s], self.seg_online[s], self.seg_offline[s]):
                segs.append((ln, on, off))
        segs = np.asarray(segs, np.int32).reshape(-1, 3)
        n_new = np.full(self.n_seq, self.n_new, np.int32)
        if call == "prefill":
            q_lo = self.new_base.astype(np.int32)
            q_hi = (self.new_base + self.n_prefill - 1).astype(np.int32)
        elif call == "decode":
            q_lo = (self.new_base + self.n_prefill).astype(np.int32)
            q_hi = q_lo.copy()
        else:
            raise ValueError(call)
        rows = self.n_slot * self.n_seq
        ret_ptr = np.zeros(rows + 1, np.int32)
        ret_list = []
        for slot in range(self.n_slot):
            for s in range(self.n_seq):
                r = slot * self.n_seq + s
                lst = self.ret_pages.get((slot, s), np.zeros(0, np.int32))
                ret_ptr[r + 1] = ret_ptr[r] + len(lst)
                ret_list.append(np.asarray(lst, np.int32))
        ret_pages = np.concatenate(ret_list) if ret_list else np.zeros(0, np.int32)
        return dict(seg_ptr=seg_ptr, segs=segs, n_new=n_new, q_lo=q_lo, q_hi=q_hi,
                    cls=self.cls.astype(np.int32), window=self.window.astype(np.int32),
                    ret_ptr=ret_ptr, ret_pages=ret_pages.astype(np.int32))


def _class_counts(mix, n_slot):
    """Largest-remainder split of n_slot into the stated percentages (integers only)."""
    base = [(pct * n_slot) // 100 for (_, pct, _, _) in mix]
    rem = [(pct * n_slot) % 100 for (_, pct, _, _) in mix]
    left = n_slot - sum(base)
    order = sorted(range(len(mix)), key=lambda i: (-rem[i], i))
    for i in order[:left]:
        base[i] += 1
    return base


def _seg_pages(lens, ps):
    # how many page-sized pieces each segment is cut into (the retrieval list
    # draws ordinals from this range)
    return int(sum((int(l) + ps - 1) // ps for l in lens))


def make_layout(name: str, seed: int = 0, **override) -> Layout:
    cfg = dict(CONFIGS[name])
    cfg.update(override)
    ci = cfg["idx"]
    ps = cfg["page_size"]
    n_slot = cfg["n_layers"] * cfg["n_kv"]

    # --- sequences and segments ---
    sq = cfg["seqs"]
    seg_len, seg_on, seg_off = [], [], []
    if sq["kind"] == "fixed":
        lens = np.asarray(sq["seg_lens"], np.int64)
        on = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
        off = np.asarray(sq["offline"], np.int64)
        seg_len, seg_on, seg_off = [lens], [on], [off]
        n_seq = 1
    else:
        n_seq = sq["n_seq"]
        rng = _rng(seed, ci, _S_LENS)
        for _ in range(n_seq):
            total = int(rng.integers(sq["len_lo"], sq["len_hi"], endpoint=True))
            lens = []
            while sum(lens) < total:
                lens.append(int(rng.integers(sq["seg_lo"], sq["seg_hi"], endpoint=True)))
            lens[-1] -= sum(lens) - total          # truncate the last one to fit
            lens = np.asarray(lens, np.int64)
            on = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
            off = rng.integers(sq["off_lo"], sq["off_hi"], size=len(lens), endpoint=True).astype(np.int64)
            seg_len.append(lens)
            seg_on.append(on)
            seg_off.append(off)
    new_base = np.asarray([int(l.sum()) for l in seg_len], np.int64)

    # --- head classes per slot ---
    cls = np.zeros(n_slot, np.int32)
    win = np.zeros(n_slot, np.int32)
    retk = np.zeros(n_slot, np.int32)
    if "slot_classes" in cfg:
        for i, (c, w) in enumerate(cfg["slot_classes"]):
            cls[i], win[i] = c, w
    else:
        counts = _class_counts(cfg["mix"], n_slot)
        labels = []
        for (c, _pct, w, k), n in zip(cfg["mix"], counts):
            labels += [(c, w, k)] * n
        perm = _rng(seed, ci, _S_CLASS).permutation(n_slot)
        for pos, j in enumerate(perm):
            c, w, k = labels[j]
            cls[pos], win[pos], retk[pos] = c, w, k

    # --- retrieval page lists (segment-page ordinals, sorted, no repeats) ---
    ret = {}
    for slot in range(n_slot):
        if cls[slot] != RETRIEVAL:
            continue
        for s in range(n_seq):
            npg = _seg_pages(seg_len[s], ps)
            k = min(int(retk[slot]), npg)
            r = _rng(seed, ci, _S_RET, slot, s)
            ret[(slot, s)] = np.sort(r.choice(npg, size=k, replace=False)).astype(np.int32)

    return Layout(name=name, seed=seed, n_seq=n_seq, seg_len=seg_len, seg_online=seg_on,
                  seg_offline=seg_off, new_base=new_base, n_prefill=cfg["n_prefill"],
                  n_decode=cfg["n_decode"], n_slot=n_slot, cls=cls, window=win, ret_k=retk,
                  ret_pages=ret, page_size=ps, head_dim=cfg["head_dim"], group=cfg["group"],
                  dtype=cfg["dtype"], theta=cfg["theta"], k_scale=cfg["k_scale"], cfg_idx=ci)


def custom_layout(*, seg_lens, offline, n_prefill, n_decode, classes, page_size, head_dim=64,
                  group=1, dtype="f32", theta=10000.0, k_scale=1.0, ret_lists=None, name="custom",
                  seed=0) -> Layout:
    """A hand-specified layout (tests).  ``seg_lens``/``offline``: one list per sequence;
    ``classes``: one (class, window) per slot; ``ret_lists``: {(slot, seq): ordinals}."""
    seg_len = [np.asarray(l, np.int64) for l in seg_lens]
    seg_on = [np.concatenate([[0], np.cumsum(l)[:-1]]).astype(np.int64) if len(l) else np.zeros(0, np.int64)
              for l in seg_len]
    seg_off = [np.asarray(o, np.int64) for o in offline]
    n_slot = len(classes)
    cls = np.asarray([c for c, _ in classes], np.int32)
    win = np.asarray([w for _, w in classes], np.int32)
    ret = {k: np.asarray(v, np.int32) for k, v in (ret_lists or {}).items()}
    retk = np.zeros(n_slot, np.int32)
    return Layout(name=name, seed=seed, n_seq=len(seg_len), seg_len=seg_len, seg_online=seg_on,
                  seg_offline=seg_off, new_base=np.asarray([int(l.sum()) for l in seg_len], np.int64),
                  n_prefill=n_prefill, n_decode=n_decode, n_slot=n_slot, cls=cls, window=win,
                  ret_k=retk, ret_pages=ret, page_size=page_size, head_dim=head_dim, group=group,
                  dtype=dtype, theta=theta, k_scale=k_scale, cfg_idx=99)


def free_list(lay: Layout, n_pool: int) -> np.ndarray:
    """A seeded permutation of the physical page ids [0, n_pool)."""
    return _rng(lay.seed, lay.cfg_idx, _S_FREE).permutation(n_pool).astype(np.int32)


# ----------------------------------------------------------------------------
# values (torch: generated on whichever device will hold them)
# ----------------------------------------------------------------------------

def _torch_dtype(lay):
    import torch
    return torch.float32 if lay.dtype == "f32" else torch.bfloat16


def unit_values(lay: Layout, slot: int, seq: int, device="cpu"):
    """K/V of one (slot, sequence): segment tokens in online-position order, then
    the new tokens.  Returns dict(seg_k, seg_v, new_k, new_v) in the storage dtype."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(lay.seed, lay.cfg_idx, _S_VAL, slot, seq))
    D, ctx, nn = lay.head_dim, lay.ctx_len(seq), lay.n_new
    dt = _torch_dtype(lay)
    out = {}
    for nm, n, sc in (("seg_k", ctx, lay.k_scale), ("seg_v", ctx, 1.0),
                      ("new_k", nn, lay.k_scale), ("new_v", nn, 1.0)):
        x = torch.randn(n, D, generator=g, device=device, dtype=torch.float32)
        if sc != 1.0:
            x.mul_(sc)
        out[nm] = x.to(dt)
    return out


def seq_queries(lay: Layout, seq: int, device="cpu"):
    """Queries of every new token of one sequence: [n_new, n_slot * group, head_dim]."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(lay.seed, lay.cfg_idx, _S_Q, seq))
    x = torch.randn(lay.n_new, lay.n_slot * lay.group, lay.head_dim, generator=g, device=device,
                    dtype=torch.float32)
    return x.to(_torch_dtype(lay))


def score_values(seed: int, n_slots: int, n_pos: int, levels: int = 0) -> np.ndarray:
    """Seeded non-negative fp32 per-slot scores [n_slots, n_pos] (inputs for the
    token selection).  levels > 0 draws from that many equally spaced values, so
    that equal scores (ties) are common."""
    r = _rng(seed, 98, _S_SCORE, n_slots, n_pos, levels)
    if levels > 0:
        return (r.integers(0, levels, size=(n_slots, n_pos)) / levels).astype(np.float32)
    return r.exponential(1.0, size=(n_slots, n_pos)).astype(np.float32)
