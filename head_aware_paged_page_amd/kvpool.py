"""Placing token K/V into the paged pools (plain device copies).

The page chain of every (slot, sequence) is laid out as include/segpaged.h
documents it: each segment starts on a fresh page, the new tokens start on a
fresh page after the last segment, and token t of a region sits at page
t // page_size, slot t % page_size of that region (the fixed-size block rule of
the PagedAttention & RadixAttention page, "The Solution: Fixed-size blocks").
Writing tokens there is ordinary indexed copying on the GPU.
"""
from __future__ import annotations

import numpy as np


def chain_token_index(seg_lens, n_new: int, page_size: int):
    """Chain page index and in-page offset of every token of one chain, in
    position order (segment tokens, then new tokens)."""
    idx, off = [], []
    base = 0
    for ln in seg_lens:
        t = np.arange(int(ln), dtype=np.int64)
        idx.append(base + t // page_size)
        off.append(t % page_size)
        base += (int(ln) + page_size - 1) // page_size
    t = np.arange(int(n_new), dtype=np.int64)
    idx.append(base + t // page_size)
    off.append(t % page_size)
    return np.concatenate(idx), np.concatenate(off)


def place(k_pool, v_pool, chain_phys, tok_idx, tok_off, K, V):
    """Write K [n, D] into k_pool [n_phys, ps, D] and V [n, D] into the dim-major
    v_pool [n_phys, D, ps] at the chain slots (tok_idx, tok_off).

    chain_phys: physical page of each chain page (torch int64, same device)."""
    phys = chain_phys[tok_idx]
    if K is not None:
        k_pool[phys, tok_off] = K
    if V is not None:
        v_pool[phys, :, tok_off] = V
