"""Per-head visible-page pack and unpack: the pages of every head's table,
gathered in table order into one contiguous buffer, and scattered back.

Test infrastructure (see the package docstring): never imported by the product.

Sources, by the pages' titles:
  * RedKnot product profile (tokenfly.club), section 3: each (layer, head) reads
    only the pages of its own table, and under prefill/decode disaggregation
    only those pages have to move between machines (the KV-transfer reduction
    it reports).
  * The is96.com commentary on the RedKnot paper, paragraphs on the per-head
    page table: a head's table lists exactly the pages that head reads.

Readings where the pages are silent:
  * A packed buffer holds whole pages (every slot of a page, tokens or not), K
    as [n_pages][page_size][head_dim] and V as [n_pages][head_dim][page_size],
    the layouts of the pools, in the order of the tables' entries.
  * A page id outside the pool packs as zeros, and unpacking skips it.
"""
from __future__ import annotations

import numpy as np


def pack(k_pool: np.ndarray, v_pool: np.ndarray, phys: np.ndarray):
    """Packed K and V of the pages phys[0], phys[1], ... (table order)."""
    n = len(phys)
    k_out = np.zeros((n,) + k_pool.shape[1:], k_pool.dtype)
    v_out = np.zeros((n,) + v_pool.shape[1:], v_pool.dtype)
    for e, p in enumerate(np.asarray(phys, np.int64)):
        if 0 <= p < len(k_pool):
            k_out[e] = k_pool[p]
            v_out[e] = v_pool[p]
    return k_out, v_out


def unpack(k_in: np.ndarray, v_in: np.ndarray, phys: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray):
    """Writes packed page e to pool page phys[e] (ids outside the pool are
    skipped); returns the updated copies of the pools."""
    k_pool, v_pool = k_pool.copy(), v_pool.copy()
    for e, p in enumerate(np.asarray(phys, np.int64)):
        if 0 <= p < len(k_pool):
            k_pool[p] = k_in[e]
            v_pool[p] = v_in[e]
    return k_pool, v_pool
