"""Softmax attention of each query over exactly its visible tokens (plain fp64).

Test infrastructure (see the package docstring): never imported by the product.

Sources:
  * RedKnot product profile (tokenfly.club), section 3, fourth building block:
    SegPagedAttention keeps every head on the ordinary (mask-free) attention
    path while each class of head sees its own window - i.e. the result is plain
    softmax attention restricted to the head's visible tokens.
  * "PagedAttention & RadixAttention" (wiki.gxlh.xyz), opening of the
    PagedAttention part: paging changes where K/V live, not the attention
    arithmetic - every query still takes dot products with the keys and
    averages the values.

Readings where the pages are silent: softmax scale 1/sqrt(D); LSE in natural log;
query head h of a call belongs to slot h // group (contiguous GQA groups);
attention is causal among new tokens for every class.
"""
from __future__ import annotations

import numpy as np

from . import tables


def attend(q, K, V, scale: float):
    """q [G, D], K/V [n, D] -> (o [G, D], lse [G]): softmax(q K^T * scale) V in fp64."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    s = (q @ K.T) * scale                       # [G, n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    o = (e @ V) / z
    lse = m[:, 0] + np.log(z[:, 0])
    return o, lse


def row_attention(lay, slot: int, seq: int, K_all, V_all, q, q_pos):
    """Attention of one (slot, seq) row.

    K_all / V_all: [n_tokens, D] keys/values of the chain's tokens in position
    order (segment tokens, then new tokens).
    q: [n_q, G, D] queries of this slot's group, q_pos: [n_q] their positions.
    Returns (O [n_q, G, D], LSE [n_q, G], counts [n_q]).
    """
    tpos, _tpage, tsp, tnew = tables.tokens(lay, seq)
    listed = lay.ret_pages.get((slot, seq), [])
    c, w = int(lay.cls[slot]), int(lay.window[slot])
    scale = 1.0 / np.sqrt(lay.head_dim)
    n_q = len(q_pos)
    G, D = q.shape[1], q.shape[2]
    O = np.zeros((n_q, G, D))
    L = np.zeros((n_q, G))
    cnt = np.zeros(n_q, np.int64)
    for i, p in enumerate(q_pos):
        idx = np.nonzero(tables.visible(c, w, listed, tpos, tsp, tnew, int(p)))[0]
        O[i], L[i] = attend(q[i], K_all[idx], V_all[idx], scale)
        cnt[i] = len(idx)
    return O, L, cnt

