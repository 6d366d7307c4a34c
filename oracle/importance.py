"""Attention importance of context tokens and the token selection for the sparse FFN.

Test infrastructure (see the package docstring): never imported by the product.

Sources, by the pages' titles:
  * RedKnot product profile (tokenfly.club), section 3, third building block
    (elastic sparse FFN): tokens are chosen for the feed-forward network by
    their attention importance, and low-contribution tokens skip it; this is
    what matters for the short 2K-8K segments of agent workloads, where the FFN
    dominates prefill.
  * The is96.com commentary on the RedKnot paper: the layered sparse FFN works
    beside the head-level reuse, because at short contexts the FFN, not
    attention, is most of the time to first token.

The pages give no scoring rule.  Readings used here (the plainest the rest
supports):
  * The importance a context token t receives in one slot is the attention the
    call's query rows (every new token of the chunk, every query head of the
    slot's group) pay to it: the sum over those rows of the row's softmax
    probability of t, P(i, t) = exp(scale q_i.k_t) / sum_{u in V(i)} exp(scale q_i.k_u)
    over the row's own visible set V(i) (0 when t is not in V(i)).  Every row's
    probabilities sum to 1, so the importances of a slot sum to its number of
    query rows.
  * The importance of t in a layer is the sum over the layer's slots (KV
    heads, each with its query group), the slots of layer l being l * n + 0 ..
    l * n + n - 1.
  * Selection: in each (layer, sequence), the k candidate positions of highest
    layer importance; equal importances go to the lower position.  The
    decision is taken in fp32, the precision the device computes in: slot
    importances rounded to fp32, summed in fp32 in slot order.
"""
from __future__ import annotations

import numpy as np

from . import tables


def row_importance(lay, slot: int, seq: int, K_all, q, q_pos, n_pos: int):
    """Importance of positions 0 .. n_pos-1 for one (slot, seq) row.

    K_all: [n_tokens, D] keys of the chain's tokens in position order (segment
    tokens, then new tokens); q: [n_q, G, D] the slot's query rows of the chunk,
    at positions q_pos.  Returns float64 [n_pos]."""
    tpos, _tpage, tsp, tnew = tables.tokens(lay, seq)
    listed = lay.ret_pages.get((slot, seq), [])
    c, w = int(lay.cls[slot]), int(lay.window[slot])
    scale = 1.0 / np.sqrt(lay.head_dim)
    imp = np.zeros(n_pos)
    for i, p in enumerate(q_pos):
        idx = np.nonzero(tables.visible(c, w, listed, tpos, tsp, tnew, int(p)))[0]
        s = (np.asarray(q[i], np.float64) @ np.asarray(K_all[idx], np.float64).T) * scale   # [G, n]
        e = np.exp(s - s.max(axis=1, keepdims=True))
        P = e / e.sum(axis=1, keepdims=True)                 # each row's softmax over its visible set
        keep = tpos[idx] < n_pos
        np.add.at(imp, tpos[idx][keep], P.sum(axis=0)[keep])
    return imp


def layer_scores(imp_slots):
    """fp32 layer importance from the slots' importances [n_slots_of_layer, n_pos]:
    each rounded to fp32, added in slot order in fp32."""
    imp_slots = np.asarray(imp_slots)
    acc = imp_slots[0].astype(np.float32)
    for s in range(1, len(imp_slots)):
        acc = (acc + imp_slots[s].astype(np.float32)).astype(np.float32)
    return acc


def select(score, k: int):
    """The k positions of highest score (equal scores: lower position first), ascending."""
    score = np.asarray(score)
    n = len(score)
    order = np.lexsort((np.arange(n), -score.astype(np.float64)))   # last key sorts first
    return np.sort(order[:k]).astype(np.int64)
