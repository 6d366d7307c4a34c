"""Segment/page allocation, per-head page tables, visible sets, relocation list.

Test infrastructure (see the package docstring): never imported by the product.

Sources, by the pages' titles:
  * RedKnot product profile (tokenfly.club), section 3: every (layer, head) is
    put in one of four classes (global, local, retrieval, dense); SegPagedAttention
    gives each head its own page table over segmented KV storage so that each
    class has its own visible window, with no attention mask.
  * The is96.com commentary on the RedKnot paper, SegPagedAttention paragraphs:
    each head owns a chain of pages holding only its own KV, and its page table
    records which pages that head reads.
  * "PagedAttention & RadixAttention" (wiki.gxlh.xyz), "The Solution: Fixed-size
    blocks" and the 4-token block walk-through after it: fixed-size blocks, a
    logical->physical block table, blocks taken from a global free pool on
    demand, the last block filled before a new one is claimed.

Readings where the pages are silent:
  * A slot is one (layer, KV head); all query heads of its group share its
    class, table and pages.
  * Allocation order: slot -> sequence -> segment -> page, then the pages of the
    new tokens; every page is taken from the front of the caller's free list.
    Each segment starts on a fresh page (its last page may be partial); the new
    tokens start on a fresh page after the last segment.  The caller states the
    new-token capacity up front (prefill chunk + decode tokens), so the page
    chain is the same for the prefill call and the decode call; token j of the
    new region sits in new page j // page_size, which is exactly what claiming a
    page only when the previous one is full gives for one chain.
  * Visible set of a query at position p (tokens with position <= p only):
      global, dense : every token;
      local(W)      : tokens with p - W < pos (W tokens including the query);
      retrieval     : tokens on the listed segment pages, plus every new token.
  * The table of a call whose queries occupy positions [q_lo, q_hi] lists, in
    ascending position, the pages holding at least one token visible to at least
    one of those queries; an entry's n_valid counts the page's tokens that exist
    at the call (position <= q_hi).
  * The relocation list has one entry per stored segment page, in allocation
    order, with delta = online base - offline base of its segment.

Window-only storage and page release (the is96.com commentary's deployment
paragraph: local heads keep only window-sized KV, which multiplies the sessions
one GPU holds; its SegPagedAttention paragraphs: each head's pages hold only its
own KV; the PagedAttention page's walk-through: at the end of a sequence its
blocks return to the free pool).  Readings:
  * A session's queries start at position keep_from (the first token of its
    prefill chunk) and never move left.  A head then stores only the pages
    holding a token that some query at a position in [keep_from, end) can see,
    end = first new position + new-token capacity: a local head the pages
    reaching into its window, a retrieval head its listed pages, global and
    dense heads every page.  The chain keeps its logical layout; a page that is
    not stored has storage id -1.
  * Allocation pops the free list in the usual order, skipping pages that are
    not stored.
  * Release: once the next query of a sequence is at position p_next, a stored
    page no query at a position in [p_next, end) can see returns to the free
    list (its storage id becomes -1).  For a local head that is a page that
    slid out of the window; at p_next >= end (the sequence is over) every page
    of every head returns, which is the walk-through's end-of-sequence release.
"""
from __future__ import annotations

import numpy as np

GLOBAL, LOCAL, RETRIEVAL, DENSE = 0, 1, 2, 3


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def chain(lay, seq: int):
    """Logical pages of one (slot, seq) chain in allocation order.

    Returns a list of dicts {pos_start, n_valid, seg, seg_page}; seg = -1 and
    seg_page = -1 mark new-token pages; seg_page is the page's ordinal among the
    sequence's segment pages (what a retrieval list refers to).
    """
    ps = lay.page_size
    pages = []
    ordinal = 0
    for s, (ln, on) in enumerate(zip(lay.seg_len[seq], lay.seg_online[seq])):
        ln, on = int(ln), int(on)
        for j in range(ceil_div(ln, ps)):
            pages.append(dict(pos_start=on + j * ps, n_valid=min(ps, ln - j * ps), seg=s, seg_page=ordinal))
            ordinal += 1
    nb = int(lay.new_base[seq])
    for j in range(ceil_div(lay.n_new, ps)):
        pages.append(dict(pos_start=nb + j * ps, n_valid=min(ps, lay.n_new - j * ps), seg=-1, seg_page=-1))
    return pages


def allocate(lay, free):
    """Pop physical pages from the front of ``free`` in allocation order.

    Returns (storage, chain_ptr): storage is the flat list of physical ids in
    allocation order; chain_ptr[row] .. chain_ptr[row+1] is row (slot, seq)'s
    slice, with row = slot * n_seq + seq.
    """
    rows = lay.n_slot * lay.n_seq
    chain_len = [len(chain(lay, seq)) for seq in range(lay.n_seq)]
    chain_ptr = np.zeros(rows + 1, np.int64)
    for slot in range(lay.n_slot):
        for seq in range(lay.n_seq):
            r = slot * lay.n_seq + seq
            chain_ptr[r + 1] = chain_ptr[r] + chain_len[seq]
    need = int(chain_ptr[-1])
    if need > len(free):
        raise MemoryError(f"free list holds {len(free)} pages, {need} needed")
    storage = np.asarray(free[:need], np.int64)
    return storage, chain_ptr


def tokens(lay, seq: int):
    """Every stored token of a (slot, seq) chain: (position, page index in the chain,
    segment-page ordinal or -1 for new tokens, is_new)."""
    pos, page, sp, new = [], [], [], []
    for i, pg in enumerate(chain(lay, seq)):
        n = pg["n_valid"]
        pos.append(np.arange(pg["pos_start"], pg["pos_start"] + n, dtype=np.int64))
        page.append(np.full(n, i, np.int64))
        sp.append(np.full(n, pg["seg_page"], np.int64))
        new.append(np.full(n, pg["seg"] < 0))
    return np.concatenate(pos), np.concatenate(page), np.concatenate(sp), np.concatenate(new)


def visible(cls: int, window: int, listed, tok_pos, tok_segpage, tok_new, p: int):
    """Boolean mask over tokens: which tokens the query at position p sees."""
    present = tok_pos <= p
    if cls in (GLOBAL, DENSE):
        return present
    if cls == LOCAL:
        return present & (tok_pos > p - window)
    if cls == RETRIEVAL:
        on_listed = np.isin(tok_segpage, np.asarray(listed, np.int64)) & ~tok_new
        return present & (on_listed | tok_new)
    raise ValueError(f"unknown class {cls}")


def phys_of(storage, chain_ptr, r: int, i: int) -> int:
    """Physical id of chain page i of row r; raises if that page is not stored."""
    v = int(storage[int(chain_ptr[r]) + i])
    if v < 0:
        raise LookupError(f"row {r}: chain page {i} is not stored")
    return v


def row_table(lay, storage, chain_ptr, slot: int, seq: int, q_lo: int, q_hi: int):
    """Table of one (slot, seq) row: int64 array [n, 3] of (phys, pos_start, n_valid)."""
    r = slot * lay.n_seq + seq
    c, w = int(lay.cls[slot]), int(lay.window[slot])
    pages = chain(lay, seq)
    tpos, tpage, tsp, tnew = tokens(lay, seq)
    listed = lay.ret_pages.get((slot, seq), [])
    seen = np.zeros(len(tpos), bool)
    for p in range(int(q_lo), int(q_hi) + 1):          # union over the call's queries
        seen |= visible(c, w, listed, tpos, tsp, tnew, p)
    present = np.bincount(tpage[tpos <= int(q_hi)], minlength=len(pages))
    out = [(phys_of(storage, chain_ptr, r, int(i)), pages[i]["pos_start"], int(present[i]))
           for i in np.unique(tpage[seen])]            # chain order = ascending position
    return np.asarray(out, np.int64).reshape(-1, 3)


def tables(lay, storage, chain_ptr, q_lo, q_hi):
    """Per-(slot, seq) page tables for a call whose queries span [q_lo[seq], q_hi[seq]].

    Returns (row_ptr, entries) with entries an int64 array [n, 3] of
    (phys, pos_start, n_valid), rows ordered slot-major (row = slot * n_seq + seq).
    """
    rows = lay.n_slot * lay.n_seq
    row_ptr = np.zeros(rows + 1, np.int64)
    out = []
    for slot in range(lay.n_slot):
        for seq in range(lay.n_seq):
            r = slot * lay.n_seq + seq
            t = row_table(lay, storage, chain_ptr, slot, seq, q_lo[seq], q_hi[seq])
            out.append(t)
            row_ptr[r + 1] = row_ptr[r] + len(t)
    ent = np.concatenate(out) if out else np.zeros((0, 3), np.int64)
    return row_ptr, ent


def reloc_list(lay, storage, chain_ptr, rows=None):
    """[(phys, delta, n_valid)] for every stored segment page, allocation order
    (optionally only for the listed rows, row = slot * n_seq + seq)."""
    out = []
    chains = {}
    for slot in range(lay.n_slot):
        for seq in range(lay.n_seq):
            r = slot * lay.n_seq + seq
            if rows is not None and r not in rows:
                continue
            if seq not in chains:
                chains[seq] = chain(lay, seq)
            for i, pg in enumerate(chains[seq]):
                if pg["seg"] < 0 or storage[chain_ptr[r] + i] < 0:      # new-token page, or not stored
                    continue
                s = pg["seg"]
                delta = int(lay.seg_online[seq][s]) - int(lay.seg_offline[seq][s])
                out.append((int(storage[chain_ptr[r] + i]), delta, pg["n_valid"]))
    return np.asarray(out, np.int64).reshape(-1, 3)


def visible_counts(lay, slot: int, seq: int, q_pos):
    """Number of visible tokens of each query position (used by the count checks)."""
    tpos, _tpage, tsp, tnew = tokens(lay, seq)
    listed = lay.ret_pages.get((slot, seq), [])
    c, w = int(lay.cls[slot]), int(lay.window[slot])
    return np.asarray([np.count_nonzero(visible(c, w, listed, tpos, tsp, tnew, int(p))) for p in q_pos],
                      np.int64)


# ------------------------------------------------------------------ window-only storage and release

def seq_end(lay, seq: int) -> int:
    """One past the last position a query of the sequence can take."""
    return int(lay.new_base[seq]) + lay.n_new


def needed_pages(lay, slot: int, seq: int, p_from: int):
    """Boolean per chain page: does some query at a position in [p_from, end)
    see at least one of the page's tokens?  (Union of the visible sets.)"""
    tpos, tpage, tsp, tnew = tokens(lay, seq)
    listed = lay.ret_pages.get((slot, seq), [])
    c, w = int(lay.cls[slot]), int(lay.window[slot])
    seen = np.zeros(len(tpos), bool)
    for p in range(int(p_from), seq_end(lay, seq)):
        seen |= visible(c, w, listed, tpos, tsp, tnew, p)
    need = np.zeros(len(chain(lay, seq)), bool)
    need[np.unique(tpage[seen])] = True
    return need


def allocate_window(lay, free, keep_from):
    """Window-only storage: every head stores only the pages some query at a
    position in [keep_from[seq], end) can see.  Returns (storage, chain_ptr)
    over the full chains, with -1 for a page that is not stored."""
    storage, chain_ptr = [], np.zeros(lay.n_slot * lay.n_seq + 1, np.int64)
    k = 0
    for slot in range(lay.n_slot):
        for seq in range(lay.n_seq):
            r = slot * lay.n_seq + seq
            for needed in needed_pages(lay, slot, seq, keep_from[seq]):
                if needed:
                    if k >= len(free):
                        raise MemoryError(f"free list holds {len(free)} pages, more needed")
                    storage.append(int(free[k]))
                    k += 1
                else:
                    storage.append(-1)
            chain_ptr[r + 1] = len(storage)
    return np.asarray(storage, np.int64), chain_ptr


def release(lay, storage, chain_ptr, p_next):
    """Return to the free list every stored page that no query at a position in
    [p_next[seq], end) can see.  Returns (released ids in row order, then chain
    order; the storage with those ids set to -1)."""
    storage = np.asarray(storage, np.int64).copy()
    out = []
    for slot in range(lay.n_slot):
        for seq in range(lay.n_seq):
            r = slot * lay.n_seq + seq
            for i, needed in enumerate(needed_pages(lay, slot, seq, p_next[seq])):
                k = int(chain_ptr[r]) + i
                if storage[k] >= 0 and not needed:
                    out.append(int(storage[k]))
                    storage[k] = -1
    return np.asarray(out, np.int64), storage
