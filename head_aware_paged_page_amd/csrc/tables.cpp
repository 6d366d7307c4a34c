// Host side of the per-head page tables: segment/page allocation (whole chains
// or window-only), the tables of a call, the relocation list, and the release
// of pages no later query can read.
//
// Follows the per-head page tables over segmented paged KV storage (RedKnot
// product profile, section 3; is96.com commentary, SegPagedAttention
// paragraphs: each head's pages hold only its own KV, and local heads keep only
// window-sized KV, its deployment paragraph) and block-table allocation from a
// global free pool with blocks returned at the end of a sequence (the
// PagedAttention page, "The Solution: Fixed-size blocks" and its walk-through).
// Allocation order and the table rule are documented in include/segpaged.h.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <vector>

#include "internal.hpp"

namespace {

using sp::fail;

struct SeqInfo {
    int64_t seg_pages = 0;   // pages holding segment tokens
    int64_t new_pages = 0;   // pages holding the new tokens
    int64_t end = 0;         // E: first new-token position
    int64_t stop = 0;        // E + n_new: one past the last position a query can take
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A checked layout: the arguments every host call shares.
struct Layout {
    const sp_layout *a = nullptr;
    int n_rows = 0;
    std::vector<SeqInfo> si;
    int64_t chain_pages = 0;   // sum of all chains' lengths

    int chain_len(int q) const { return (int)(si[q].seg_pages + si[q].new_pages); }
    void listed(int r, const int32_t **p, int *n) const {
        if (a->ret_ptr) { *p = a->ret_pages + a->ret_ptr[r]; *n = a->ret_ptr[r + 1] - a->ret_ptr[r]; }
        else { *p = nullptr; *n = 0; }
    }
};

int check_layout(const sp_layout *a, Layout *L) {
    if (!a) return fail(SP_EINVAL, "layout is NULL");
    const int n_seq = a->n_seq, n_slot = a->n_slot, ps = a->page_size;
    if (n_seq < 1 || n_slot < 1) return fail(SP_EINVAL, "n_seq=%d n_slot=%d must be >= 1", n_seq, n_slot);
    if (ps < 1) return fail(SP_EINVAL, "page_size=%d must be >= 1", ps);
    if (!a->seg_ptr || !a->n_new || !a->cls || !a->window) return fail(SP_EINVAL, "a layout array is NULL");
    if ((int64_t)n_slot * n_seq > INT32_MAX - 1) return fail(SP_EINVAL, "too many rows");
    const int n_rows = n_slot * n_seq;
    if (a->seg_ptr[0] != 0) return fail(SP_EINVAL, "seg_ptr[0] must be 0");
    if (a->seg_ptr[n_seq] > 0 && !a->segs) return fail(SP_EINVAL, "segs is NULL");
    L->a = a;
    L->n_rows = n_rows;
    L->si.assign(n_seq, SeqInfo{});
    for (int q = 0; q < n_seq; ++q) {
        if (a->seg_ptr[q + 1] < a->seg_ptr[q]) return fail(SP_EINVAL, "seg_ptr not ascending at %d", q);
        int64_t end = 0, pages = 0;
        for (int s = a->seg_ptr[q]; s < a->seg_ptr[q + 1]; ++s) {
            const sp_segment &g = a->segs[s];
            if (g.len < 1) return fail(SP_EINVAL, "seq %d segment %d: len %d < 1", q, s, g.len);
            if (g.online_base < end)
                return fail(SP_EINVAL, "seq %d segment %d: online_base %d overlaps or precedes the previous segment",
                            q, s, g.online_base);
            if ((int64_t)g.online_base + g.len > INT32_MAX)
                return fail(SP_EINVAL, "seq %d segment %d: positions overflow int32", q, s);
            const int64_t delta = (int64_t)g.online_base - g.offline_base;
            if (delta > INT32_MAX || delta < INT32_MIN)
                return fail(SP_EINVAL, "seq %d segment %d: position shift overflows int32", q, s);
            end = (int64_t)g.online_base + g.len;
            pages += cdiv(g.len, ps);
        }
        if (a->n_new[q] < 1) return fail(SP_EINVAL, "seq %d: n_new %d < 1", q, a->n_new[q]);
        if (end + a->n_new[q] > INT32_MAX) return fail(SP_EINVAL, "seq %d: new-token positions overflow int32", q);
        L->si[q] = SeqInfo{pages, cdiv(a->n_new[q], ps), end, end + a->n_new[q]};
    }
    bool any_ret = false;
    for (int s = 0; s < n_slot; ++s) {
        if (a->cls[s] < SP_GLOBAL || a->cls[s] > SP_DENSE) return fail(SP_EINVAL, "slot %d: class %d", s, a->cls[s]);
        if (a->cls[s] == SP_LOCAL && a->window[s] < 1)
            return fail(SP_EINVAL, "slot %d: local window %d < 1", s, a->window[s]);
        any_ret |= a->cls[s] == SP_RETRIEVAL;
    }
    if (any_ret && (!a->ret_ptr || !a->ret_pages)) return fail(SP_EINVAL, "retrieval slot without ret_ptr/ret_pages");
    if (a->ret_ptr) {
        if (a->ret_ptr[0] != 0) return fail(SP_EINVAL, "ret_ptr[0] must be 0");
        if (a->ret_ptr[n_rows] > 0 && !a->ret_pages) return fail(SP_EINVAL, "ret_pages is NULL");
        for (int r = 0; r < n_rows; ++r) {
            const int slot = r / n_seq, q = r % n_seq;
            const int b0 = a->ret_ptr[r], b1 = a->ret_ptr[r + 1];
            if (b1 < b0) return fail(SP_EINVAL, "ret_ptr not ascending at row %d", r);
            if (a->cls[slot] != SP_RETRIEVAL && b1 > b0) return fail(SP_EINVAL, "row %d lists pages but is not retrieval", r);
            for (int k = b0; k < b1; ++k) {
                if (a->ret_pages[k] < 0 || a->ret_pages[k] >= L->si[q].seg_pages)
                    return fail(SP_EINVAL, "row %d: listed page %d outside [0, %lld)", r, a->ret_pages[k],
                                (long long)L->si[q].seg_pages);
                if (k > b0 && a->ret_pages[k] <= a->ret_pages[k - 1])
                    return fail(SP_EINVAL, "row %d: listed pages not strictly ascending", r);
            }
        }
    }
    int64_t total = 0;
    for (int q = 0; q < n_seq; ++q) total += L->si[q].seg_pages + L->si[q].new_pages;
    total *= n_slot;
    if (total > INT32_MAX) return fail(SP_EINVAL, "%lld pages overflow int32", (long long)total);
    L->chain_pages = total;
    return SP_OK;
}

// Query ranges of a call: E <= q_lo <= q_hi < E + n_new.
int check_queries(const Layout &L, const int32_t *q_lo, const int32_t *q_hi) {
    if (!q_lo || !q_hi) return fail(SP_EINVAL, "q_lo/q_hi is NULL");
    for (int q = 0; q < L.a->n_seq; ++q)
        if (q_lo[q] < L.si[q].end || q_hi[q] < q_lo[q] || q_hi[q] >= L.si[q].stop)
            return fail(SP_EINVAL, "seq %d: query range [%d, %d] outside the new tokens [%lld, %lld)", q, q_lo[q],
                        q_hi[q], (long long)L.si[q].end, (long long)L.si[q].stop);
    return SP_OK;
}

// Calls fn(chain_index, pos_start, n_tokens) for every page of row r's chain in
// chain order (= ascending position); n_tokens counts every token the page will
// ever hold (new-token pages at full capacity).
template <class Fn>
void for_each_page(const Layout &L, int r, Fn fn) {
    const sp_layout &a = *L.a;
    const int q = r % a.n_seq, ps = a.page_size;
    const SeqInfo &si = L.si[q];
    int64_t ci = 0;
    for (int s = a.seg_ptr[q]; s < a.seg_ptr[q + 1]; ++s) {
        const int64_t len = a.segs[s].len, on = a.segs[s].online_base;
        for (int64_t j = 0; j * ps < len; ++j, ++ci) fn(ci, on + j * ps, std::min<int64_t>(ps, len - j * ps), s);
    }
    for (int64_t j = 0; j < si.new_pages; ++j, ++ci)
        fn(ci, si.end + j * ps, std::min<int64_t>(ps, (int64_t)a.n_new[q] - j * ps), -1);
}

// needed[ci] = 1 if some query of row r at a position in [p_from, E + n_new)
// can see a token of chain page ci: none once the sequence is over; for a
// local(W) head the pages whose last position is >= p_from - W + 1 (a token t
// is seen by the query at t, and the largest such p_from is t + W - 1); for a
// retrieval head its listed segment pages and the new-token pages; otherwise
// every page.
void needed_pages(const Layout &L, int r, int64_t p_from, std::vector<uint8_t> *needed) {
    const sp_layout &a = *L.a;
    const int slot = r / a.n_seq, q = r % a.n_seq;
    needed->assign((size_t)L.chain_len(q), 0);
    if (p_from >= L.si[q].stop) return;
    const int c = a.cls[slot];
    if (c == SP_LOCAL) {
        const int64_t lo = p_from - a.window[slot] + 1;
        for_each_page(L, r, [&](int64_t ci, int64_t start, int64_t n, int) { (*needed)[ci] = start + n - 1 >= lo; });
    } else if (c == SP_RETRIEVAL) {
        const int32_t *lp; int ln;
        L.listed(r, &lp, &ln);
        for (int k = 0; k < ln; ++k) (*needed)[lp[k]] = 1;
        for (int64_t j = 0; j < L.si[q].new_pages; ++j) (*needed)[L.si[q].seg_pages + j] = 1;
    } else {
        std::fill(needed->begin(), needed->end(), 1);
    }
}

// Walks the table of one (slot, seq) row in ascending position and calls
// emit(chain_index, pos_start, n_valid) for every page the call's queries see.
template <class Emit>
void walk_row(const Layout &L, int r, int q_lo, int q_hi, Emit emit) {
    const sp_layout &a = *L.a;
    const int slot = r / a.n_seq, q = r % a.n_seq, ps = a.page_size;
    const int cls = a.cls[slot], window = a.window[slot];
    const sp_segment *segs = a.segs + a.seg_ptr[q];
    const int n_segs = a.seg_ptr[q + 1] - a.seg_ptr[q];
    const SeqInfo &si = L.si[q];
    int64_t ci = 0;  // chain index (= segment-page ordinal for segment pages)
    if (cls == SP_GLOBAL || cls == SP_DENSE) {
        for (int s = 0; s < n_segs; ++s) {
            const int64_t len = segs[s].len, on = segs[s].online_base;
            for (int64_t j = 0; j * ps < len; ++j, ++ci)
                emit(ci, on + j * ps, std::min<int64_t>(ps, len - j * ps));
        }
    } else if (cls == SP_LOCAL) {
        // union of the windows (p - W, p] over p in [q_lo, q_hi]
        const int64_t lo = (int64_t)q_lo - window + 1;
        for (int s = 0; s < n_segs; ++s) {
            const int64_t len = segs[s].len, on = segs[s].online_base;
            const int64_t np = cdiv(len, ps);
            int64_t j0 = 0;
            if (on + len - 1 < lo) j0 = np;                 // whole segment left of every window
            else if (lo > on) j0 = (lo - on) / ps;          // first page reaching position lo
            for (int64_t j = j0; j < np; ++j)
                emit(ci + j, on + j * ps, std::min<int64_t>(ps, len - j * ps));
            ci += np;
        }
    } else {  // SP_RETRIEVAL: the listed segment pages
        const int32_t *listed; int n_listed;
        L.listed(r, &listed, &n_listed);
        int s = 0;
        int64_t first = 0;  // ordinal of segment s's first page
        for (int k = 0; k < n_listed; ++k) {
            const int64_t o = listed[k];
            while (first + cdiv(segs[s].len, ps) <= o) first += cdiv(segs[s].len, ps), ++s;
            const int64_t j = o - first, len = segs[s].len;
            emit(o, segs[s].online_base + j * ps, std::min<int64_t>(ps, len - j * ps));
        }
    }
    ci = si.seg_pages;
    // new-token pages: tokens at positions <= q_hi exist at this call
    const int64_t lo = (cls == SP_LOCAL) ? (int64_t)q_lo - window + 1 : INT64_MIN;
    const int n_new = a.n_new[q];
    for (int64_t j = 0; j < si.new_pages; ++j) {
        const int64_t start = si.end + j * ps;
        if (start > q_hi) break;
        const int64_t cap = std::min<int64_t>(ps, n_new - j * ps);
        const int64_t present = std::min<int64_t>(cap, (int64_t)q_hi - start + 1);
        if (start + present - 1 < lo) continue;
        emit(ci + j, start, present);
    }
}

// Tables of a call over given chains.  Count pass when entries is NULL.
int make_tables(const Layout &L, const int32_t *q_lo, const int32_t *q_hi, const int32_t *chain_ptr,
                const int32_t *storage, int32_t *row_ptr, sp_entry *entries, int64_t *n_entries) {
    int64_t e = 0;
    if (row_ptr) row_ptr[0] = 0;
    for (int r = 0; r < L.n_rows; ++r) {
        const int q = r % L.a->n_seq;
        int64_t n = 0;
        int bad = -1;
        walk_row(L, r, q_lo[q], q_hi[q], [&](int64_t ci, int64_t start, int64_t nv) {
            const int32_t phys = storage ? storage[chain_ptr[r] + ci] : 0;
            if (phys < 0 && bad < 0) bad = (int)ci;
            if (entries) entries[e + n] = sp_entry{phys, (int32_t)start, (int32_t)nv, 0};
            ++n;
        });
        if (n == 0) return fail(SP_EINVAL, "row %d: empty table", r);
        if (bad >= 0)
            return fail(SP_EINVAL, "row %d: the call's queries read chain page %d, which is not stored (released, "
                                   "or outside the window the storage was built for)", r, bad);
        e += n;
        if (e > INT32_MAX) return fail(SP_EINVAL, "%lld entries overflow int32", (long long)e);
        if (row_ptr) row_ptr[r + 1] = (int32_t)e;
    }
    *n_entries = e;
    return SP_OK;
}

// Sorts relocation items by physical page (ids are distinct).  Dense pools
// (ids below 8x the item count) take one bucket pass, others a comparison sort.
void sort_by_phys(sp_reloc *rl, int64_t n) {
    if (n < 2) return;
    int32_t mx = 0;
    for (int64_t i = 0; i < n; ++i) mx = std::max(mx, rl[i].phys);
    if ((int64_t)mx < 8 * n + 1024) {
        std::vector<int64_t> at((size_t)mx + 1, -1);
        for (int64_t i = 0; i < n; ++i) at[rl[i].phys] = i;
        std::vector<sp_reloc> out;
        out.reserve((size_t)n);
        for (int32_t p = 0; p <= mx; ++p)
            if (at[p] >= 0) out.push_back(rl[at[p]]);
        std::copy(out.begin(), out.end(), rl);
    } else {
        std::sort(rl, rl + n, [](const sp_reloc &x, const sp_reloc &y) { return x.phys < y.phys; });
    }
}

// Free-list ids used must be non-negative and distinct.
int check_free_prefix(const int32_t *free_list, int64_t n) {
    int32_t mx = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (free_list[i] < 0) return fail(SP_EINVAL, "free_list[%lld] = %d is negative", (long long)i, free_list[i]);
        mx = std::max(mx, free_list[i]);
    }
    std::vector<uint64_t> seen(((size_t)mx >> 6) + 1, 0);
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t v = (uint32_t)free_list[i];
        uint64_t &w = seen[v >> 6];
        const uint64_t bit = 1ull << (v & 63);
        if (w & bit) return fail(SP_EINVAL, "free_list repeats page %d", free_list[i]);
        w |= bit;
    }
    return SP_OK;
}

}  // namespace

extern "C" int segpaged_build_tables_ex(const sp_layout *lay, const int32_t *q_lo, const int32_t *q_hi,
                                        const int32_t *keep_from, int64_t n_free, const int32_t *free_list,
                                        int32_t *chain_ptr, int32_t *storage, int32_t *row_ptr, sp_entry *entries,
                                        sp_reloc *reloc, int64_t counts[4]) {
    sp::clear_error();
    if (!counts) return fail(SP_EINVAL, "counts is NULL");
    counts[0] = counts[1] = counts[2] = counts[3] = 0;
    Layout L;
    int rc = check_layout(lay, &L);
    if (rc) return rc;
    rc = check_queries(L, q_lo, q_hi);
    if (rc) return rc;
    const int n_seq = lay->n_seq;
    if (keep_from)
        for (int q = 0; q < n_seq; ++q)
            if (keep_from[q] < 0 || keep_from[q] > q_lo[q])
                return fail(SP_EINVAL, "seq %d: keep_from %d outside [0, q_lo = %d]", q, keep_from[q], q_lo[q]);

    // stored pages per row (all of them without keep_from)
    int64_t taken = 0, n_reloc = 0;
    std::vector<std::vector<uint8_t>> needed(keep_from ? L.n_rows : 0);
    for (int r = 0; r < L.n_rows; ++r) {
        const int q = r % n_seq;
        if (keep_from) {
            needed_pages(L, r, keep_from[q], &needed[r]);
            for (int64_t ci = 0; ci < L.chain_len(q); ++ci)
                if (needed[r][ci]) {
                    ++taken;
                    n_reloc += ci < L.si[q].seg_pages;
                }
        } else {
            taken += L.chain_len(q);
            n_reloc += L.si[q].seg_pages;
        }
    }
    int64_t n_ent = 0;
    rc = make_tables(L, q_lo, q_hi, chain_ptr, nullptr, nullptr, nullptr, &n_ent);   // count and check rows
    if (rc) return rc;
    counts[0] = L.chain_pages;
    counts[1] = n_ent;
    counts[2] = n_reloc;
    counts[3] = taken;
    const bool any_out = chain_ptr || storage || row_ptr || entries || reloc;
    if (!any_out) return SP_OK;   // count query
    if (!(chain_ptr && storage && row_ptr && entries && reloc))
        return fail(SP_EINVAL, "outputs must be all NULL (count query) or all non-NULL");
    if (n_free < taken)
        return fail(SP_ENOMEM, "free list holds %lld pages, %lld needed", (long long)n_free, (long long)taken);
    if (!free_list) return fail(SP_EINVAL, "free_list is NULL");
    rc = check_free_prefix(free_list, taken);
    if (rc) return rc;

    // storage: allocation order (slot -> seq -> segment -> page -> new pages)
    // pops the free list from the front, skipping pages that are not stored
    chain_ptr[0] = 0;
    int64_t k = 0;
    for (int r = 0; r < L.n_rows; ++r) {
        const int q = r % n_seq;
        const int n = L.chain_len(q);
        chain_ptr[r + 1] = chain_ptr[r] + n;
        for (int ci = 0; ci < n; ++ci)
            storage[chain_ptr[r] + ci] = (!keep_from || needed[r][ci]) ? free_list[k++] : -1;
    }

    // relocation list, ascending physical page: the relocation then sweeps the
    // pool in address order instead of gathering pages scattered by the free
    // list (items are independent, so their order is free)
    int64_t m = 0;
    for (int r = 0; r < L.n_rows; ++r) {
        for_each_page(L, r, [&](int64_t ci, int64_t, int64_t n, int s) {
            const int32_t phys = storage[chain_ptr[r] + ci];
            if (s < 0 || phys < 0) return;
            const sp_segment &g = lay->segs[s];
            reloc[m++] = sp_reloc{phys, g.online_base - g.offline_base, (int32_t)n, 0};
        });
    }
    sort_by_phys(reloc, m);

    return make_tables(L, q_lo, q_hi, chain_ptr, storage, row_ptr, entries, &n_ent);
}

extern "C" int segpaged_build_tables(int n_seq, const int32_t *seg_ptr, const sp_segment *segs,
                                     const int32_t *n_new, const int32_t *q_lo, const int32_t *q_hi,
                                     int n_slot, const int32_t *cls, const int32_t *window,
                                     const int32_t *ret_ptr, const int32_t *ret_pages,
                                     int page_size, int64_t n_free, const int32_t *free_list,
                                     int32_t *chain_ptr, int32_t *storage, int32_t *row_ptr,
                                     sp_entry *entries, sp_reloc *reloc, int64_t counts[3]) {
    if (!counts) {
        sp::clear_error();
        return fail(SP_EINVAL, "counts is NULL");
    }
    const sp_layout lay{n_seq, seg_ptr, segs, n_new, n_slot, cls, window, ret_ptr, ret_pages, page_size};
    int64_t c4[4];
    const int rc = segpaged_build_tables_ex(&lay, q_lo, q_hi, nullptr, n_free, free_list, chain_ptr, storage,
                                            row_ptr, entries, reloc, c4);
    counts[0] = c4[0];
    counts[1] = c4[1];
    counts[2] = c4[2];
    return rc;
}

extern "C" int segpaged_tables_from_chains(const sp_layout *lay, const int32_t *q_lo, const int32_t *q_hi,
                                           const int32_t *chain_ptr, const int32_t *storage, int32_t *row_ptr,
                                           sp_entry *entries, int64_t *n_entries) {
    sp::clear_error();
    if (!n_entries) return fail(SP_EINVAL, "n_entries is NULL");
    *n_entries = 0;
    Layout L;
    int rc = check_layout(lay, &L);
    if (rc) return rc;
    rc = check_queries(L, q_lo, q_hi);
    if (rc) return rc;
    if (!chain_ptr || !storage) return fail(SP_EINVAL, "chain_ptr/storage is NULL");
    for (int r = 0; r < L.n_rows; ++r)
        if (chain_ptr[r + 1] - chain_ptr[r] != L.chain_len(r % lay->n_seq) || (r == 0 && chain_ptr[0] != 0))
            return fail(SP_EINVAL, "chain_ptr does not match the layout at row %d", r);
    if ((entries == nullptr) != (row_ptr == nullptr))
        return fail(SP_EINVAL, "row_ptr and entries must both be NULL (count query) or both non-NULL");
    return make_tables(L, q_lo, q_hi, chain_ptr, storage, row_ptr, entries, n_entries);
}

extern "C" int segpaged_release_pages(const sp_layout *lay, const int32_t *p_next, const int32_t *chain_ptr,
                                      int32_t *storage, int32_t *released, int64_t *n_released) {
    sp::clear_error();
    if (!n_released) return fail(SP_EINVAL, "n_released is NULL");
    *n_released = 0;
    Layout L;
    int rc = check_layout(lay, &L);
    if (rc) return rc;
    if (!p_next || !chain_ptr || !storage || !released) return fail(SP_EINVAL, "a pointer is NULL");
    for (int q = 0; q < lay->n_seq; ++q)
        if (p_next[q] < L.si[q].end) return fail(SP_EINVAL, "seq %d: p_next %d before the new tokens (%lld)", q,
                                                 p_next[q], (long long)L.si[q].end);
    for (int r = 0; r < L.n_rows; ++r)
        if (chain_ptr[r + 1] - chain_ptr[r] != L.chain_len(r % lay->n_seq) || (r == 0 && chain_ptr[0] != 0))
            return fail(SP_EINVAL, "chain_ptr does not match the layout at row %d", r);
    std::vector<uint8_t> need;
    int64_t m = 0;
    for (int r = 0; r < L.n_rows; ++r) {
        needed_pages(L, r, p_next[r % lay->n_seq], &need);
        for (int64_t ci = 0; ci < (int64_t)need.size(); ++ci) {
            int32_t &id = storage[chain_ptr[r] + ci];
            if (id >= 0 && !need[ci]) {
                released[m++] = id;
                id = -1;
            }
        }
    }
    *n_released = m;
    return SP_OK;
}
