// segpaged_build_tables: segment/page allocation, per-head page tables and the
// relocation list (host only).
//
// Follows the per-head page tables over segmented paged KV storage (RedKnot
// product profile, section 3; is96.com commentary, SegPagedAttention
// paragraphs) and block-table allocation from a global free pool (the
// PagedAttention page, "The Solution: Fixed-size blocks").  Allocation order and
// the table rule are documented in include/segpaged.h.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "internal.hpp"

namespace {

struct SeqInfo {
    int64_t seg_pages = 0;   // pages holding segment tokens
    int64_t new_pages = 0;   // pages holding the new tokens
    int64_t end = 0;         // E: first new-token position
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Walks the table of one (slot, seq) row in ascending position and calls
// emit(chain_index, pos_start, n_valid) for every page the call's queries see.
template <class Emit>
void walk_row(int cls, int window, const sp_segment *segs, int n_segs, const SeqInfo &si,
              int n_new, int q_lo, int q_hi, int ps, const int32_t *listed, int n_listed,
              Emit emit) {
    // segment pages
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
        int s = 0;
        int64_t first = 0;  // ordinal of segment s's first page
        for (int k = 0; k < n_listed; ++k) {
            const int64_t o = listed[k];
            while (first + cdiv(segs[s].len, ps) <= o) first += cdiv(segs[s].len, ps), ++s;
            const int64_t j = o - first, len = segs[s].len;
            emit(o, segs[s].online_base + j * ps, std::min<int64_t>(ps, len - j * ps));
        }
        ci = si.seg_pages;
    }
    ci = si.seg_pages;
    // new-token pages: tokens at positions <= q_hi exist at this call
    const int64_t lo = (cls == SP_LOCAL) ? (int64_t)q_lo - window + 1 : INT64_MIN;
    for (int64_t j = 0; j < si.new_pages; ++j) {
        const int64_t start = si.end + j * ps;
        if (start > q_hi) break;
        const int64_t cap = std::min<int64_t>(ps, n_new - j * ps);
        const int64_t present = std::min<int64_t>(cap, (int64_t)q_hi - start + 1);
        if (start + present - 1 < lo) continue;
        emit(ci + j, start, present);
    }
}

}  // namespace

// Sorts relocation items by physical page (ids are distinct).  Dense pools
// (ids below 8x the item count) take one bucket pass, others a comparison sort.
static void sort_by_phys(sp_reloc *rl, int64_t n) {
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
        std::sort(rl, rl + n, [](const sp_reloc &a, const sp_reloc &b) { return a.phys < b.phys; });
    }
}

extern "C" int segpaged_build_tables(int n_seq, const int32_t *seg_ptr, const sp_segment *segs,
                                     const int32_t *n_new, const int32_t *q_lo, const int32_t *q_hi,
                                     int n_slot, const int32_t *cls, const int32_t *window,
                                     const int32_t *ret_ptr, const int32_t *ret_pages,
                                     int page_size, int64_t n_free, const int32_t *free_list,
                                     int32_t *chain_ptr, int32_t *storage, int32_t *row_ptr,
                                     sp_entry *entries, sp_reloc *reloc, int64_t counts[3]) {
    using sp::fail;
    sp::clear_error();
    if (!counts) return fail(SP_EINVAL, "counts is NULL");
    counts[0] = counts[1] = counts[2] = 0;
    if (n_seq < 1 || n_slot < 1) return fail(SP_EINVAL, "n_seq=%d n_slot=%d must be >= 1", n_seq, n_slot);
    if (page_size < 1) return fail(SP_EINVAL, "page_size=%d must be >= 1", page_size);
    if (!seg_ptr || !n_new || !q_lo || !q_hi || !cls || !window)
        return fail(SP_EINVAL, "a layout array is NULL");
    if ((int64_t)n_slot * n_seq > INT32_MAX - 1) return fail(SP_EINVAL, "too many rows");
    const int n_rows = n_slot * n_seq;
    if (seg_ptr[0] != 0) return fail(SP_EINVAL, "seg_ptr[0] must be 0");
    if (seg_ptr[n_seq] > 0 && !segs) return fail(SP_EINVAL, "segs is NULL");
    const int ps = page_size;

    // ---- sequences
    std::vector<SeqInfo> si(n_seq);
    for (int q = 0; q < n_seq; ++q) {
        if (seg_ptr[q + 1] < seg_ptr[q]) return fail(SP_EINVAL, "seg_ptr not ascending at %d", q);
        int64_t end = 0, pages = 0;
        for (int s = seg_ptr[q]; s < seg_ptr[q + 1]; ++s) {
            const sp_segment &g = segs[s];
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
        if (n_new[q] < 1) return fail(SP_EINVAL, "seq %d: n_new %d < 1", q, n_new[q]);
        if (end + n_new[q] > INT32_MAX) return fail(SP_EINVAL, "seq %d: new-token positions overflow int32", q);
        if (q_lo[q] < end || q_hi[q] < q_lo[q] || q_hi[q] >= end + n_new[q])
            return fail(SP_EINVAL, "seq %d: query range [%d, %d] outside the new tokens [%lld, %lld)", q, q_lo[q],
                        q_hi[q], (long long)end, (long long)(end + n_new[q]));
        si[q].seg_pages = pages;
        si[q].new_pages = cdiv(n_new[q], ps);
        si[q].end = end;
    }

    // ---- slots
    bool any_ret = false;
    for (int s = 0; s < n_slot; ++s) {
        if (cls[s] < SP_GLOBAL || cls[s] > SP_DENSE) return fail(SP_EINVAL, "slot %d: class %d", s, cls[s]);
        if (cls[s] == SP_LOCAL && window[s] < 1) return fail(SP_EINVAL, "slot %d: local window %d < 1", s, window[s]);
        any_ret |= cls[s] == SP_RETRIEVAL;
    }
    if (any_ret && (!ret_ptr || !ret_pages)) return fail(SP_EINVAL, "retrieval slot without ret_ptr/ret_pages");
    if (ret_ptr) {
        if (ret_ptr[0] != 0) return fail(SP_EINVAL, "ret_ptr[0] must be 0");
        if (ret_ptr[n_rows] > 0 && !ret_pages) return fail(SP_EINVAL, "ret_pages is NULL");
        for (int r = 0; r < n_rows; ++r) {
            const int slot = r / n_seq, q = r % n_seq;
            const int a = ret_ptr[r], b = ret_ptr[r + 1];
            if (b < a) return fail(SP_EINVAL, "ret_ptr not ascending at row %d", r);
            if (cls[slot] != SP_RETRIEVAL && b > a) return fail(SP_EINVAL, "row %d lists pages but is not retrieval", r);
            for (int k = a; k < b; ++k) {
                if (ret_pages[k] < 0 || ret_pages[k] >= si[q].seg_pages)
                    return fail(SP_EINVAL, "row %d: listed page %d outside [0, %lld)", r, ret_pages[k],
                                (long long)si[q].seg_pages);
                if (k > a && ret_pages[k] <= ret_pages[k - 1])
                    return fail(SP_EINVAL, "row %d: listed pages not strictly ascending", r);
            }
        }
    }

    // ---- counts
    int64_t total_pages = 0, total_reloc = 0;
    for (int q = 0; q < n_seq; ++q) {
        total_pages += si[q].seg_pages + si[q].new_pages;
        total_reloc += si[q].seg_pages;
    }
    total_pages *= n_slot;
    total_reloc *= n_slot;
    if (total_pages > INT32_MAX) return fail(SP_EINVAL, "%lld pages overflow int32", (long long)total_pages);
    auto listed_of = [&](int r, const int32_t **p, int *n) {
        if (ret_ptr) { *p = ret_pages + ret_ptr[r]; *n = ret_ptr[r + 1] - ret_ptr[r]; }
        else { *p = nullptr; *n = 0; }
    };
    int64_t total_entries = 0;
    for (int r = 0; r < n_rows; ++r) {
        const int slot = r / n_seq, q = r % n_seq;
        const int32_t *lp; int ln;
        listed_of(r, &lp, &ln);
        int64_t n = 0;
        walk_row(cls[slot], window[slot], segs + seg_ptr[q], seg_ptr[q + 1] - seg_ptr[q], si[q], n_new[q],
                 q_lo[q], q_hi[q], ps, lp, ln, [&](int64_t, int64_t, int64_t) { ++n; });
        if (n == 0) return fail(SP_EINVAL, "row %d: empty table", r);
        total_entries += n;
    }
    if (total_entries > INT32_MAX) return fail(SP_EINVAL, "%lld entries overflow int32", (long long)total_entries);
    counts[0] = total_pages;
    counts[1] = total_entries;
    counts[2] = total_reloc;
    const bool any_out = chain_ptr || storage || row_ptr || entries || reloc;
    if (!any_out) return SP_OK;   // count query
    if (!(chain_ptr && storage && row_ptr && entries && reloc))
        return fail(SP_EINVAL, "outputs must be all NULL (count query) or all non-NULL");
    if (n_free < total_pages)
        return fail(SP_ENOMEM, "free list holds %lld pages, %lld needed", (long long)n_free, (long long)total_pages);
    if (!free_list) return fail(SP_EINVAL, "free_list is NULL");

    // ---- the consumed prefix of the free list: non-negative and distinct
    int32_t mx = 0;
    for (int64_t i = 0; i < total_pages; ++i) {
        if (free_list[i] < 0) return fail(SP_EINVAL, "free_list[%lld] = %d is negative", (long long)i, free_list[i]);
        mx = std::max(mx, free_list[i]);
    }
    {
        std::vector<uint64_t> seen(((size_t)mx >> 6) + 1, 0);
        for (int64_t i = 0; i < total_pages; ++i) {
            const uint32_t v = (uint32_t)free_list[i];
            uint64_t &w = seen[v >> 6];
            const uint64_t bit = 1ull << (v & 63);
            if (w & bit) return fail(SP_EINVAL, "free_list repeats page %d", free_list[i]);
            w |= bit;
        }
    }

    // ---- storage: allocation order pops the free list from the front
    chain_ptr[0] = 0;
    for (int r = 0; r < n_rows; ++r) {
        const int q = r % n_seq;
        chain_ptr[r + 1] = chain_ptr[r] + (int32_t)(si[q].seg_pages + si[q].new_pages);
    }
    std::memcpy(storage, free_list, sizeof(int32_t) * (size_t)total_pages);

    // ---- relocation list, ascending physical page: the relocation then sweeps
    // the pool in address order instead of gathering pages scattered by the
    // free list (items are independent, so their order is free)
    int64_t k = 0;
    for (int r = 0; r < n_rows; ++r) {
        const int q = r % n_seq;
        int64_t ci = chain_ptr[r];
        for (int s = seg_ptr[q]; s < seg_ptr[q + 1]; ++s) {
            const sp_segment &g = segs[s];
            const int32_t delta = g.online_base - g.offline_base;
            for (int64_t j = 0; j * ps < g.len; ++j)
                reloc[k++] = sp_reloc{storage[ci++], delta, (int32_t)std::min<int64_t>(ps, g.len - j * ps), 0};
        }
    }
    sort_by_phys(reloc, k);

    // ---- tables
    row_ptr[0] = 0;
    int64_t e = 0;
    for (int r = 0; r < n_rows; ++r) {
        const int slot = r / n_seq, q = r % n_seq;
        const int32_t *lp; int ln;
        listed_of(r, &lp, &ln);
        const int32_t *chain = storage + chain_ptr[r];
        walk_row(cls[slot], window[slot], segs + seg_ptr[q], seg_ptr[q + 1] - seg_ptr[q], si[q], n_new[q],
                 q_lo[q], q_hi[q], ps, lp, ln, [&](int64_t ci, int64_t start, int64_t n) {
                     entries[e++] = sp_entry{chain[ci], (int32_t)start, (int32_t)n, 0};
                 });
        row_ptr[r + 1] = (int32_t)e;
    }
    return SP_OK;
}
