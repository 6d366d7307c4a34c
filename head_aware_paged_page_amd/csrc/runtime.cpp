// Host runtime of libsegpaged: errors, launch planning, argument validation and
// the device entry points (the kernels live in the .hip files).
#include <algorithm>
#include <functional>
#include <map>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.hpp"

namespace sp {

static thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = 0; }

int check_hip(hipError_t e, const char *what) {
    if (e == hipSuccess) return SP_OK;
    return fail(SP_EHIP, "%s: %s", what, hipGetErrorString(e));
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static bool bf16_supported(int head_dim) { return head_dim == 64 || head_dim == 128; }

int make_plan(int kind, int dtype, int head_dim, int page_size, int group, int n_seq, int n_slot,
              const int32_t *h_tok_ptr, const int32_t *h_row_ptr, Plan *plan) {
    if (kind != SP_WS_PREFILL && kind != SP_WS_DECODE) return fail(SP_EINVAL, "workspace kind %d", kind);
    if (dtype != SP_F32 && dtype != SP_BF16) return fail(SP_EINVAL, "dtype %d", dtype);
    if (n_seq < 1 || n_slot < 1) return fail(SP_EINVAL, "n_seq=%d n_slot=%d must be >= 1", n_seq, n_slot);
    if (group < 1 || group > 16) return fail(SP_EUNSUPPORTED, "group %d outside 1..16", group);
    if (head_dim < 16 || head_dim > 256 || head_dim % 16) return fail(SP_EUNSUPPORTED, "head_dim %d", head_dim);
    if (page_size < 1) return fail(SP_EINVAL, "page_size %d", page_size);
    if (!h_row_ptr) return fail(SP_EINVAL, "h_row_ptr is NULL");
    if (kind == SP_WS_PREFILL && !h_tok_ptr) return fail(SP_EINVAL, "h_tok_ptr is NULL");
    if ((int64_t)n_slot * n_seq > INT32_MAX - 1) return fail(SP_EINVAL, "too many rows");
    const int n_rows = n_slot * n_seq;
    if (h_row_ptr[0] != 0) return fail(SP_EINVAL, "row_ptr[0] must be 0");
    for (int r = 0; r < n_rows; ++r)
        if (h_row_ptr[r + 1] <= h_row_ptr[r]) return fail(SP_EINVAL, "row %d has an empty or negative table", r);
    if (kind == SP_WS_PREFILL) {
        if (h_tok_ptr[0] != 0) return fail(SP_EINVAL, "tok_ptr[0] must be 0");
        for (int q = 0; q < n_seq; ++q)
            if (h_tok_ptr[q + 1] < h_tok_ptr[q]) return fail(SP_EINVAL, "tok_ptr not ascending at %d", q);
    }

    Plan p;
    p.kind = kind;
    p.n_rows = n_rows;
    size_t off = 0;
    p.off_item_ptr = off; off += sizeof(int32_t) * (n_rows + 1);
    p.off_item_ptr2 = off; off += sizeof(int32_t) * (n_rows + 1);
    p.off_part_ptr = off; off += sizeof(int32_t) * (n_rows + 1);
    p.off_nsplit = off;   off += sizeof(int32_t) * n_rows;
    off = align_up(off, 256);
    p.off_zero = off;     off += 256;          // zero-filled by the plan kernel

    if (dtype == SP_F32) {
        // The fp32 kernels take one query token per workgroup and never split.
        p.rows_per_tile = group;
        p.tok_per_tile = 1;
        p.chunk_pages = INT_MAX;
        p.bytes = off + 256;
        p.off_part_o = p.off_part_lse = off;
        *plan = p;
        return SP_OK;
    }
    if (!bf16_supported(head_dim)) return fail(SP_EUNSUPPORTED, "bf16 head_dim %d (64 or 128)", head_dim);

    // work units (row, q-tile) and their page counts
    int64_t units = 0, work = 0;
    if (kind == SP_WS_PREFILL) {
        // 8 waves of 32 query rows: one staged K/V tile feeds 256 rows
        p.waves = 8;
        p.rows_per_tile = kPrefillRowsPerWave * p.waves;
        p.tok_per_tile = p.rows_per_tile / group;
        for (int r = 0; r < n_rows; ++r) {
            const int q = r % n_seq;
            const int64_t nt = h_tok_ptr[q + 1] - h_tok_ptr[q];
            const int64_t nq = (nt + p.tok_per_tile - 1) / p.tok_per_tile;
            units += nq;
            work += nq * (h_row_ptr[r + 1] - h_row_ptr[r]);
        }
    } else {
        p.rows_per_tile = group;
        p.tok_per_tile = 1;
        for (int r = 0; r < n_rows; ++r) {
            units += 1;
            work += h_row_ptr[r + 1] - h_row_ptr[r];
        }
    }
    const int min_chunk = std::max(1, (kind == SP_WS_PREFILL ? kMinSplitKeysPrefill : kMinSplitKeysDecode) / page_size);
    if (kind == SP_WS_PREFILL) {
        // One persistent workgroup per CU takes the items long-first from a
        // counter: list scheduling, longest item first.  Every candidate chunk
        // (the longest row split k ways, k = 1, 2, ...) is scored by running
        // that schedule over the items' estimated costs (64-key tiles of the
        // row's table plus a fixed set-up per item); the shortest makespan
        // wins, and a finer chunk must beat a coarser one by 1 %.  Items of a
        // row share one cost, so the schedule runs per cost class on a
        // histogram of CU loads: each class fills the least loaded CUs first.
        // A split item also writes its partial result (about a tile's time)
        // and the merge reads it back after the main pass (kMergeTiles per
        // item, spread over the CUs).  An item that holds an end of its row
        // (the start of a windowed row, the query tokens' own keys) pays for
        // the tiles there that need bounds or zeroed value slots; the host
        // cannot tell windowed rows from others, so every row start counts.
        // The kernel cuts a q-tile's visible pages into ns chunks of
        // ceil(pages / ns) rounded up to whole tiles; the last takes the rest.
        const int ppt = std::max(1, kPrefillKeysPerTile / page_size);
        auto cost = [&](int64_t pages, int edges) {
            return (double)((pages + ppt - 1) / ppt + kPrefillSetupTiles + edges * kPrefillEdgeTiles);
        };
        int e_max = 1;
        for (int r = 0; r < n_rows; ++r) e_max = std::max(e_max, h_row_ptr[r + 1] - h_row_ptr[r]);
        // A row's items depend only on its table length and its sequence's
        // token count, so rows are counted per (entries, tokens) once and each
        // candidate is scored per group rather than per row.
        std::map<std::pair<int, int>, int64_t> groups;
        for (int r = 0; r < n_rows; ++r) {
            const int q = r % n_seq;
            const int nt = h_tok_ptr[q + 1] - h_tok_ptr[q];
            if (nt > 0) groups[{h_row_ptr[r + 1] - h_row_ptr[r], nt}] += 1;
        }
        std::map<double, int64_t, std::greater<double>> cls;   // cost -> items, longest first
        std::map<double, int64_t> loads;                       // CU load -> CUs
        auto makespan = [&](int c, int64_t *n_items) {
            cls.clear();
            *n_items = 0;
            int64_t n_parts = 0;
            for (const auto &g : groups) {
                const int e = g.first.first, nt = g.first.second;
                const int64_t rows = g.second;
                const int nq = (nt + p.tok_per_tile - 1) / p.tok_per_tile;
                int ns, it;
                row_items(e, nq, c, &ns, &it);
                *n_items += rows * it;
                if (ns > 1) n_parts += rows * it;
                for (int j = 0; j < nq; ++j) {
                    // q-tile j sees at most the row's pages less those of the
                    // chunk's later tokens (exact for a row without a window)
                    const int t_end = std::min(nt, (j + 1) * p.tok_per_tile);
                    const int64_t v = std::max(1, e - (nt - t_end) / page_size);
                    if (ns == 1) {
                        cls[cost(v, 2)] += rows;
                        continue;
                    }
                    const int64_t ch = ((v + ns - 1) / ns + ppt - 1) / ppt * ppt;
                    const int64_t last = std::max<int64_t>(1, v - (int64_t)(ns - 1) * ch);
                    cls[cost(ch, 1) + 1.0] += rows;                       // first chunk: the row start
                    if (ns > 2) cls[cost(ch, 0) + 1.0] += rows * (ns - 2);
                    cls[cost(last, 1) + 1.0] += rows;                     // last chunk: the query tokens
                }
            }
            loads.clear();
            loads[0.0] = kPlanCUs;
            for (const auto &kv : cls) {
                int64_t n = kv.second;
                while (n > 0) {
                    auto lo = loads.begin();
                    const double lvl = lo->first;
                    const int64_t m = lo->second;
                    if (n >= m) {   // every CU at the lowest level takes items while it stays lowest
                        int64_t each = n / m;
                        const auto nx = std::next(lo);
                        if (nx != loads.end()) each = std::min<int64_t>(each, (int64_t)((nx->first - lvl) / kv.first) + 1);
                        loads.erase(lo);
                        loads[lvl + each * kv.first] += m;
                        n -= each * m;
                    } else {
                        lo->second -= n;
                        loads[lvl + kv.first] += n;
                        n = 0;
                    }
                }
            }
            return loads.rbegin()->first + kMergeTiles * (double)n_parts / kPlanCUs;
        };
        int64_t n0 = 0;
        double best = makespan(INT_MAX, &n0);
        int best_c = INT_MAX;
        for (int k = 2; k <= kMaxSplits; ++k) {
            const int c = (e_max + k - 1) / k;
            if (c < min_chunk) break;
            if (c == (e_max + k - 2) / (k - 1)) continue;   // same chunk as k-1
            int64_t n_items = 0;
            const double est = makespan(c, &n_items);
            if (est < 0.99 * best) {
                best = est;
                best_c = c;
            }
            if (n_items > 16 * kPlanCUs) break;   // finer chunks only add set-ups
        }
        p.chunk_pages = best_c;
    } else {
        // Every item is resident at once, and a CU's share of the HBM stream
        // depends on how many decode waves it holds: four per CU stream at
        // about 4.5 TB/s chip-wide, eight at about 6.6, and a CU holding more
        // than the rest finishes last.  So the chunk is the finest whose items
        // fit kDecodeWgPerCU per CU (one workgroup of eight waves; two of four
        // measured slightly slower, their items and partials twice as many);
        // the item count falls as the chunk grows, so a bisection finds it.
        // Rows that alone outnumber that fall back to a fixed item target.
        int e_max = 1;
        for (int r = 0; r < n_rows; ++r) e_max = std::max(e_max, h_row_ptr[r + 1] - h_row_ptr[r]);
        auto n_items = [&](int c) {
            int64_t n = 0;
            for (int r = 0; r < n_rows; ++r) {
                int ns, it;
                row_items(h_row_ptr[r + 1] - h_row_ptr[r], 1, c, &ns, &it);
                n += it;
            }
            return n;
        };
        const int64_t slots = (int64_t)kDecodeWgPerCU * kPlanCUs;
        int lo_c = std::max(min_chunk, (e_max + kMaxSplits - 1) / kMaxSplits);
        int hi_c = std::max(lo_c, std::min(kDecodeMaxChunk, e_max));
        if (n_items(hi_c) <= slots) {
            while (lo_c < hi_c) {
                const int mid = lo_c + (hi_c - lo_c) / 2;
                if (n_items(mid) <= slots) hi_c = mid;
                else lo_c = mid + 1;
            }
            p.chunk_pages = lo_c;
        } else {
            const int64_t c = (work + kTargetDecodeItems - 1) / kTargetDecodeItems;
            p.chunk_pages = (int)std::min<int64_t>(kDecodeMaxChunk, std::max<int64_t>(min_chunk, c));
        }
    }
    int64_t items = 0, parts = 0;
    for (int r = 0; r < n_rows; ++r) {
        int nq = 1;
        if (kind == SP_WS_PREFILL) {
            const int q = r % n_seq;
            const int nt = h_tok_ptr[q + 1] - h_tok_ptr[q];
            nq = (nt + p.tok_per_tile - 1) / p.tok_per_tile;
        }
        int ns, it;
        const int64_t e_row = h_row_ptr[r + 1] - h_row_ptr[r];
        if (kind == SP_WS_DECODE && e_row > (int64_t)kMaxSplits * p.chunk_pages)
            return fail(SP_EUNSUPPORTED, "row %d: %lld table entries exceed one decode call's split capacity", r,
                        (long long)e_row);
        row_items((int)e_row, nq, p.chunk_pages, &ns, &it);
        items += it;
        if (ns > 1) {
            parts += it;
            const int per = (p.rows_per_tile + ns - 1) / ns;
            if (kind == SP_WS_PREFILL && ns >= kDeepMergeSplits) p.merge_rows_deep = std::max(p.merge_rows_deep, per);
            else p.merge_rows = std::max(p.merge_rows, per);
        }
    }
    if (items > INT32_MAX) return fail(SP_EINVAL, "too many work items");
    p.n_items = items;
    p.n_parts = parts;
    p.off_part_o = off;
    // partial outputs: fp16 for prefill (normalised), fp32 for decode
    const size_t po_bytes = kind == SP_WS_PREFILL ? 2 : sizeof(float);
    off += align_up(po_bytes * (size_t)parts * p.rows_per_tile * head_dim, 256);
    p.off_part_lse = off;
    off += align_up(sizeof(float) * (size_t)parts * p.rows_per_tile, 256);
    p.bytes = std::max<size_t>(off, 256);
    *plan = p;
    return SP_OK;
}

}  // namespace sp

using sp::fail;

extern "C" const char *segpaged_strerror(int status) {
    switch (status) {
        case SP_OK: return "ok";
        case SP_EINVAL: return "invalid argument";
        case SP_ENOMEM: return "free list too short";
        case SP_EHIP: return "HIP runtime error";
        case SP_EUNSUPPORTED: return "unsupported configuration";
        case SP_EWORKSPACE: return "workspace too small";
        default: return "unknown status";
    }
}

extern "C" const char *segpaged_last_error(void) { return sp::g_err; }

extern "C" int segpaged_version(void) { return 100; }

static int check_importance_plan(int dtype, int head_dim, int page_size, int group, int n_seq, int n_slot,
                                 const int32_t *h_tok_ptr, const int32_t *h_row_ptr, sp::ImportancePlan *ip) {
    if (dtype != SP_F32 && dtype != SP_BF16) return fail(SP_EINVAL, "dtype %d", dtype);
    if (n_seq < 1 || n_slot < 1) return fail(SP_EINVAL, "n_seq=%d n_slot=%d must be >= 1", n_seq, n_slot);
    if (group < 1 || group > 16) return fail(SP_EUNSUPPORTED, "group %d outside 1..16", group);
    if (dtype == SP_BF16) {
        if (head_dim != 64 && head_dim != 128) return fail(SP_EUNSUPPORTED, "bf16 head_dim %d (64 or 128)", head_dim);
        if (page_size != 16 && page_size != 32) return fail(SP_EUNSUPPORTED, "bf16 page_size %d (16 or 32)", page_size);
    } else if (head_dim < 16 || head_dim > 256 || head_dim % 16 || page_size < 1) {
        return fail(SP_EUNSUPPORTED, "fp32 head_dim %d page_size %d", head_dim, page_size);
    }
    if (!h_row_ptr || !h_tok_ptr) return fail(SP_EINVAL, "h_row_ptr/h_tok_ptr is NULL");
    if ((int64_t)n_slot * n_seq > INT32_MAX - 1) return fail(SP_EINVAL, "too many rows");
    const int n_rows = n_slot * n_seq;
    if (h_row_ptr[0] != 0 || h_tok_ptr[0] != 0) return fail(SP_EINVAL, "row_ptr[0] and tok_ptr[0] must be 0");
    for (int r = 0; r < n_rows; ++r)
        if (h_row_ptr[r + 1] <= h_row_ptr[r]) return fail(SP_EINVAL, "row %d has an empty or negative table", r);
    for (int q = 0; q < n_seq; ++q)
        if (h_tok_ptr[q + 1] < h_tok_ptr[q]) return fail(SP_EINVAL, "tok_ptr not ascending at %d", q);
    return sp::plan_importance(dtype, head_dim, page_size, group, n_seq, n_slot, h_tok_ptr, h_row_ptr, ip);
}

extern "C" int segpaged_workspace_bytes(int kind, int dtype, int head_dim, int page_size, int group, int n_seq,
                                        int n_slot, const int32_t *h_tok_ptr, const int32_t *h_row_ptr,
                                        size_t *bytes) {
    sp::clear_error();
    if (!bytes) return fail(SP_EINVAL, "bytes is NULL");
    if (kind == SP_WS_IMPORTANCE) {
        sp::ImportancePlan ip;
        const int rc = check_importance_plan(dtype, head_dim, page_size, group, n_seq, n_slot, h_tok_ptr, h_row_ptr,
                                             &ip);
        if (rc) return rc;
        *bytes = ip.bytes;
        return SP_OK;
    }
    sp::Plan p;
    const int rc = sp::make_plan(kind, dtype, head_dim, page_size, group, n_seq, n_slot, h_tok_ptr, h_row_ptr, &p);
    if (rc) return rc;
    *bytes = p.bytes;
    return SP_OK;
}

extern "C" int rope_relocate(const void *k_in, void *k_out, int dtype, int page_size, int head_dim, int64_t n_phys,
                             int n, const sp_reloc *d_list, double rope_theta, void *stream) {
    sp::clear_error();
    if (dtype != SP_F32 && dtype != SP_BF16) return fail(SP_EINVAL, "dtype %d", dtype);
    if (head_dim < 16 || head_dim > 256 || head_dim % 16)
        return fail(SP_EUNSUPPORTED, "head_dim %d (16..256, multiple of 16)", head_dim);
    if (page_size < 1 || page_size > 1024) return fail(SP_EUNSUPPORTED, "page_size %d (1..1024)", page_size);
    if (n < 0 || n_phys < 0) return fail(SP_EINVAL, "n=%d n_phys=%lld", n, (long long)n_phys);
    if (!(rope_theta > 0.0)) return fail(SP_EINVAL, "rope_theta must be > 0");
    if (n == 0) return SP_OK;
    if (!k_in || !k_out || !d_list) return fail(SP_EINVAL, "a pointer is NULL");
    const size_t esz = dtype == SP_F32 ? 4 : 2;
    const size_t pool = (size_t)n_phys * page_size * head_dim * esz;
    const char *a = (const char *)k_in, *b = (const char *)k_out;
    if (a != b && a < b + pool && b < a + pool) return fail(SP_EINVAL, "k_in and k_out partially overlap");
    return sp::launch_relocate(k_in, k_out, dtype, page_size, head_dim, n_phys, n, d_list, rope_theta,
                               (hipStream_t)stream);
}

static int check_attn(int dtype, int head_dim, int page_size, int group, int n_seq, int n_slot, const void *q,
                      const void *k, const void *v, int64_t n_phys, float scale, const void *out, const int32_t *cls,
                      const int32_t *win, const int32_t *row_ptr, const sp_entry *ent, const int32_t *pos,
                      const void *ws, bool decode) {
    if (dtype != SP_F32 && dtype != SP_BF16) return fail(SP_EINVAL, "dtype %d", dtype);
    if (dtype == SP_BF16) {
        if (head_dim != 64 && head_dim != 128) return fail(SP_EUNSUPPORTED, "bf16 head_dim %d (64 or 128)", head_dim);
        const bool ok = decode ? (page_size == 16 || page_size == 32)
                               : (page_size == 16 || page_size == 32 || page_size == 64);
        if (!ok) return fail(SP_EUNSUPPORTED, "bf16 page_size %d", page_size);
    }
    if (group < 1 || group > 16) return fail(SP_EUNSUPPORTED, "group %d outside 1..16", group);
    if (!(scale > 0.0f) || scale != scale) return fail(SP_EINVAL, "softmax_scale must be > 0");
    if (n_phys < 1) return fail(SP_EINVAL, "n_phys %lld", (long long)n_phys);
    if (!q || !k || !v || !out || !cls || !win || !row_ptr || !ent || !pos || !ws)
        return fail(SP_EINVAL, "a pointer is NULL");
    (void)n_seq; (void)n_slot;
    return SP_OK;
}

extern "C" int segpaged_prefill(int dtype, int head_dim, int page_size, int group, int n_seq, int n_slot,
                                const int32_t *h_tok_ptr, const int32_t *h_row_ptr, const int32_t *d_tok_ptr,
                                const int32_t *d_q_pos0, const int32_t *d_cls, const int32_t *d_window,
                                const int32_t *d_row_ptr, const sp_entry *d_entries, const void *q,
                                const void *k_pool, const void *v_pool, int64_t n_phys, float softmax_scale,
                                void *out, float *lse, void *workspace, size_t workspace_bytes, void *stream) {
    sp::clear_error();
    sp::Plan p;
    int rc = sp::make_plan(SP_WS_PREFILL, dtype, head_dim, page_size, group, n_seq, n_slot, h_tok_ptr, h_row_ptr, &p);
    if (rc) return rc;
    rc = check_attn(dtype, head_dim, page_size, group, n_seq, n_slot, q, k_pool, v_pool, n_phys, softmax_scale, out,
                    d_cls, d_window, d_row_ptr, d_entries, d_q_pos0, workspace, false);
    if (rc) return rc;
    if (!d_tok_ptr) return fail(SP_EINVAL, "d_tok_ptr is NULL");
    if (workspace_bytes < p.bytes)
        return fail(SP_EWORKSPACE, "workspace %zu bytes, %zu needed", workspace_bytes, p.bytes);
    if (((uintptr_t)workspace) % 256) return fail(SP_EINVAL, "workspace must be 256-byte aligned");
    const int64_t n_tok = h_tok_ptr[n_seq];
    if (n_tok == 0) return SP_OK;
    sp::AttnArgs a{dtype, head_dim, page_size, group, n_seq, n_slot, h_row_ptr, h_tok_ptr, d_tok_ptr, d_q_pos0, d_cls, d_window,
                   d_row_ptr, d_entries, q, k_pool, v_pool, n_phys, softmax_scale, out, lse, workspace};
    return sp::launch_prefill(a, p, n_tok, (hipStream_t)stream);
}

extern "C" int segpaged_decode(int dtype, int head_dim, int page_size, int group, int n_seq, int n_slot,
                               const int32_t *h_row_ptr, const int32_t *d_q_pos, const int32_t *d_cls,
                               const int32_t *d_window, const int32_t *d_row_ptr, const sp_entry *d_entries,
                               const void *q, const void *k_pool, const void *v_pool, int64_t n_phys,
                               float softmax_scale, void *out, float *lse, void *workspace, size_t workspace_bytes,
                               void *stream) {
    sp::clear_error();
    sp::Plan p;
    int rc = sp::make_plan(SP_WS_DECODE, dtype, head_dim, page_size, group, n_seq, n_slot, nullptr, h_row_ptr, &p);
    if (rc) return rc;
    rc = check_attn(dtype, head_dim, page_size, group, n_seq, n_slot, q, k_pool, v_pool, n_phys, softmax_scale, out,
                    d_cls, d_window, d_row_ptr, d_entries, d_q_pos, workspace, true);
    if (rc) return rc;
    if (workspace_bytes < p.bytes)
        return fail(SP_EWORKSPACE, "workspace %zu bytes, %zu needed", workspace_bytes, p.bytes);
    if (((uintptr_t)workspace) % 256) return fail(SP_EINVAL, "workspace must be 256-byte aligned");
    sp::AttnArgs a{dtype, head_dim, page_size, group, n_seq, n_slot, h_row_ptr, nullptr, nullptr, d_q_pos, d_cls, d_window,
                   d_row_ptr, d_entries, q, k_pool, v_pool, n_phys, softmax_scale, out, lse, workspace};
    return sp::launch_decode(a, p, (hipStream_t)stream);
}

static int page_copy(bool unpack, int dtype, int head_dim, int page_size, int64_t n_entries, const sp_entry *d_entries,
                     const void *src_k, const void *src_v, void *dst_k, void *dst_v, int64_t n_phys, void *stream) {
    sp::clear_error();
    if (dtype != SP_F32 && dtype != SP_BF16) return fail(SP_EINVAL, "dtype %d", dtype);
    if (head_dim < 16 || head_dim > 256 || head_dim % 16)
        return fail(SP_EUNSUPPORTED, "head_dim %d (16..256, multiple of 16)", head_dim);
    if (page_size < 1 || page_size > 1024) return fail(SP_EUNSUPPORTED, "page_size %d (1..1024)", page_size);
    if (n_entries < 0 || n_phys < 0) return fail(SP_EINVAL, "n_entries=%lld n_phys=%lld", (long long)n_entries,
                                                  (long long)n_phys);
    if (n_entries == 0) return SP_OK;
    if (!d_entries || !src_k || !src_v || !dst_k || !dst_v) return fail(SP_EINVAL, "a pointer is NULL");
    const int64_t page_bytes = (int64_t)page_size * head_dim * (dtype == SP_F32 ? 4 : 2);
    if (page_bytes > INT32_MAX) return fail(SP_EINVAL, "page too large");
    return sp::launch_page_copy(unpack, d_entries, n_entries, src_k, src_v, dst_k, dst_v, n_phys, (int)page_bytes,
                                (hipStream_t)stream);
}

extern "C" int segpaged_pack_pages(int dtype, int head_dim, int page_size, int64_t n_entries,
                                   const sp_entry *d_entries, const void *k_pool, const void *v_pool, int64_t n_phys,
                                   void *k_out, void *v_out, void *stream) {
    return page_copy(false, dtype, head_dim, page_size, n_entries, d_entries, k_pool, v_pool, k_out, v_out, n_phys,
                     stream);
}

extern "C" int segpaged_unpack_pages(int dtype, int head_dim, int page_size, int64_t n_entries,
                                     const sp_entry *d_entries, const void *k_in, const void *v_in, void *k_pool,
                                     void *v_pool, int64_t n_phys, void *stream) {
    return page_copy(true, dtype, head_dim, page_size, n_entries, d_entries, k_in, v_in, k_pool, v_pool, n_phys,
                     stream);
}

extern "C" int segpaged_token_importance(int dtype, int head_dim, int page_size, int group, int n_seq, int n_slot,
                                         const int32_t *h_tok_ptr, const int32_t *h_row_ptr,
                                         const int32_t *d_tok_ptr, const int32_t *d_q_pos0, const int32_t *d_cls,
                                         const int32_t *d_window, const int32_t *d_row_ptr,
                                         const sp_entry *d_entries, const void *q, const void *k_pool,
                                         int64_t n_phys, float softmax_scale, const float *lse,
                                         const int32_t *h_pos_ptr, const int32_t *d_pos_ptr, float *imp,
                                         void *workspace, size_t workspace_bytes, void *stream) {
    sp::clear_error();
    sp::ImportancePlan ip;
    int rc = check_importance_plan(dtype, head_dim, page_size, group, n_seq, n_slot, h_tok_ptr, h_row_ptr, &ip);
    if (rc) return rc;
    if (!(softmax_scale > 0.0f) || softmax_scale != softmax_scale) return fail(SP_EINVAL, "softmax_scale must be > 0");
    if (n_phys < 1) return fail(SP_EINVAL, "n_phys %lld", (long long)n_phys);
    if (!d_tok_ptr || !d_q_pos0 || !d_cls || !d_window || !d_row_ptr || !d_entries || !q || !k_pool || !lse ||
        !h_pos_ptr || !d_pos_ptr || !imp || !workspace)
        return fail(SP_EINVAL, "a pointer is NULL");
    if (h_pos_ptr[0] != 0) return fail(SP_EINVAL, "pos_ptr[0] must be 0");
    for (int q2 = 0; q2 < n_seq; ++q2)
        if (h_pos_ptr[q2 + 1] < h_pos_ptr[q2]) return fail(SP_EINVAL, "pos_ptr not ascending at %d", q2);
    if (workspace_bytes < ip.bytes)
        return fail(SP_EWORKSPACE, "workspace %zu bytes, %zu needed", workspace_bytes, ip.bytes);
    if (((uintptr_t)workspace) % 256) return fail(SP_EINVAL, "workspace must be 256-byte aligned");
    sp::ImportanceArgs a{dtype, head_dim, page_size, group, n_seq, n_slot, h_row_ptr, h_tok_ptr, d_tok_ptr, d_q_pos0,
                         d_cls, d_window, d_row_ptr, d_pos_ptr, d_entries, q, k_pool, n_phys, softmax_scale, lse,
                         (int64_t)h_pos_ptr[n_seq], imp, workspace};
    return sp::launch_importance(a, ip, (hipStream_t)stream);
}

extern "C" int segpaged_select_tokens(int n_layers, int slots_per_layer, int n_seq, const int32_t *h_pos_ptr,
                                      const int32_t *d_pos_ptr, const float *imp, const int32_t *h_sel_ptr,
                                      const int32_t *d_sel_ptr, float *score, int32_t *sel, void *stream) {
    sp::clear_error();
    if (n_layers < 1 || slots_per_layer < 1 || n_seq < 1)
        return fail(SP_EINVAL, "n_layers=%d slots_per_layer=%d n_seq=%d must be >= 1", n_layers, slots_per_layer,
                    n_seq);
    if ((int64_t)n_layers * slots_per_layer > INT32_MAX) return fail(SP_EINVAL, "too many slots");
    if (!h_pos_ptr || !d_pos_ptr || !imp || !h_sel_ptr || !d_sel_ptr || !score || !sel)
        return fail(SP_EINVAL, "a pointer is NULL");
    if (h_pos_ptr[0] != 0 || h_sel_ptr[0] != 0) return fail(SP_EINVAL, "pos_ptr[0] and sel_ptr[0] must be 0");
    int max_len = 0;
    for (int q = 0; q < n_seq; ++q) {
        const int len = h_pos_ptr[q + 1] - h_pos_ptr[q], k = h_sel_ptr[q + 1] - h_sel_ptr[q];
        if (len < 0) return fail(SP_EINVAL, "pos_ptr not ascending at %d", q);
        if (k < 0 || k > len) return fail(SP_EINVAL, "seq %d: k = %d outside [0, %d candidates]", q, k, len);
        max_len = std::max(max_len, len);
    }
    if (n_seq > 65535 || n_layers > 65535) return fail(SP_EUNSUPPORTED, "at most 65535 sequences and layers");
    sp::SelectArgs a{n_layers, slots_per_layer, n_seq, max_len, d_pos_ptr, d_sel_ptr, (int64_t)h_pos_ptr[n_seq],
                     (int64_t)h_sel_ptr[n_seq], imp, score, sel};
    return sp::launch_select(a, (hipStream_t)stream);
}
