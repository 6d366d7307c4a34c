// segpaged_token_importance: the attention importance every context token
// receives from a chunk's query rows, and segpaged_select_tokens: the tokens
// of highest importance per (layer, sequence), for the sparse FFN.
//
// Follows the RedKnot product profile, section 3, third building block (the
// elastic sparse FFN chooses tokens for the feed-forward network by attention
// importance and lets low-contribution tokens skip it) and the is96.com
// commentary's paragraph on the layered sparse FFN.  The importance of key t
// in a slot is the softmax probability mass the chunk's rows give it,
//   imp(t) = sum_rows exp(scale q.k_t - lse_row)   over the rows that see t,
// with lse the log-sum-exp the prefill returned for the same rows.
//
// The bf16 kernel is the score half of the prefill, turned around: a wave
// keeps one 32-key tile of K in registers (B operand of
// v_mfma_f32_32x32x16_bf16, S = Q K^T) and streams the q-tile's query rows
// from LDS (A operand), 32 rows at a time.  The accumulator enters each
// product holding -lse / scale, so a score leaves the matrix core as
// q.k - lse / scale; one multiply by scale * log2(e), one exp2 and one add per
// (row, key) then fold the probability into the lane's key column, and the
// two lane halves that hold one key combine at the end.  The queries are used
// as given, as in the prefill, so the probabilities of a row sum to one
// against the prefill's lse to fp32 rounding.  Items are
// (row, q-tile, chunk of 1024 keys); a row with several q-tiles writes one
// partial column per q-tile and a second kernel sums them in q-tile order, so
// every result is computed in one fixed order (bit-reproducible).
#include <algorithm>

#include "device_common.hpp"

namespace sp {
namespace {

constexpr int IW = 8;                     // waves per workgroup
constexpr int IQ = 256;                   // query rows (token x head) per q-tile
constexpr int IK = 32;                    // keys per wave tile
constexpr int kImpChunkKeys = 1024;       // keys per work item
constexpr int kImpInlineRows = 128;

struct ImpParams {
    const bf16 *q, *kp;
    const float *lse;
    float *imp, *part;
    const int32_t *tok_ptr, *q_pos0, *cls, *window, *row_ptr, *pos_ptr;
    const int4 *entries;
    const int32_t *item_ptr;    // workspace plan (rows beyond the inline capacity)
    const int64_t *part_ptr;
    const int64_t *red_ptr;
    int n_seq, n_rows, G, Hq, tpt;
    int64_t n_phys, n_pos;
    float scale_log2;
};

struct ImpInlinePlan {
    int32_t item_ptr[kImpInlineRows + 1];
    int64_t part_ptr[kImpInlineRows + 1];
    int64_t red_ptr[kImpInlineRows + 1];
};

// Work items of one row: q-tiles x chunks of its table (every q-tile walks the
// whole table in chunks; a chunk outside a q-tile's visible range has nothing
// to compute).  Same formula on host and device.
__host__ __device__ inline int imp_chunks(int n_entries, int ps) {
    const int per = kImpChunkKeys / ps;
    return (n_entries + per - 1) / per;
}

template <int D>
__device__ __forceinline__ int sq_chunk(int row, int c) {   // 16-byte chunk c of Q row `row` in LDS
    return row * (D / 8) + (c ^ (row & 7));
}

template <int D, int PS, bool INL>
__global__ __launch_bounds__(IW * 64) void importance_bf16_kernel(ImpParams P, ImpInlinePlan L) {
    constexpr int DK = D / 16;           // k-steps
    constexpr int PPT = IK / PS;         // pages per key tile
    __shared__ u32x4 sQ[IQ * D / 8];
    __shared__ __align__(16) float sL[IQ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t *item_ptr = INL ? L.item_ptr : P.item_ptr;
    const int b = blockIdx.x;
    const int r = find_row(item_ptr, P.n_rows, b);
    const int local = b - item_ptr[r];
    const int e_beg = P.row_ptr[r], e_end = P.row_ptr[r + 1];
    const int n_ent = e_end - e_beg;
    const int nch = imp_chunks(n_ent, PS);
    const int j = local / nch, ch = local % nch;
    const int seq = r % P.n_seq, slot = r / P.n_seq, G = P.G;
    const int tok_base = P.tok_ptr[seq];
    const int ntok_seq = P.tok_ptr[seq + 1] - tok_base;
    const int nq = (ntok_seq + P.tpt - 1) / P.tpt;
    const int t0 = j * P.tpt;
    const int ntok = min(P.tpt, ntok_seq - t0);
    const int nrows = ntok * G;
    const int p0 = P.q_pos0[seq] + t0, p_last = p0 + ntok - 1;
    const bool is_local = P.cls[slot] == SP_LOCAL;
    const int W = is_local ? P.window[slot] : 0;
    const int len = P.pos_ptr[seq + 1] - P.pos_ptr[seq];
    float *imp_row = P.imp + (int64_t)slot * P.n_pos + P.pos_ptr[seq];
    const bool partial = nq > 1;
    float *part = partial ? P.part + (INL ? L.part_ptr[r] : P.part_ptr[r]) + (int64_t)j * n_ent * PS : nullptr;

    // this item's share of the table, and what of it the q-tile sees
    const int per = kImpChunkKeys / PS;
    const int c_lo = e_beg + ch * per, c_hi = min(e_end, c_lo + per);
    int lo, hi;
    visible_range(P.entries, e_beg, e_end, p_last, is_local, p0 - W, &lo, &hi);
    const int my_lo = max(lo, c_lo), my_hi = min(hi, c_hi);
    if (partial) {   // entries of the chunk the q-tile does not see: zero partials
        for (int idx = tid; idx < (c_hi - c_lo) * PS; idx += IW * 64) {
            const int e = c_lo + idx / PS;
            if (e < my_lo || e >= my_hi) part[(int64_t)(e - e_beg) * PS + idx % PS] = 0.f;
        }
    }
    if (my_hi <= my_lo) return;

    // ---- the q-tile's rows (token, head) as given (the prefill does not round
    // them either), and their -lse / scale: a score then enters the MFMA
    // accumulator as q.k - lse / scale, and c = scale * log2(e) times it is the
    // log2 of the probability
    const float cl = P.scale_log2;
    {
        constexpr int CPR = D / 8;   // 16-byte chunks per row
        for (int idx = tid; idx < IQ * CPR; idx += IW * 64) {
            const int row = idx / CPR, c = idx % CPR;
            u32x4 w = u32x4{0, 0, 0, 0};
            if (row < nrows) {
                const int tq = row / G, g = row % G;
                w = *(const u32x4 *)(P.q + ((int64_t)(tok_base + t0 + tq) * P.Hq + (int64_t)slot * G + g) * D + 8 * c);
            }
            sQ[sq_chunk<D>(row, c)] = w;
        }
        for (int row = tid; row < IQ; row += IW * 64) {
            float nl = -INFINITY;   // rows past the q-tile: every probability 0
            if (row < nrows) {
                const int tq = row / G, g = row % G;
                nl = -P.lse[(int64_t)(tok_base + t0 + tq) * P.Hq + (int64_t)slot * G + g] * kLog2e / cl;
            }
            sL[row] = nl;
        }
    }
    __syncthreads();

    const int kc = lane & 31, half = lane >> 5;
    const int nqb = (nrows + 31) / 32;
    const int n_tiles = (my_hi - my_lo + PPT - 1) / PPT;
    for (int t = wave; t < n_tiles; t += IW) {
        // this lane's key: column kc of the tile = slot kc % PS of page kc / PS
        const int e = my_lo + t * PPT + kc / PS, ks = kc % PS;
        int4 en = int4{0, 0, 0, 0};
        const bool e_ok = e < my_hi;
        if (e_ok) en = P.entries[e];
        const bool in_pool = (uint32_t)en.x < (uint32_t)min(P.n_phys, (int64_t)INT32_MAX);
        const bool valid = e_ok && in_pool && ks < en.z;
        const int pos = en.y + ks;
        const bf16 *src = P.kp + ((int64_t)(in_pool ? en.x : 0) * PS + ks) * D + 8 * half;
        u32x4 kb[DK];
#pragma unroll
        for (int s = 0; s < DK; ++s) kb[s] = *(const u32x4 *)(src + 16 * s);
        // every key of the tile exists and every row sees it: no bounds
        const bool seen_by_all = valid && pos <= p0 && (!is_local || pos > p_last - W);
        const bool full = __ballot(seen_by_all) == ~0ull;
        float col = 0.f;
        for (int qb = 0; qb < nqb; ++qb) {
            f32x16 acc;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 l4 = *(const f32x4 *)&sL[qb * 32 + 8 * g4 + 4 * half];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[4 * g4 + i] = l4[i];
            }
            const int arow = qb * 32 + kc;
#pragma unroll
            for (int s = 0; s < DK; ++s) {
                const bf16x8 a = u4_as_bf16x8(sQ[sq_chunk<D>(arow, 2 * s + half)]);
                acc = mfma32x32x16(a, u4_as_bf16x8(kb[s]), acc);
            }
            float sum = 0.f;
            if (full) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sum += __builtin_amdgcn_exp2f(acc[i] * cl);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = qb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                    const int pq = p0 + row / G;
                    const bool vis = valid && pos <= pq && (!is_local || pos > pq - W);
                    sum += vis ? __builtin_amdgcn_exp2f(acc[i] * cl) : 0.f;
                }
            }
            col += sum;
        }
        col += __shfl_xor(col, 32, 64);
        if (half == 0 && e_ok) {
            if (partial) part[(int64_t)(e - e_beg) * PS + ks] = valid ? col : 0.f;
            else if (valid && pos < len) imp_row[pos] = col;
        }
    }
}

// Sums the q-tile partials of every row with several q-tiles, in q-tile order.
template <int PS, bool INL>
__global__ __launch_bounds__(256) void importance_reduce_kernel(ImpParams P, ImpInlinePlan L, int64_t n_total) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t *red_ptr = INL ? L.red_ptr : P.red_ptr;
    // row of this block's first element (blocks may straddle rows: each thread finds its own)
    if (i >= n_total) return;
    int lo = 0, hi = P.n_rows;                       // largest r with red_ptr[r] <= i
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (red_ptr[mid] <= i) lo = mid;
        else hi = mid;
    }
    const int r = lo;
    const int64_t el = i - red_ptr[r];
    const int seq = r % P.n_seq, slot = r / P.n_seq;
    const int e_beg = P.row_ptr[r], n_ent = P.row_ptr[r + 1] - e_beg;
    const int ntok_seq = P.tok_ptr[seq + 1] - P.tok_ptr[seq];
    const int nq = (ntok_seq + P.tpt - 1) / P.tpt;
    const float *part = P.part + (INL ? L.part_ptr[r] : P.part_ptr[r]) + el;
    float s = 0.f;
    for (int j = 0; j < nq; ++j) s += part[(int64_t)j * n_ent * PS];
    const int4 en = P.entries[e_beg + el / PS];
    const int ks = (int)(el % PS);
    const int len = P.pos_ptr[seq + 1] - P.pos_ptr[seq];
    const int pos = en.y + ks;
    if ((uint32_t)en.x < (uint32_t)min(P.n_phys, (int64_t)INT32_MAX) && ks < en.z && pos < len)
        P.imp[(int64_t)slot * P.n_pos + P.pos_ptr[seq] + pos] = s;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *x, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = 0.f;
}

// Plan of a call with more rows than the inline plan holds: per-row prefix
// sums of items, partial floats and reduce elements, by one workgroup.
__global__ __launch_bounds__(1024) void importance_plan_kernel(const int32_t *__restrict__ row_ptr,
                                                               const int32_t *__restrict__ tok_ptr, int n_seq,
                                                               int n_rows, int tpt, int ps, int32_t *item_ptr,
                                                               int64_t *part_ptr, int64_t *red_ptr) {
    __shared__ int64_t s_it[1024], s_pt[1024], s_rd[1024];
    __shared__ int64_t carry[3];
    const int tid = threadIdx.x;
    if (tid == 0) carry[0] = carry[1] = carry[2] = 0;
    __syncthreads();
    for (int base = 0; base < n_rows; base += 1024) {
        const int r = base + tid;
        int64_t it = 0, pt = 0, rd = 0;
        if (r < n_rows) {
            const int q = r % n_seq;
            const int ntok = tok_ptr[q + 1] - tok_ptr[q];
            const int nq = (ntok + tpt - 1) / tpt;
            const int ne = row_ptr[r + 1] - row_ptr[r];
            it = (int64_t)nq * imp_chunks(ne, ps);
            if (nq > 1) {
                pt = (int64_t)nq * ne * ps;
                rd = (int64_t)ne * ps;
            }
        }
        s_it[tid] = it;
        s_pt[tid] = pt;
        s_rd[tid] = rd;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {   // inclusive scans
            const int64_t a = tid >= off ? s_it[tid - off] : 0, c = tid >= off ? s_pt[tid - off] : 0,
                          d = tid >= off ? s_rd[tid - off] : 0;
            __syncthreads();
            s_it[tid] += a;
            s_pt[tid] += c;
            s_rd[tid] += d;
            __syncthreads();
        }
        if (r < n_rows) {
            item_ptr[r] = (int32_t)(carry[0] + s_it[tid] - it);
            part_ptr[r] = carry[1] + s_pt[tid] - pt;
            red_ptr[r] = carry[2] + s_rd[tid] - rd;
        }
        __syncthreads();
        if (tid == 1023) {
            carry[0] += s_it[1023];
            carry[1] += s_pt[1023];
            carry[2] += s_rd[1023];
        }
        __syncthreads();
    }
    if (tid == 0) {
        item_ptr[n_rows] = (int32_t)carry[0];
        part_ptr[n_rows] = carry[1];
        red_ptr[n_rows] = carry[2];
    }
}

// ---------------------------------------------------------------- fp32 (the tiny config)
// One thread per key: the sum over every query row of the row, in row order.
struct ImpF32Params {
    const float *q, *kp, *lse;
    float *imp;
    const int32_t *tok_ptr, *q_pos0, *cls, *window, *row_ptr, *pos_ptr;
    const int4 *entries;
    int n_seq, G, Hq, D, ps;
    int64_t n_phys, n_pos;
    float scale;
};

__global__ __launch_bounds__(256) void importance_f32_kernel(ImpF32Params P) {
    const int r = blockIdx.y;
    const int seq = r % P.n_seq, slot = r / P.n_seq;
    const int e_beg = P.row_ptr[r], e_end = P.row_ptr[r + 1];
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= (int64_t)(e_end - e_beg) * P.ps) return;
    const int4 en = P.entries[e_beg + k / P.ps];
    const int ks = (int)(k % P.ps);
    if ((uint32_t)en.x >= (uint32_t)min(P.n_phys, (int64_t)INT32_MAX) || ks >= en.z) return;
    const int pos = en.y + ks;
    const int len = P.pos_ptr[seq + 1] - P.pos_ptr[seq];
    if (pos >= len) return;
    const bool is_local = P.cls[slot] == SP_LOCAL;
    const int W = is_local ? P.window[slot] : 0;
    const float *kv = P.kp + ((int64_t)en.x * P.ps + ks) * P.D;
    const int tb = P.tok_ptr[seq], nt = P.tok_ptr[seq + 1] - tb;
    float s = 0.f;
    for (int t = 0; t < nt; ++t) {
        const int pq = P.q_pos0[seq] + t;
        if (pos > pq || (is_local && pos <= pq - W)) continue;
        for (int g = 0; g < P.G; ++g) {
            const int64_t h = (int64_t)(tb + t) * P.Hq + (int64_t)slot * P.G + g;
            const float *qv = P.q + h * P.D;
            float d = 0.f;
            for (int i = 0; i < P.D; ++i) d = fmaf(qv[i], kv[i], d);
            s += expf(d * P.scale - P.lse[h]);
        }
    }
    P.imp[(int64_t)slot * P.n_pos + P.pos_ptr[seq] + pos] = s;
}

// ---------------------------------------------------------------- token selection
// The layer scores (each position's slot importances added in fp32 in slot
// order) come from a grid-wide kernel; then one workgroup per (sequence,
// layer) finds the k-th largest score T by a radix select over the fp32 bit
// patterns (scores are >= 0, so the bit patterns order like the values), 8
// bits per pass from the top, and one ordered pass writes every position above
// T and the lowest positions equal to T, in ascending order.  A sequence's
// scores are staged in LDS when they fit (every pass then reads LDS);
// otherwise the passes read them from global memory SE positions per thread
// at a time.  Each thread owns consecutive positions, so the ordered pass
// needs one pair of block-wide scans per chunk.
constexpr int SW = 16;                 // waves of a selection workgroup
constexpr int SE = 16;                 // consecutive positions per thread and chunk
constexpr int SCHUNK = SW * 64 * SE;
constexpr int kSelLds = 32768;         // longest candidate list staged in LDS (128 KB)

struct SelParams {
    const float *imp;
    float *score;
    int32_t *sel;
    const int32_t *pos_ptr, *sel_ptr;
    int spl, n_seq, n_layers;
    int64_t n_pos, sel_total;
};

__global__ __launch_bounds__(256) void layer_score_kernel(SelParams P) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int layer = blockIdx.y;
    if (t >= P.n_pos) return;
    const float *imp = P.imp + (int64_t)layer * P.spl * P.n_pos + t;
    float v[8];
    float s = 0.f;
    int j = 0;
    for (; j + 8 <= P.spl; j += 8) {     // eight loads in flight, added in slot order
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = imp[(int64_t)(j + i) * P.n_pos];
#pragma unroll
        for (int i = 0; i < 8; ++i) s = (j + i == 0) ? v[i] : s + v[i];
    }
    for (; j < P.spl; ++j) s = j == 0 ? imp[0] : s + imp[(int64_t)j * P.n_pos];
    P.score[(int64_t)layer * P.n_pos + t] = s;
}

// Exclusive prefix over the workgroup of small non-negative counts (and the total).
__device__ __forceinline__ int block_exclusive_scan(int x, int *s_wave, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int v = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(v, off, 64);
        if (lane >= off) v += y;
    }
    if (lane == 63) s_wave[wave] = v;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < SW; ++w) {
        const int c = s_wave[w];
        before += w < wave ? c : 0;
        all += c;
    }
    __syncthreads();
    *total = all;
    return before + v - x;
}

template <bool IN_LDS>
__global__ __launch_bounds__(SW * 64) void select_kernel(SelParams P) {
    // one 256-bin histogram per wave (scores of one magnitude share a top
    // byte, so a single shared histogram would serialise every atomic on a
    // bin or two); a wave whose active lanes all fall in one bin adds them
    // with one atomic
    __shared__ int hist[SW][256];
    __shared__ int s_wave[SW];
    __shared__ int s_bin, s_above;
    __shared__ uint32_t s_score[IN_LDS ? kSelLds : 1];
    const int seq = blockIdx.x, layer = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t base = P.pos_ptr[seq];
    const int len = P.pos_ptr[seq + 1] - P.pos_ptr[seq];
    const int k = P.sel_ptr[seq + 1] - P.sel_ptr[seq];
    if (k == 0) return;
    const uint32_t *g_score = (const uint32_t *)(P.score + (int64_t)layer * P.n_pos + base);
    if (IN_LDS) {
        for (int t = tid; t < len; t += SW * 64) s_score[t] = g_score[t];
        __syncthreads();
    }
    auto load_chunk = [&](int t0, uint32_t (&u)[SE]) {
#pragma unroll
        for (int i = 0; i < SE; ++i) u[i] = t0 + i < len ? (IN_LDS ? s_score[t0 + i] : g_score[t0 + i]) : 0u;
    };
    uint32_t prefix = 0, mask = 0;
    int remaining = k;                 // how many of the selected lie at or below the current prefix
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = lane; i < 256; i += 64) hist[wave][i] = 0;
        __syncthreads();
        for (int c0 = 0; c0 < len; c0 += SCHUNK) {
            const int t0 = c0 + tid * SE;
            uint32_t u[SE];
            load_chunk(t0, u);
#pragma unroll
            for (int i = 0; i < SE; ++i) {
                const bool act = t0 + i < len && (u[i] & mask) == prefix;
                const int bin = (int)((u[i] >> shift) & 255u);
                const uint64_t am = __ballot(act);
                if (!am) continue;
                const int lb = __builtin_amdgcn_readlane(bin, (int)__builtin_ctzll(am));
                if (__ballot(act && bin != lb) == 0) {
                    if (lane == 0) atomicAdd(&hist[wave][lb], (int)__popcll(am));
                } else if (act) {
                    atomicAdd(&hist[wave][bin], 1);
                }
            }
        }
        __syncthreads();
        // counts per bin, highest bin first, summed over the waves; the bin
        // where the running count from the top reaches `remaining`
        int c = 0, v = 0;
        if (tid < 256) {                     // waves 0..3: bins 255 - tid
            const int b = 255 - tid;
#pragma unroll
            for (int w = 0; w < SW; ++w) c += hist[w][b];
            v = c;                           // inclusive scan within the wave
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(v, off, 64);
                if (lane >= off) v += y;
            }
            if (lane == 63) s_wave[wave] = v;
        }
        __syncthreads();
        if (tid < 256) {
            int before = 0;
            for (int w = 0; w < wave; ++w) before += s_wave[w];
            const int incl = before + v, excl = incl - c;
            if (excl < remaining && incl >= remaining) {   // exactly one bin
                s_bin = 255 - tid;
                s_above = excl;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)s_bin << shift;
        mask |= 255u << shift;
        remaining -= s_above;
        __syncthreads();
    }
    // T = prefix: every position above T, and the `remaining` lowest positions equal to T
    int32_t *out = P.sel + (int64_t)layer * P.sel_total + P.sel_ptr[seq];
    int eq_before = 0, out_before = 0;
    for (int c0 = 0; c0 < len; c0 += SCHUNK) {
        const int t0 = c0 + tid * SE;
        uint32_t u[SE];
        load_chunk(t0, u);
        int n_eq = 0;
#pragma unroll
        for (int i = 0; i < SE; ++i) n_eq += (t0 + i < len && u[i] == prefix) ? 1 : 0;
        int eq_total;
        int eq_rank = eq_before + block_exclusive_scan(n_eq, s_wave, &eq_total);
        int take[SE], n_take = 0;
#pragma unroll
        for (int i = 0; i < SE; ++i) {
            const bool in = t0 + i < len;
            const bool gt = in && u[i] > prefix, eq = in && u[i] == prefix;
            take[i] = gt || (eq && eq_rank < remaining);
            eq_rank += eq ? 1 : 0;
            n_take += take[i];
        }
        int take_total;
        int idx = out_before + block_exclusive_scan(n_take, s_wave, &take_total);
#pragma unroll
        for (int i = 0; i < SE; ++i)
            if (take[i]) out[idx++] = t0 + i;
        eq_before += eq_total;
        out_before += take_total;
    }
}

}  // namespace

// Host plan of one importance call: item count, partial floats, reduce elements,
// per-row prefixes for up to kImpInlineRows rows.
int plan_importance(int dtype, int head_dim, int page_size, int group, int n_seq, int n_slot,
                    const int32_t *h_tok_ptr, const int32_t *h_row_ptr, ImportancePlan *out) {
    ImportancePlan p;
    p.n_rows = n_seq * n_slot;
    if (dtype == SP_F32) {
        if (p.n_rows > 65535) return fail(SP_EUNSUPPORTED, "fp32 importance: %d rows (at most 65535)", p.n_rows);
        int64_t e_max = 0;
        for (int r = 0; r < p.n_rows; ++r) e_max = std::max<int64_t>(e_max, h_row_ptr[r + 1] - h_row_ptr[r]);
        p.e_max = e_max;
        p.bytes = 256;
        *out = p;
        return SP_OK;
    }
    p.tpt = IQ / group;
    int64_t items = 0, parts = 0, red = 0;
    for (int r = 0; r < p.n_rows; ++r) {
        const int q = r % n_seq;
        const int nt = h_tok_ptr[q + 1] - h_tok_ptr[q];
        const int nq = (nt + p.tpt - 1) / p.tpt;
        const int ne = h_row_ptr[r + 1] - h_row_ptr[r];
        items += (int64_t)nq * imp_chunks(ne, page_size);
        if (nq > 1) {
            parts += (int64_t)nq * ne * page_size;
            red += (int64_t)ne * page_size;
        }
    }
    if (items > INT32_MAX) return fail(SP_EINVAL, "too many importance work items");
    p.n_items = items;
    p.n_part = parts;
    p.n_red = red;
    size_t off = 0;
    p.off_item_ptr = off; off += sizeof(int32_t) * (p.n_rows + 1);
    off = (off + 255) / 256 * 256;
    p.off_part_ptr = off; off += sizeof(int64_t) * (p.n_rows + 1);
    p.off_red_ptr = off;  off += sizeof(int64_t) * (p.n_rows + 1);
    off = (off + 255) / 256 * 256;
    p.off_part = off;     off += sizeof(float) * (size_t)parts;
    p.bytes = std::max<size_t>(off, 256);
    (void)head_dim;
    *out = p;
    return SP_OK;
}

int launch_importance(const ImportanceArgs &a, const ImportancePlan &p, hipStream_t stream) {
    const int64_t n_imp = (int64_t)a.n_slot * a.n_pos;
    if (n_imp > 0) {
        const int64_t blocks = std::min<int64_t>((n_imp + 255) / 256, 8192);
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a.imp, n_imp);
    }
    if (a.dtype == SP_F32) {
        ImpF32Params P;
        P.q = (const float *)a.q;
        P.kp = (const float *)a.k_pool;
        P.lse = a.lse;
        P.imp = a.imp;
        P.tok_ptr = a.d_tok_ptr;
        P.q_pos0 = a.d_q_pos0;
        P.cls = a.d_cls;
        P.window = a.d_window;
        P.row_ptr = a.d_row_ptr;
        P.pos_ptr = a.d_pos_ptr;
        P.entries = (const int4 *)a.d_entries;
        P.n_seq = a.n_seq;
        P.G = a.group;
        P.Hq = a.n_slot * a.group;
        P.D = a.head_dim;
        P.ps = a.page_size;
        P.n_phys = a.n_phys;
        P.n_pos = a.n_pos;
        P.scale = a.scale;
        const int64_t gx = (p.e_max * a.page_size + 255) / 256;
        if (gx > 0)
            hipLaunchKernelGGL(importance_f32_kernel, dim3((unsigned)gx, (unsigned)p.n_rows), dim3(256), 0, stream, P);
        return check_hip(hipGetLastError(), "importance launch");
    }
    char *w = (char *)a.ws;
    ImpParams P;
    P.q = (const bf16 *)a.q;
    P.kp = (const bf16 *)a.k_pool;
    P.lse = a.lse;
    P.imp = a.imp;
    P.part = (float *)(w + p.off_part);
    P.tok_ptr = a.d_tok_ptr;
    P.q_pos0 = a.d_q_pos0;
    P.cls = a.d_cls;
    P.window = a.d_window;
    P.row_ptr = a.d_row_ptr;
    P.pos_ptr = a.d_pos_ptr;
    P.entries = (const int4 *)a.d_entries;
    P.item_ptr = (const int32_t *)(w + p.off_item_ptr);
    P.part_ptr = (const int64_t *)(w + p.off_part_ptr);
    P.red_ptr = (const int64_t *)(w + p.off_red_ptr);
    P.n_seq = a.n_seq;
    P.n_rows = p.n_rows;
    P.G = a.group;
    P.Hq = a.n_slot * a.group;
    P.tpt = p.tpt;
    P.n_phys = a.n_phys;
    P.n_pos = a.n_pos;
    P.scale_log2 = a.scale * kLog2e;
    const bool inl = p.n_rows <= kImpInlineRows;
    ImpInlinePlan L;
    if (inl) {
        int64_t it = 0, pt = 0, rd = 0;
        for (int r = 0; r < p.n_rows; ++r) {
            const int q = r % a.n_seq;
            const int nt = a.h_tok_ptr[q + 1] - a.h_tok_ptr[q];
            const int nq = (nt + p.tpt - 1) / p.tpt;
            const int ne = a.h_row_ptr[r + 1] - a.h_row_ptr[r];
            L.item_ptr[r] = (int32_t)it;
            L.part_ptr[r] = pt;
            L.red_ptr[r] = rd;
            it += (int64_t)nq * imp_chunks(ne, a.page_size);
            if (nq > 1) {
                pt += (int64_t)nq * ne * a.page_size;
                rd += (int64_t)ne * a.page_size;
            }
        }
        L.item_ptr[p.n_rows] = (int32_t)it;
        L.part_ptr[p.n_rows] = pt;
        L.red_ptr[p.n_rows] = rd;
    } else {
        L.item_ptr[0] = 0;
        hipLaunchKernelGGL(importance_plan_kernel, dim3(1), dim3(1024), 0, stream, a.d_row_ptr, a.d_tok_ptr, a.n_seq,
                           p.n_rows, p.tpt, a.page_size, (int32_t *)(w + p.off_item_ptr),
                           (int64_t *)(w + p.off_part_ptr), (int64_t *)(w + p.off_red_ptr));
    }
    if (p.n_items == 0) return check_hip(hipGetLastError(), "importance launch");
    const dim3 grid((unsigned)p.n_items), rgrid((unsigned)((p.n_red + 255) / 256));
#define SP_IMP_CASE(DD, PSV)                                                                                         \
    if (a.head_dim == DD && a.page_size == PSV) {                                                                    \
        if (inl) {                                                                                                   \
            hipLaunchKernelGGL((importance_bf16_kernel<DD, PSV, true>), grid, dim3(IW * 64), 0, stream, P, L);       \
            if (p.n_red) hipLaunchKernelGGL((importance_reduce_kernel<PSV, true>), rgrid, dim3(256), 0, stream, P, L, \
                                            p.n_red);                                                                \
        } else {                                                                                                     \
            hipLaunchKernelGGL((importance_bf16_kernel<DD, PSV, false>), grid, dim3(IW * 64), 0, stream, P, L);      \
            if (p.n_red) hipLaunchKernelGGL((importance_reduce_kernel<PSV, false>), rgrid, dim3(256), 0, stream, P,   \
                                            L, p.n_red);                                                             \
        }                                                                                                            \
    }
    SP_IMP_CASE(128, 16) else SP_IMP_CASE(128, 32) else SP_IMP_CASE(64, 16) else SP_IMP_CASE(64, 32)
    else return fail(SP_EUNSUPPORTED, "bf16 importance head_dim %d page_size %d", a.head_dim, a.page_size);
#undef SP_IMP_CASE
    return check_hip(hipGetLastError(), "importance launch");
}

int launch_select(const SelectArgs &a, hipStream_t stream) {
    SelParams P;
    P.imp = a.imp;
    P.score = a.score;
    P.sel = a.sel;
    P.pos_ptr = a.d_pos_ptr;
    P.sel_ptr = a.d_sel_ptr;
    P.spl = a.slots_per_layer;
    P.n_seq = a.n_seq;
    P.n_layers = a.n_layers;
    P.n_pos = a.n_pos;
    P.sel_total = a.sel_total;
    if (a.n_pos > 0)
        hipLaunchKernelGGL(layer_score_kernel, dim3((unsigned)((a.n_pos + 255) / 256), (unsigned)a.n_layers),
                           dim3(256), 0, stream, P);
    const dim3 grid((unsigned)a.n_seq, (unsigned)a.n_layers);
    if (a.max_len <= kSelLds) hipLaunchKernelGGL(select_kernel<true>, grid, dim3(SW * 64), 0, stream, P);
    else hipLaunchKernelGGL(select_kernel<false>, grid, dim3(SW * 64), 0, stream, P);
    return check_hip(hipGetLastError(), "select launch");
}

}  // namespace sp
