// segpaged_prefill for bf16: MFMA attention of a chunk of new tokens over each
// head's own page table, with no mask tensor.
//
// Follows the RedKnot product profile, section 3 (SegPagedAttention: every head
// reads only its own pages and each class its own visible window, on the
// mask-free attention path) and the is96.com commentary's SegPagedAttention
// paragraphs (a page table per head listing the pages it reads).  Prefill is the
// compute-bound phase (the Prefill/Decode explainer listed on the
// PagedAttention & RadixAttention page), so the two contractions run on the
// gfx950 matrix cores.
//
// Work item = (row = (slot, seq), q-tile, kv split).  A q-tile holds all
// `group` query heads of up to 32*NW/group consecutive tokens, so each staged
// K/V tile feeds every head of the slot.  Each wave owns 32 query rows.
//
// Per 64-key tile (one to four pages):
//   K  [64 keys][D]  -> LDS, token-major as stored;
//   V^T[D][64 keys]  -> LDS, copied straight from the dim-major V pages;
//   S^T = K Q^T      (v_mfma_f32_32x32x16_bf16: keys x queries), so every lane
//                    holds one query's scores and the row softmax needs a single
//                    cross-lane step;
//   O^T += V^T P^T   (same instruction: dims x queries), P^T taken directly from
//                    the S^T registers.
// The K rows fed to the first product are permuted (sigma below) so that the
// score registers of each lane are exactly the 8 consecutive keys the second
// product's B operand wants - no shuffles between the two products.
// Bounds come from positions and only boundary tiles evaluate them.
#include "device_common.hpp"

namespace sp {
namespace {

constexpr int BN = kPrefillKeysPerTile;   // 64 keys per tile

struct PrefillParams {
    const bf16 *q, *kp, *vp;
    bf16 *out;
    float *lse;
    const int32_t *tok_ptr, *q_pos0, *cls, *window, *row_ptr;
    const int4 *entries;
    const int32_t *item_ptr, *part_ptr, *nsplit;
    float *part_o, *part_lse;
    int n_seq, n_rows, G, ps, tpt, Hq;
    int64_t n_phys;
    float scale_log2;   // softmax_scale * log2(e)
};

// Table entries of the (up to four) pages of one 64-key tile, workgroup-uniform.
// Kept as four named values and selected with compares so that they stay in
// registers (an array indexed by a lane-varying page would go to scratch).
struct TileEntries {
    int4 a, b, c, d;
    __device__ __forceinline__ int4 pick(int pg) const {
        const int4 lo = pg == 0 ? a : b;
        const int4 hi = pg == 2 ? c : d;
        return pg < 2 ? lo : hi;
    }
};

// Output row m of a 32x32 MFMA tile <- K row sigma(m) of the 32-key block.
// Lane (n, h) holds rows m = (v/4)*8 + 4h + v%4; sigma maps them to keys
// 16*(v/8) + 8h + v%8, i.e. it swaps bits 2 and 3 of m.
__device__ __forceinline__ int sigma(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <int D, int NW, int PS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_bf16_kernel(
    PrefillParams P) {
    constexpr int NT = NW * 64;
    constexpr int BM = 32 * NW;
    constexpr int KS = D + 8;      // LDS row stride of K (bf16), padded against bank conflicts
    constexpr int VS = BN + 8;     // LDS row stride of V^T
    constexpr int DK = D / 16;     // k-steps of the QK^T product
    constexpr int DT = D / 32;     // 32-dim tiles of the output
    constexpr int KCH = BN * D / 8;                 // 16-byte chunks per K (or V) tile
    constexpr int CPT = (KCH + NT - 1) / NT;        // chunks per thread
    __shared__ __attribute__((aligned(16))) bf16 sK[2][BN * KS];
    __shared__ __attribute__((aligned(16))) bf16 sV[2][D * VS];
    __shared__ int sPos[2][BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, h = lane >> 5;

    // ---- work item
    const int b = blockIdx.x;
    const int r = find_row(P.item_ptr, P.n_rows, b);
    const int ns = P.nsplit[r];
    const int local = b - P.item_ptr[r];
    const int qt = local / ns, sp_i = local % ns;
    const int seq = r % P.n_seq, slot = r / P.n_seq;
    const int tok_base = P.tok_ptr[seq];
    const int t0 = qt * P.tpt;
    const int ntok = min(P.tpt, P.tok_ptr[seq + 1] - tok_base - t0);
    const int p0 = P.q_pos0[seq] + t0, p_last = p0 + ntok - 1;
    const int G = P.G;
    constexpr int ps = PS;
    const bool is_local = P.cls[slot] == SP_LOCAL;
    const int W = is_local ? P.window[slot] : 0;
    const int nrows = ntok * G;

    // ---- the q-tile's visible entry range, then this split's share
    const int e_beg = P.row_ptr[r], e_end = P.row_ptr[r + 1];
    const int4 *E = P.entries;
    int lo, hi;
    visible_range(E, e_beg, e_end, p_last, is_local, p0 - W, &lo, &hi);
    constexpr int ppt = BN / ps;                        // pages per tile
    int chunk = (hi - lo + ns - 1) / ns;
    chunk = (chunk + ppt - 1) / ppt * ppt;
    const int my_lo = min(hi, lo + sp_i * chunk);
    const int my_hi = min(hi, my_lo + chunk);
    const int n_tiles = (my_hi - my_lo + ppt - 1) / ppt;

    // ---- queries of this wave: row = 32*wave + n -> (token, head)
    const int row = 32 * wave + n;
    const bool row_ok = row < nrows;
    const int tq = row / G, g = row % G;
    const int pq = p0 + tq;                    // this lane's query position
    const int lowq = is_local ? pq - W : INT32_MIN;   // visible iff lowq < pos <= pq
    bf16x8 qf[DK];
    {
        const bf16 *qrow = P.q + ((int64_t)(tok_base + t0 + tq) * P.Hq + (int64_t)slot * G + g) * D;
#pragma unroll
        for (int s = 0; s < DK; ++s) {
            u32x4 v = {0, 0, 0, 0};
            if (row_ok) v = *(const u32x4 *)(qrow + 16 * s + 8 * h);
            qf[s] = u4_as_bf16x8(v);
        }
    }

    // ---- tile staging: the tile's (up to 4) table entries are workgroup-uniform;
    // data loads take no branch on them (empty slots read page 0 and are zeroed)
    auto fetch_entries = [&](int t, TileEntries &te) {
        const int e0 = my_lo + t * ppt;
        auto clean = [&](int4 en) {
            if (en.x < 0 || en.x >= P.n_phys) en = int4{0, 0, 0, 0};
            en.z = min(en.z, ps);
            return en;
        };
        if (e0 + ppt <= my_hi) {            // the usual case: one scalar burst
            te.a = clean(E[e0]);
            te.b = ppt > 1 ? clean(E[e0 + 1]) : int4{0, 0, 0, 0};
            te.c = ppt > 2 ? clean(E[e0 + 2]) : int4{0, 0, 0, 0};
            te.d = ppt > 3 ? clean(E[e0 + 3]) : int4{0, 0, 0, 0};
        } else {                            // the item's last, partial tile
            auto get = [&](int pg) { return e0 + pg < my_hi ? clean(E[e0 + pg]) : int4{0, 0, 0, 0}; };
            te.a = get(0);
            te.b = get(1);
            te.c = get(2);
            te.d = get(3);
        }
    };
    auto tile_full = [&](const TileEntries &te) {
        // no bounds needed if every slot holds a token visible to every query of the q-tile
        const int4 x[4] = {te.a, te.b, te.c, te.d};
        bool full = true;
        int kmin = INT32_MAX, kmax = INT32_MIN;
#pragma unroll
        for (int pg = 0; pg < 4; ++pg)
            if (pg < ppt) {
                full = full && x[pg].z == ps;
                kmin = min(kmin, x[pg].y);
                kmax = max(kmax, x[pg].y + x[pg].z - 1);
            }
        return full && kmax <= p0 && (!is_local || kmin > p_last - W);
    };
    // Per-thread chunk geometry, fixed for the whole item.  A page spans
    // D*ps/8 >= 64 chunks, so the page of each chunk is uniform across a wave:
    // its base address is computed in scalar registers once per tile and the
    // lanes only add their constant offsets.
    static_assert(D * ps / 8 % 64 == 0, "a page must cover whole waves of 16-byte chunks");
    constexpr int per_page = D * ps / 8;
    int k_pg[CPT], k_tk[CPT], k_off[CPT], k_lds[CPT], v_pg[CPT], v_k8[CPT], v_off[CPT], v_lds[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = tid + i * NT;
        const int j = c / (D / 8), col = (c % (D / 8)) * 8;
        k_pg[i] = __builtin_amdgcn_readfirstlane(c / per_page);
        k_tk[i] = j % ps;
        k_off[i] = k_tk[i] * D + col;
        k_lds[i] = j * KS + col;
        const int rem = c % per_page;
        const int d = rem / (ps / 8), k8 = (rem % (ps / 8)) * 8;
        v_pg[i] = k_pg[i];
        v_k8[i] = k8;
        v_off[i] = d * ps + k8;
        v_lds[i] = d * VS + v_pg[i] * ps + k8;
    }
    u32x4 rk[CPT], rv[CPT];
    auto load_tile = [&](const TileEntries &te) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            if (KCH % NT == 0 || tid + i * NT < KCH) {
                const int4 en = te.pick(k_pg[i]);   // wave-uniform
                const bf16 *kb = P.kp + (int64_t)en.x * (ps * D);
                const bf16 *vb = P.vp + (int64_t)en.x * (ps * D);
                const u32x4 kv = *(const u32x4 *)(kb + k_off[i]);
                const u32x4 vv = *(const u32x4 *)(vb + v_off[i]);
                rk[i] = k_tk[i] < en.z ? kv : u32x4{0, 0, 0, 0};
                const int keep = en.z - v_k8[i];
                rv[i] = keep >= 8 ? vv : (keep > 0 ? keep_first_bf16(vv, keep) : u32x4{0, 0, 0, 0});
            }
        }
    };
    auto store_tile = [&](const TileEntries &te, int buf) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            if (KCH % NT == 0 || tid + i * NT < KCH) {
                *(u32x4 *)&sK[buf][k_lds[i]] = rk[i];
                *(u32x4 *)&sV[buf][v_lds[i]] = rv[i];
            }
        }
        if (tid < BN) {
            const int pg = tid / ps, tk = tid % ps;
            const int4 en = te.pick(pg);
            sPos[buf][tid] = tk < en.z ? en.y + tk : kPosInvalid;
        }
    };

    // ---- running softmax state (log2 domain) and O^T accumulators
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{0};

    TileEntries te_cur, te_nxt;
    bool full_cur = false, full_nxt = false;
    if (n_tiles > 0) {
        fetch_entries(0, te_cur);
        full_cur = tile_full(te_cur);
        load_tile(te_cur);
        store_tile(te_cur, 0);
    }
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < n_tiles) {
            fetch_entries(t + 1, te_nxt);
            full_nxt = tile_full(te_nxt);
            load_tile(te_nxt);
        }

        // S^T = K Q^T over the two 32-key halves of the tile
        f32x16 S[BN / 32];
#pragma unroll
        for (int kt = 0; kt < BN / 32; ++kt) {
            S[kt] = f32x16{0};
            const bf16 *krow = &sK[buf][(32 * kt + sigma(n)) * KS + 8 * h];
#pragma unroll
            for (int s = 0; s < DK; ++s) {
                const bf16x8 a = *(const bf16x8 *)(krow + 16 * s);
                S[kt] = mfma32x32x16(a, qf[s], S[kt]);
            }
        }
        // bounds (boundary tiles only) and online softmax; the running max is kept
        // on raw scores (the scale is positive) and folded into one FMA per exp
        if (!full_cur) {
#pragma unroll
            for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int kpos = sPos[buf][32 * kt + 16 * (v >> 3) + 8 * h + (v & 7)];
                    S[kt][v] = (kpos <= pq && kpos > lowq) ? S[kt][v] : -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[kt][v]);
        mx = fmaxf(mx, xor_lane(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float c = P.scale_log2;
        // exponents are <= 0 here; v_exp_f32 flushes results below 2^-126 to zero, which is harmless
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c);
        const float off = -m_use * c;
        float rs = 0.f;
#pragma unroll
        for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = __builtin_amdgcn_exp2f(fmaf(S[kt][v], c, off));
                S[kt][v] = p;
                rs += p;
            }
        l_run = l_run * alpha + rs;
        m_run = m_new;
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
        }

        // O^T += V^T P^T, 16 keys per step
#pragma unroll
        for (int s2 = 0; s2 < BN / 16; ++s2) {
            const int kt = s2 >> 1, u = s2 & 1;
            u32x4 pk;
#pragma unroll
            for (int w = 0; w < 4; ++w) pk[w] = pack_bf16x2(S[kt][8 * u + 2 * w], S[kt][8 * u + 2 * w + 1]);
            const bf16x8 pb = u4_as_bf16x8(pk);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8 a = *(const bf16x8 *)&sV[buf][(32 * dt + n) * VS + 16 * s2 + 8 * h];
                acc[dt] = mfma32x32x16(a, pb, acc[dt]);
            }
        }

        if (t + 1 < n_tiles) {
            store_tile(te_nxt, buf ^ 1);
            full_cur = full_nxt;
        }
        __syncthreads();
    }

    // ---- epilogue
    const float l = l_run + xor_lane(l_run, 32);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse = l > 0.f ? (m_run * P.scale_log2 + log2f(l)) * kLn2 : -INFINITY;
    if (!row_ok) return;
    if (ns == 1) {
        bf16 *orow = P.out + ((int64_t)(tok_base + t0 + tq) * P.Hq + (int64_t)slot * G + g) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 32 * dt + 8 * q4 + 4 * h;
                u32x2 w;
                w[0] = pack_bf16x2(acc[dt][4 * q4 + 0] * inv, acc[dt][4 * q4 + 1] * inv);
                w[1] = pack_bf16x2(acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv);
                *(u32x2 *)(orow + d) = w;
            }
        if (P.lse && h == 0) P.lse[(int64_t)(tok_base + t0 + tq) * P.Hq + (int64_t)slot * G + g] = lse;
    } else {
        const int64_t part = (int64_t)P.part_ptr[r] + local;
        float *po = P.part_o + (part * BM + row) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 32 * dt + 8 * q4 + 4 * h;
                *(float4 *)(po + d) = make_float4(acc[dt][4 * q4] * inv, acc[dt][4 * q4 + 1] * inv,
                                                  acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv);
            }
        if (h == 0) P.part_lse[part * BM + row] = lse;
    }
}

// Combines the kv splits of every split q-tile: O = sum_s e^{lse_s-M} o_s / sum_s e^{lse_s-M}.
// Launched over the same work items: item (q-tile, split s) merges rows
// [s * ceil(rows/ns), (s+1) * ceil(rows/ns)) of its q-tile, so all splits share
// the work.  One wave per row: the split weights are formed once per row (in
// LDS), then each lane accumulates its dims over the splits.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillParams P, int BM) {
    __shared__ float sw[4][kMaxSplits];
    const int b = blockIdx.x;
    const int r = find_row(P.item_ptr, P.n_rows, b);
    const int ns = P.nsplit[r];
    if (ns == 1) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int local = b - P.item_ptr[r];
    const int qt = local / ns, sp_i = local % ns;
    const int seq = r % P.n_seq, slot = r / P.n_seq;
    const int tok_base = P.tok_ptr[seq];
    const int t0 = qt * P.tpt;
    const int ntok = min(P.tpt, P.tok_ptr[seq + 1] - tok_base - t0);
    const int nrows = ntok * P.G;
    const int per = (nrows + ns - 1) / ns;
    const int r0 = sp_i * per, r1 = min(nrows, r0 + per);
    const int64_t part0 = (int64_t)P.part_ptr[r] + (int64_t)qt * ns;   // splits part0 .. part0+ns-1
    constexpr int DPL = D / 64;                                      // dims per lane
    for (int row = r0 + wave; row < r1; row += 4) {
        float M = -INFINITY;
        for (int s = lane; s < ns; s += 64) M = fmaxf(M, P.part_lse[(part0 + s) * BM + row]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
        float z = 0.f;
        for (int s = lane; s < ns; s += 64) {
            const float l = P.part_lse[(part0 + s) * BM + row];
            const float wgt = M == -INFINITY ? 0.f : __expf(l - M);
            sw[wave][s] = wgt;
            z += wgt;
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) z += __shfl_xor(z, m, 64);
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        float o[DPL];
#pragma unroll
        for (int i = 0; i < DPL; ++i) o[i] = 0.f;
        const float *src = P.part_o + (part0 * BM + row) * D + DPL * lane;
#pragma unroll 8
        for (int s = 0; s < ns; ++s) {
            const float wgt = sw[wave][s];
            const float *q = src + (int64_t)s * BM * D;
            if (DPL == 2) {
                const float2 v = *(const float2 *)q;
                o[0] += wgt * v.x;
                o[DPL - 1] += wgt * v.y;
            } else {
                o[0] += wgt * q[0];
            }
        }
        const float inv = z > 0.f ? 1.f / z : 0.f;
        const int tq = row / P.G, g = row % P.G;
        const int64_t orow = (int64_t)(tok_base + t0 + tq) * P.Hq + (int64_t)slot * P.G + g;
        if (DPL == 2) {
            *(uint32_t *)(P.out + orow * D + 2 * lane) = pack_bf16x2(o[0] * inv, o[DPL - 1] * inv);
        } else {
            P.out[orow * D + lane] = f32_to_bf16(o[0] * inv);
        }
        if (P.lse && lane == 0) P.lse[orow] = z > 0.f ? M + logf(z) : -INFINITY;
        __builtin_amdgcn_wave_barrier();
    }
}

// Writes the work-item prefix sums of the launch plan into the workspace; one
// workgroup, the same integer formulas as the host plan (row_items).
__global__ __launch_bounds__(256) void plan_kernel(const int32_t *__restrict__ row_ptr,
                                                   const int32_t *__restrict__ tok_ptr, int n_seq, int n_rows,
                                                   int tpt, int chunk, int32_t *item_ptr, int32_t *part_ptr,
                                                   int32_t *nsplit) {
    __shared__ int s_items[256], s_parts[256];
    __shared__ int carry_i, carry_p;
    if (threadIdx.x == 0) { carry_i = 0; carry_p = 0; }
    __syncthreads();
    for (int base = 0; base < n_rows; base += 256) {
        const int r = base + threadIdx.x;
        int it = 0, pt = 0;
        if (r < n_rows) {
            int nq = 1;
            if (tok_ptr) {
                const int q = r % n_seq;
                nq = (tok_ptr[q + 1] - tok_ptr[q] + tpt - 1) / tpt;
            }
            int ns;
            row_items(row_ptr[r + 1] - row_ptr[r], nq, chunk, &ns, &it);
            nsplit[r] = ns;
            pt = ns > 1 ? it : 0;
        }
        s_items[threadIdx.x] = it;
        s_parts[threadIdx.x] = pt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {   // inclusive scan
            const int a = threadIdx.x >= off ? s_items[threadIdx.x - off] : 0;
            const int c = threadIdx.x >= off ? s_parts[threadIdx.x - off] : 0;
            __syncthreads();
            s_items[threadIdx.x] += a;
            s_parts[threadIdx.x] += c;
            __syncthreads();
        }
        if (r < n_rows) {
            item_ptr[r] = carry_i + s_items[threadIdx.x] - it;
            part_ptr[r] = carry_p + s_parts[threadIdx.x] - pt;
        }
        __syncthreads();
        if (threadIdx.x == 255) { carry_i += s_items[255]; carry_p += s_parts[255]; }
        __syncthreads();
    }
    if (threadIdx.x == 0) { item_ptr[n_rows] = carry_i; part_ptr[n_rows] = carry_p; }
}

}  // namespace

int launch_plan(const Plan &p, const int32_t *d_row_ptr, const int32_t *d_tok_ptr, int n_seq, void *ws,
                hipStream_t stream) {
    char *w = (char *)ws;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, d_row_ptr, d_tok_ptr, n_seq, p.n_rows,
                       p.tok_per_tile, p.chunk_pages, (int32_t *)(w + p.off_item_ptr),
                       (int32_t *)(w + p.off_part_ptr), (int32_t *)(w + p.off_nsplit));
    return check_hip(hipGetLastError(), "plan launch");
}

int launch_prefill_f32(const AttnArgs &a, int64_t n_tok, hipStream_t stream);

int launch_prefill(const AttnArgs &a, const Plan &p, int64_t n_tok, hipStream_t stream) {
    if (a.dtype == SP_F32) return launch_prefill_f32(a, n_tok, stream);
    int rc = launch_plan(p, a.d_row_ptr, a.d_tok_ptr, a.n_seq, a.ws, stream);
    if (rc) return rc;
    char *w = (char *)a.ws;
    PrefillParams P;
    P.q = (const bf16 *)a.q;
    P.kp = (const bf16 *)a.k_pool;
    P.vp = (const bf16 *)a.v_pool;
    P.out = (bf16 *)a.out;
    P.lse = a.lse;
    P.tok_ptr = a.d_tok_ptr;
    P.q_pos0 = a.d_q_pos;
    P.cls = a.d_cls;
    P.window = a.d_window;
    P.row_ptr = a.d_row_ptr;
    P.entries = (const int4 *)a.d_entries;
    P.item_ptr = (const int32_t *)(w + p.off_item_ptr);
    P.part_ptr = (const int32_t *)(w + p.off_part_ptr);
    P.nsplit = (const int32_t *)(w + p.off_nsplit);
    P.part_o = (float *)(w + p.off_part_o);
    P.part_lse = (float *)(w + p.off_part_lse);
    P.n_seq = a.n_seq;
    P.n_rows = p.n_rows;
    P.G = a.group;
    P.ps = a.page_size;
    P.tpt = p.tok_per_tile;
    P.Hq = a.n_slot * a.group;
    P.n_phys = a.n_phys;
    P.scale_log2 = a.scale * kLog2e;
    const dim3 grid((unsigned)p.n_items);
#define SP_PREFILL_CASE(DD, PSV)                                                                        \
    if (a.head_dim == DD && a.page_size == PSV) {                                                       \
        if (p.waves == 8)                                                                               \
            hipLaunchKernelGGL((prefill_bf16_kernel<DD, 8, PSV>), grid, dim3(512), 0, stream, P);      \
        else                                                                                            \
            hipLaunchKernelGGL((prefill_bf16_kernel<DD, 4, PSV>), grid, dim3(256), 0, stream, P);      \
        if (p.n_parts)                                                                                  \
            hipLaunchKernelGGL(prefill_merge_kernel<DD>, grid, dim3(256), 0, stream, P, p.rows_per_tile); \
    }
    SP_PREFILL_CASE(128, 16) else SP_PREFILL_CASE(128, 32) else SP_PREFILL_CASE(128, 64)
    else SP_PREFILL_CASE(64, 16) else SP_PREFILL_CASE(64, 32) else SP_PREFILL_CASE(64, 64)
    else return fail(SP_EUNSUPPORTED, "bf16 prefill head_dim %d page_size %d", a.head_dim, a.page_size);
#undef SP_PREFILL_CASE
    return check_hip(hipGetLastError(), "prefill launch");
}

}  // namespace sp
