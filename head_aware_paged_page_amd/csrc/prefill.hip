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

// Output row m of a 32x32 MFMA tile <- K row sigma(m) of the 32-key block.
// Lane (n, h) holds rows m = (v/4)*8 + 4h + v%4; sigma maps them to keys
// 16*(v/8) + 8h + v%8, i.e. it swaps bits 2 and 3 of m.
__device__ __forceinline__ int sigma(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_bf16_kernel(PrefillParams P) {
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
    __shared__ int sFull[2];

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
    const int G = P.G, ps = P.ps;
    const bool is_local = P.cls[slot] == SP_LOCAL;
    const int W = is_local ? P.window[slot] : 0;
    const int nrows = ntok * G;

    // ---- the q-tile's visible entry range, then this split's share
    const int e_beg = P.row_ptr[r], e_end = P.row_ptr[r + 1];
    const int4 *E = P.entries;
    const int hi = first_greater(e_beg, e_end, p_last, [&](int e) { return E[e].y; });
    int lo = e_beg;
    if (is_local) lo = first_greater(e_beg, hi, p0 - W, [&](int e) { return E[e].y + E[e].z - 1; });
    const int ppt = BN / ps;                            // pages per tile
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

    // ---- tile staging: global -> registers -> LDS
    u32x4 rk[CPT], rv[CPT];
    auto load_tile = [&](int t) {
        const int e0 = my_lo + t * ppt;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT;
            rk[i] = u32x4{0, 0, 0, 0};
            rv[i] = u32x4{0, 0, 0, 0};
            if (c < KCH) {
                // K: chunk c -> key row j, 8 dims
                const int j = c / (D / 8), col = (c % (D / 8)) * 8;
                const int pg = j / ps, tk = j % ps;
                const int e = e0 + pg;
                if (e < my_hi) {
                    const int4 en = E[e];
                    if (tk < en.z && en.x >= 0 && en.x < P.n_phys)
                        rk[i] = *(const u32x4 *)(P.kp + ((int64_t)en.x * ps + tk) * D + col);
                }
                // V^T: chunk c -> page-major walk of the dim-major pages
                const int per_page = D * ps / 8;
                const int pv = c / per_page, rem = c % per_page;
                const int d = rem / (ps / 8), k8 = (rem % (ps / 8)) * 8;
                const int ev = e0 + pv;
                if (ev < my_hi) {
                    const int4 en = E[ev];
                    if (k8 < en.z && en.x >= 0 && en.x < P.n_phys) {
                        const u32x4 v = *(const u32x4 *)(P.vp + ((int64_t)en.x * D + d) * ps + k8);
                        rv[i] = keep_first_bf16(v, en.z - k8);
                    }
                }
            }
        }
    };
    auto store_tile = [&](int t, int buf) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT;
            if (c < KCH) {
                const int j = c / (D / 8), col = (c % (D / 8)) * 8;
                *(u32x4 *)&sK[buf][j * KS + col] = rk[i];
                const int per_page = D * ps / 8;
                const int pv = c / per_page, rem = c % per_page;
                const int d = rem / (ps / 8), k8 = (rem % (ps / 8)) * 8;
                *(u32x4 *)&sV[buf][d * VS + pv * ps + k8] = rv[i];
            }
        }
        if (tid < BN) {
            const int e0 = my_lo + t * ppt;
            const int pg = tid / ps, tk = tid % ps, e = e0 + pg;
            int pos = kPosInvalid;
            if (e < my_hi) {
                const int4 en = E[e];
                if (tk < en.z && en.x >= 0 && en.x < P.n_phys) pos = en.y + tk;
            }
            sPos[buf][tid] = pos;
        }
        if (tid == 0) {
            // the tile needs no bounds if every slot holds a token visible to every query of the q-tile
            const int e0 = my_lo + t * ppt;
            bool full = e0 + ppt <= my_hi;
            int kmin = INT32_MAX, kmax = INT32_MIN;
            for (int pg = 0; full && pg < ppt; ++pg) {
                const int4 en = E[e0 + pg];
                full = en.z == ps && en.x >= 0 && en.x < P.n_phys;
                kmin = min(kmin, en.y);
                kmax = max(kmax, en.y + en.z - 1);
            }
            full = full && kmax <= p0 && (!is_local || kmin > p_last - W);
            sFull[buf] = full;
        }
    };

    // ---- running softmax state (log2 domain) and O^T accumulators
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{0};

    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0, 0);
    }
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < n_tiles) load_tile(t + 1);

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
        // scale, bounds (boundary tiles only), online softmax
        const bool full = sFull[buf];
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < BN / 32; ++kt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float x = S[kt][v] * P.scale_log2;
                if (!full) {
                    const int kpos = sPos[buf][32 * kt + 16 * (v >> 3) + 8 * h + (v & 7)];
                    if (!(kpos <= pq && kpos > lowq)) x = -INFINITY;
                }
                S[kt][v] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = fmaxf(mx, xor_lane(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float rs = 0.f;
#pragma unroll
        for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = exp2f(S[kt][v] - m_use);
                S[kt][v] = p;
                rs += p;
            }
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;

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

        if (t + 1 < n_tiles) store_tile(t + 1, buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue
    const float l = l_run + xor_lane(l_run, 32);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse = l > 0.f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
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
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillParams P, int BM) {
    const int b = blockIdx.x;
    const int r = find_row(P.item_ptr, P.n_rows, b);
    const int ns = P.nsplit[r];
    const int local = b - P.item_ptr[r];
    if (ns == 1 || local % ns != 0) return;
    const int qt = local / ns;
    const int seq = r % P.n_seq, slot = r / P.n_seq;
    const int tok_base = P.tok_ptr[seq];
    const int t0 = qt * P.tpt;
    const int ntok = min(P.tpt, P.tok_ptr[seq + 1] - tok_base - t0);
    const int nrows = ntok * P.G;
    const int64_t part0 = (int64_t)P.part_ptr[r] + local;   // splits are part0 .. part0+ns-1
    constexpr int TPR = D / 4;                               // threads per row (4 dims each)
    for (int idx = threadIdx.x; idx < nrows * TPR; idx += 256) {
        const int row = idx / TPR, d = (idx % TPR) * 4;
        float M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, P.part_lse[(part0 + s) * BM + row]);
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        float z = 0.f;
        if (M != -INFINITY) {
            for (int s = 0; s < ns; ++s) {
                const float wgt = __expf(P.part_lse[(part0 + s) * BM + row] - M);
                const float4 v = *(const float4 *)(P.part_o + ((part0 + s) * BM + row) * D + d);
                o.x += wgt * v.x; o.y += wgt * v.y; o.z += wgt * v.z; o.w += wgt * v.w;
                z += wgt;
            }
        }
        const float inv = z > 0.f ? 1.f / z : 0.f;
        const int tq = row / P.G, g = row % P.G;
        const int64_t orow = (int64_t)(tok_base + t0 + tq) * P.Hq + (int64_t)slot * P.G + g;
        u32x2 w;
        w[0] = pack_bf16x2(o.x * inv, o.y * inv);
        w[1] = pack_bf16x2(o.z * inv, o.w * inv);
        *(u32x2 *)(P.out + orow * D + d) = w;
        if (P.lse && d == 0) P.lse[orow] = z > 0.f ? M + logf(z) : -INFINITY;
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
    if (a.head_dim == 128) {
        hipLaunchKernelGGL((prefill_bf16_kernel<128, 4>), grid, dim3(256), 0, stream, P);
        if (p.n_parts) hipLaunchKernelGGL(prefill_merge_kernel<128>, grid, dim3(256), 0, stream, P, p.rows_per_tile);
    } else {
        hipLaunchKernelGGL((prefill_bf16_kernel<64, 4>), grid, dim3(256), 0, stream, P);
        if (p.n_parts) hipLaunchKernelGGL(prefill_merge_kernel<64>, grid, dim3(256), 0, stream, P, p.rows_per_tile);
    }
    return check_hip(hipGetLastError(), "prefill launch");
}

}  // namespace sp
