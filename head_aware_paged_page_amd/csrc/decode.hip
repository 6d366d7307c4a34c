// segpaged_decode for bf16: one query token per sequence attends over each
// head's own page table, split over the page list, merged by log-sum-exp.
//
// Follows the RedKnot product profile, section 3 (each head reads only its own
// pages / visible window, no mask) and the RedKnot HotpotQA tutorial page, which
// notes the decode side is left essentially unchanged: it is the ordinary
// split-K paged decode, walking the per-head table.  Decode is bound by memory
// bandwidth (the Prefill/Decode explainer listed on the PagedAttention &
// RadixAttention page), so the kernel is built around streaming K/V pages
// straight from HBM into MFMA operand registers, with no LDS staging:
//   K pages are token-major: lane (key, 8-dim group) loads 16 B = the A operand
//   of S^T = K Q^T (v_mfma_f32_16x16x32_bf16, keys x heads);
//   V pages are dim-major: lane (dim, 8-key group) loads 16 B = the A operand of
//   O^T = V^T P^T (same instruction, dims x heads).
// The keys fed to the first product are permuted so that each lane's scores are
// the 8 consecutive keys its B operand of the second product needs.  Each wave
// streams 32-key blocks (one or two pages) with the next block's loads in
// flight; the waves of a workgroup merge through LDS at the end.
#include "device_common.hpp"

namespace sp {
namespace {

constexpr int KB = kDecodeKeysPerBlock;   // 32 keys per block
constexpr int NWD = kDecodeWaves;

struct DecodeParams {
    const bf16 *q, *kp, *vp;
    bf16 *out;
    float *lse;
    const int32_t *q_pos, *cls, *window, *row_ptr;
    const int4 *entries;
    const int32_t *item_ptr, *item_ptr2, *part_ptr, *nsplit;
    float *part_o, *part_lse;
    int n_seq, n_rows, G, ps, Hq;
    int64_t n_phys;
    float scale_log2;
};


template <int D>
struct Block {
    u32x4 k[2][D / 32];   // S^T A operands: [key tile][k-step]
    u32x4 v[D / 16];      // O^T A operands: [dim tile]
    int y[2], z[2];       // pos_start / n_valid of the block's (one or two) pages, wave-uniform
};

// Loads one 32-key block whose table entries sit in LDS at sE[e0 - base ..]
// (already sanitised: out-of-range pages have n_valid 0).
template <int D, int ps>
__device__ __forceinline__ void load_block(const DecodeParams &P, const int4 *sE, int e0, int e_hi, Block<D> &B) {
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, grp = lane >> 4;
    // entries of the block's pages (one or two), wave-uniform; kept as plain
    // integers (a select between two int4 values of an array can become an
    // indexed load from private memory)
    int px[2], py[2], pz[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int e = e0 + i;
        px[i] = py[i] = pz[i] = 0;
        if (i * ps < KB && e < e_hi) {
            const int4 v = sE[i];
            px[i] = __builtin_amdgcn_readfirstlane(v.x);
            py[i] = __builtin_amdgcn_readfirstlane(v.y);
            pz[i] = __builtin_amdgcn_readfirstlane(v.z);
        }
        B.y[i] = py[i];
        B.z[i] = pz[i];
    }
    // K: A operand row m of key tile kt is key 8*(m/4) + 4*kt + m%4; dims 32*s + 8*grp.
    // Slots without a token are read from page 0 and never zeroed: their scores
    // are replaced by -inf before use, so whatever they hold cannot leak.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        const int j = 8 * (m >> 2) + 4 * kt + (m & 3);
        const int pg = j / ps, tk = j % ps;
        const int phys = pg ? px[1] : px[0];
        const bf16 *src = P.kp + ((int64_t)phys * ps + tk) * D + 8 * grp;
#pragma unroll
        for (int s = 0; s < D / 32; ++s) B.k[kt][s] = *(const u32x4 *)(src + 32 * s);
    }
    // V^T: A operand row = dim 16*dt + m, keys 8*grp .. 8*grp+7.  Values of empty
    // slots are zeroed when the block is used, not here: the loads must stay in
    // flight while the previous block computes.
    {
        const int j = 8 * grp;
        const int pg = j / ps, tk = j % ps;
        const int phys = pg ? px[1] : px[0];
        const bf16 *src = P.vp + ((int64_t)phys * D + m) * ps + tk;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) B.v[dt] = *(const u32x4 *)(src + (int64_t)16 * dt * ps);
    }
}

// Position of key j (0..31) of a block, kPosInvalid if its slot holds no token.
template <int ps, int D>
__device__ __forceinline__ int block_pos(const Block<D> &B, int j) {
    const int pg = j / ps, tk = j % ps;
    const int y = pg ? B.y[1] : B.y[0], z = pg ? B.z[1] : B.z[0];
    return tk < z ? y + tk : kPosInvalid;
}

template <int D, int PS, bool INL>
__global__ __launch_bounds__(NWD * 64) __attribute__((amdgpu_waves_per_eu(3, 3))) void decode_bf16_kernel(
    DecodeParams P, InlinePlan L) {
    constexpr int DS = D / 32;   // k-steps of S^T
    constexpr int DT = D / 16;   // dim tiles of O^T
    __shared__ float sM[NWD][16], sL[NWD][16];
    __shared__ float sO[NWD][D][17];
    __shared__ int4 sE[kDecodeMaxChunk + 2];

    const int lane = threadIdx.x & 63;
    // The wave index is uniform, but the compiler cannot tell from threadIdx.x:
    // said explicitly, the block loop below is a scalar loop rather than an
    // exec-masked one (32K decode kernel 43 -> 35 us).
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, grp = lane >> 4;

    int r, sp_i;
    if (INL) item_of(L.item_ptr, L.item_ptr2, P.n_rows, blockIdx.x, &r, &sp_i);
    else item_of(P.item_ptr, P.item_ptr2, P.n_rows, blockIdx.x, &r, &sp_i);
    const int ns = INL ? L.nsplit[r] : P.nsplit[r];
    const int seq = r % P.n_seq, slot = r / P.n_seq;
    const int G = P.G;
    constexpr int ps = PS;
    const int p = P.q_pos[seq];
    const bool is_local = P.cls[slot] == SP_LOCAL;
    const int low = is_local ? p - P.window[slot] : INT32_MIN;   // visible iff low < pos <= p

    const int e_beg = P.row_ptr[r], e_end = P.row_ptr[r + 1];
    const int4 *E = P.entries;
    int lo, hi;
    visible_range(E, e_beg, e_end, p, is_local, low, &lo, &hi);
    constexpr int ppb = KB / ps;                      // pages per 32-key block (page_size 16 or 32)
    int chunk = (hi - lo + ns - 1) / ns;
    chunk = (chunk + ppb - 1) / ppb * ppb;
    const int my_lo = min(hi, lo + sp_i * chunk);
    const int my_hi = min(hi, my_lo + min(chunk, kDecodeMaxChunk));
    const int n_blocks = (my_hi - my_lo + ppb - 1) / ppb;

    // Q^T B operand: head n of the slot, dims 32*s + 8*grp (read before the
    // barrier below, so their latency overlaps that of the entries)
    bf16x8 qf[DS];
    {
        const bool ok = n < G;
        const bf16 *qrow = P.q + ((int64_t)seq * P.Hq + (int64_t)slot * G + (ok ? n : 0)) * D + 8 * grp;
#pragma unroll
        for (int s = 0; s < DS; ++s) qf[s] = u4_as_bf16x8(ok ? *(const u32x4 *)(qrow + 32 * s) : u32x4{0, 0, 0, 0});
    }

    // this split's table entries -> LDS, sanitised (out-of-range pages hold no token)
    for (int i = threadIdx.x; i < my_hi - my_lo; i += NWD * 64) {
        int4 en = E[my_lo + i];
        if (en.x < 0 || en.x >= P.n_phys) en = int4{0, 0, 0, 0};
        en.z = min(en.z, ps);
        sE[i] = en;
    }
    __syncthreads();


    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One block in registers per wave; latency is hidden across the waves (three
    // per SIMD) rather than by a second register buffer, which would halve them.
    auto use = [&](Block<D> &cur) {
        f32x4 S[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            S[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < DS; ++s) S[kt] = mfma16x16x32(u4_as_bf16x8(cur.k[kt][s]), qf[s], S[kt]);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int kpos = block_pos<PS, D>(cur, 8 * grp + 4 * kt + v);
                float x = S[kt][v] * P.scale_log2;
                if (!(kpos <= p && kpos > low)) x = -INFINITY;
                S[kt][v] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, xor_lane(mx, 16));
        mx = fmaxf(mx, xor_lane(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);   // exponent <= 0
        float rs = 0.f;
        u32x4 pk;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            float pv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                pv[v] = __builtin_amdgcn_exp2f(S[kt][v] - m_use);
                rs += pv[v];
            }
            pk[2 * kt] = pack_bf16x2(pv[0], pv[1]);
            pk[2 * kt + 1] = pack_bf16x2(pv[2], pv[3]);
        }
        l_run = l_run * alpha + rs;
        m_run = m_new;
        // values of empty slots must be zero (their weight is zero, but 0 * NaN
        // is not); only blocks that hold such slots pay for it
        const int keep = (8 * grp / PS ? cur.z[1] : cur.z[0]) - (8 * grp) % PS;
        if (__any(keep < 8)) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                cur.v[dt] = keep >= 8 ? cur.v[dt] : (keep > 0 ? keep_first_bf16(cur.v[dt], keep) : u32x4{0, 0, 0, 0});
        }
        const bf16x8 pb = u4_as_bf16x8(pk);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma16x16x32(u4_as_bf16x8(cur.v[dt]), pb, acc[dt] * alpha);
    };
    auto load = [&](int bk, Block<D> &B) { load_block<D, PS>(P, sE + bk * ppb, my_lo + bk * ppb, my_hi, B); };
    Block<D> blk_regs;
    for (int blk = wave; blk < n_blocks; blk += NWD) {
        load(blk, blk_regs);
        use(blk_regs);
    }

    // ---- combine the workgroup's waves
    float l = l_run + xor_lane(l_run, 16);
    l += xor_lane(l, 32);
    if (grp == 0) {
        sM[wave][n] = m_run;
        sL[wave][n] = l;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 4; ++v) sO[wave][16 * dt + 4 * grp + v][n] = acc[dt][v];
    __syncthreads();
    const int64_t part = ns > 1 ? (int64_t)(INL ? L.part_ptr[r] : P.part_ptr[r]) + sp_i : 0;
    for (int idx = threadIdx.x; idx < G * D; idx += NWD * 64) {
        const int hh = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWD; ++w) M = fmaxf(M, sM[w][hh]);
        float o = 0.f, z = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < NWD; ++w) {
                const float f = exp2f(sM[w][hh] - M);
                o += f * sO[w][d][hh];
                z += f * sL[w][hh];
            }
        }
        const float inv = z > 0.f ? 1.f / z : 0.f;
        const float lse = z > 0.f ? (M + log2f(z)) * kLn2 : -INFINITY;
        const int64_t orow = (int64_t)seq * P.Hq + (int64_t)slot * G + hh;
        if (ns == 1) {
            P.out[orow * D + d] = f32_to_bf16(o * inv);
            if (P.lse && d == 0) P.lse[orow] = lse;
        } else {
            P.part_o[(part * G + hh) * D + d] = o * inv;
            if (d == 0) P.part_lse[part * G + hh] = lse;
        }
    }
}

// Merges the splits of every split row: one workgroup of kMergeWaves waves per
// (row, head).  The threads read the split LSEs together (thread s, s + 256,
// ...) and form the weights e^{lse_s - M} in LDS; then O = sum_s w_s o_s /
// sum_s w_s.  Lane (g, c) of wave w accumulates dims 8c .. 8c+7 over splits
// w*SG + g, + kMergeWaves*SG, ..., so a row cut into many splits (a small
// call splits its rows finely) is summed by 16 lane groups at once; the
// groups are added by lane exchanges within a wave and through LDS across
// waves.  The partial outputs of a lane's first kPreSplits splits are loaded
// before the LSEs are reduced, so both loads are in flight together.
constexpr int kMergeWaves = 4;

template <int D, bool INL>
__global__ __launch_bounds__(64 * kMergeWaves) void decode_merge_kernel(DecodeParams P, InlinePlan L) {
    constexpr int CH = D / 8, SG = 64 / CH, TG = SG * kMergeWaves;
    constexpr int kPreSplits = 8;
    __shared__ float sw[kMaxSplits];
    __shared__ float sMr[kMergeWaves], sZr[kMergeWaves];
    __shared__ float sO[kMergeWaves][D];
    const int r = blockIdx.x, hh = blockIdx.y;
    const int ns = INL ? L.nsplit[r] : P.nsplit[r];
    if (ns == 1) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int seq = r % P.n_seq, slot = r / P.n_seq, G = P.G;
    const int64_t part0 = INL ? L.part_ptr[r] : P.part_ptr[r];
    const int c = lane % CH, g = wave * SG + lane / CH;
    const float *src = P.part_o + (part0 * G + hh) * D + 8 * c;
    f32x4 pre0[kPreSplits], pre1[kPreSplits];
#pragma unroll
    for (int i = 0; i < kPreSplits; ++i) {
        const int s = g + i * TG;
        if (s < ns) {
            pre0[i] = *(const f32x4 *)(src + (int64_t)s * G * D);
            pre1[i] = *(const f32x4 *)(src + (int64_t)s * G * D + 4);
        }
    }
    float M = -INFINITY;
    for (int s = tid; s < ns; s += 64 * kMergeWaves) M = fmaxf(M, P.part_lse[(part0 + s) * G + hh]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
    if (lane == 0) sMr[wave] = M;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) M = fmaxf(M, sMr[w]);
    float z = 0.f;
    for (int s = tid; s < ns; s += 64 * kMergeWaves) {
        const float wgt = M == -INFINITY ? 0.f : __expf(P.part_lse[(part0 + s) * G + hh] - M);
        sw[s] = wgt;
        z += wgt;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) z += __shfl_xor(z, m, 64);
    if (lane == 0) sZr[wave] = z;
    __syncthreads();   // the weights and the partial sums of z
    z = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) z += sZr[w];
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
    for (int i = 0; i < kPreSplits; ++i) {
        const int s = g + i * TG;
        if (s < ns) {
            const float wgt = sw[s];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[e] += wgt * pre0[i][e];
                o[4 + e] += wgt * pre1[i][e];
            }
        }
    }
#pragma unroll 4
    for (int s = g + kPreSplits * TG; s < ns; s += TG) {
        const float wgt = sw[s];
        const f32x4 a0 = *(const f32x4 *)(src + (int64_t)s * G * D), a1 = *(const f32x4 *)(src + (int64_t)s * G * D + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o[e] += wgt * a0[e];
            o[4 + e] += wgt * a1[e];
        }
    }
#pragma unroll
    for (int off = CH; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], off, 64);
    if (lane < CH) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sO[wave][8 * c + e] = o[e];
    }
    __syncthreads();
    if (wave != 0 || lane >= CH) return;
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += sO[w][8 * c + e];
    const float inv = z > 0.f ? 1.f / z : 0.f;
    const int64_t orow = (int64_t)seq * P.Hq + (int64_t)slot * G + hh;
    u32x4 pk;
#pragma unroll
    for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(o[2 * i] * inv, o[2 * i + 1] * inv);
    *(u32x4 *)(P.out + orow * D + 8 * c) = pk;
    if (P.lse && lane == 0) P.lse[orow] = z > 0.f ? M + logf(z) : -INFINITY;
}

}  // namespace

int launch_plan(const Plan &p, const int32_t *d_row_ptr, const int32_t *d_tok_ptr, int n_seq, void *ws,
                hipStream_t stream);
int launch_decode_f32(const AttnArgs &a, hipStream_t stream);

int launch_decode(const AttnArgs &a, const Plan &p, hipStream_t stream) {
    if (a.dtype == SP_F32) return launch_decode_f32(a, stream);
    // Few rows: the plan (the same integer formulas as the plan kernel) goes in
    // the kernel arguments; otherwise the plan kernel writes it to the workspace.
    const bool inl = p.n_rows <= kInlineRows && a.h_row_ptr != nullptr;
    InlinePlan L;
    if (inl) {
        fill_inline_plan(p.n_rows, a.n_seq, a.h_row_ptr, nullptr, 1, p.chunk_pages, &L);
    } else {
        L.item_ptr[0] = 0;
        const int rc = launch_plan(p, a.d_row_ptr, nullptr, a.n_seq, a.ws, stream);
        if (rc) return rc;
    }
    char *w = (char *)a.ws;
    DecodeParams P;
    P.q = (const bf16 *)a.q;
    P.kp = (const bf16 *)a.k_pool;
    P.vp = (const bf16 *)a.v_pool;
    P.out = (bf16 *)a.out;
    P.lse = a.lse;
    P.q_pos = a.d_q_pos;
    P.cls = a.d_cls;
    P.window = a.d_window;
    P.row_ptr = a.d_row_ptr;
    P.entries = (const int4 *)a.d_entries;
    P.item_ptr = (const int32_t *)(w + p.off_item_ptr);
    P.item_ptr2 = (const int32_t *)(w + p.off_item_ptr2);
    P.part_ptr = (const int32_t *)(w + p.off_part_ptr);
    P.nsplit = (const int32_t *)(w + p.off_nsplit);
    P.part_o = (float *)(w + p.off_part_o);
    P.part_lse = (float *)(w + p.off_part_lse);
    P.n_seq = a.n_seq;
    P.n_rows = p.n_rows;
    P.G = a.group;
    P.ps = a.page_size;
    P.Hq = a.n_slot * a.group;
    P.n_phys = a.n_phys;
    P.scale_log2 = a.scale * kLog2e;
    const dim3 grid((unsigned)p.n_items);
    const dim3 mgrid(p.n_rows, a.group);
#define SP_DECODE_CASE(DD, PSV)                                                                                 \
    if (a.head_dim == DD && a.page_size == PSV) {                                                               \
        if (inl) {                                                                                              \
            hipLaunchKernelGGL((decode_bf16_kernel<DD, PSV, true>), grid, dim3(NWD * 64), 0, stream, P, L);    \
            if (p.n_parts) hipLaunchKernelGGL((decode_merge_kernel<DD, true>), mgrid, dim3(64 * kMergeWaves), 0, stream, P, L); \
        } else {                                                                                                \
            hipLaunchKernelGGL((decode_bf16_kernel<DD, PSV, false>), grid, dim3(NWD * 64), 0, stream, P, L);   \
            if (p.n_parts) hipLaunchKernelGGL((decode_merge_kernel<DD, false>), mgrid, dim3(64 * kMergeWaves), 0, stream, P, L); \
        }                                                                                                       \
    }
    SP_DECODE_CASE(128, 16) else SP_DECODE_CASE(128, 32) else SP_DECODE_CASE(64, 16) else SP_DECODE_CASE(64, 32)
    else return fail(SP_EUNSUPPORTED, "bf16 decode head_dim %d page_size %d", a.head_dim, a.page_size);
#undef SP_DECODE_CASE
    return check_hip(hipGetLastError(), "decode launch");
}

}  // namespace sp
