// fp32 SegPaged attention (prefill and decode): exact-precision path, VALU only.
//
// Same computation as the bf16 kernels - softmax attention of each query over
// the tokens its head's page table and class make visible (RedKnot product
// profile, section 3) - with fp32 inputs, fp32 arithmetic and fp32 outputs and
// no reduced precision anywhere.  A workgroup of kF32Waves waves takes one
// (query token, query head); its waves share the head's table in chunks of 64
// keys (wave w takes chunks w, w + kF32Waves, ...): 64 / page_size whole pages
// for pages of at most 64 keys (lane t scores key t % page_size of the chunk's
// page t / page_size), or 64 keys of one longer page.  The query sits in LDS,
// key rows are read as float4s; the wave takes the chunk's max and weights,
// and lane d then accumulates output dims d, d + 64, ... over the chunk's keys
// from the dim-major value pages.  A running (max, sum) carries each wave's
// softmax across its chunks, and the waves' states are merged at the end
// (log-sum-exp weights, in fp32), so the chain of dependent loads a call waits
// for is an eighth of the table's.
#include "device_common.hpp"

namespace sp {
namespace {

struct F32Params {
    const float *q, *kp, *vp;
    float *out, *lse;
    const int32_t *tok_ptr;   // prefill: [n_seq+1]; decode: nullptr (token = seq)
    const int32_t *q_pos, *cls, *window, *row_ptr;
    const int4 *entries;
    int n_seq, G, ps, Hq, D;
    int64_t n_phys;
    float scale;
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

constexpr int kF32MaxDim = 256;
constexpr int kF32Waves = 8;   // waves per (query token, query head)

// Orders this wave's LDS writes before its lanes read each other's (one wave's
// LDS operations complete in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

// Scores the key at (page phys, slot kk) against the query in LDS.
__device__ __forceinline__ float f32_score(const F32Params &P, int phys, int kk, const float *sq) {
    const float4 *krow = (const float4 *)(P.kp + ((int64_t)phys * P.ps + kk) * P.D);
    const float4 *q4 = (const float4 *)sq;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int j = 0; j < P.D / 4; ++j) {
        const float4 k = krow[j], qq = q4[j];
        a0 = fmaf(qq.x, k.x, a0);
        a1 = fmaf(qq.y, k.y, a1);
        a2 = fmaf(qq.z, k.z, a2);
        a3 = fmaf(qq.w, k.w, a3);
    }
    return ((a0 + a1) + (a2 + a3)) * P.scale;
}

template <bool LONG_PAGES>
__global__ __launch_bounds__(64 * kF32Waves) void attn_f32_kernel(F32Params P) {
    constexpr int NW = kF32Waves;
    __shared__ __attribute__((aligned(16))) float sq[kF32MaxDim];
    __shared__ float sw_all[NW][64];
    __shared__ int sPhys_all[NW][64], sNv_all[NW][64];   // per page of a chunk: id, keys to read from its value page (0: none)
    __shared__ float sM[NW], sL[NW];
    __shared__ float sO[NW][kF32MaxDim];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    float *sw = sw_all[wave];
    int *sPhys = sPhys_all[wave], *sNv = sNv_all[wave];
    const int tok = blockIdx.x, head = blockIdx.y;
    const int slot = head / P.G;
    int seq, p;
    if (P.tok_ptr) {
        int lo = 0, hi = P.n_seq;   // tok_ptr[lo] <= tok < tok_ptr[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (P.tok_ptr[mid] <= tok) lo = mid; else hi = mid;
        }
        while (lo + 1 < P.n_seq && P.tok_ptr[lo + 1] <= tok) ++lo;   // skip sequences without tokens
        seq = lo;
        p = P.q_pos[seq] + (tok - P.tok_ptr[seq]);
    } else {
        seq = tok;
        p = P.q_pos[seq];
    }
    const int r = slot * P.n_seq + seq;
    const bool is_local = P.cls[slot] == SP_LOCAL;
    const int low = is_local ? p - P.window[slot] : INT32_MIN;   // visible iff low < pos <= p
    const int D = P.D, ps = P.ps;

    const float *qrow = P.q + ((int64_t)tok * P.Hq + head) * D;
    for (int d = threadIdx.x; d < D; d += 64 * NW) sq[d] = qrow[d];
    __syncthreads();

    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = 0.f;
    float m = -INFINITY, l = 0.f;
    // one softmax step over a chunk whose visible keys have scores s (-inf
    // elsewhere) and whose value pages sPhys / sNv describe (n_pg pages,
    // columns c0 .. c0 + sNv - 1 of each)
    auto step = [&](float s, bool vis, int n_pg, int c0) {
        const float m_new = fmaxf(m, wave_max(s));
        if (m_new == -INFINITY) return;                 // nothing visible yet (wave-uniform)
        const float alpha = expf(m - m_new);            // 0 while m is -inf
        const float w = vis ? expf(s - m_new) : 0.f;
        l = l * alpha + wave_sum(w);
        sw[lane] = w;
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = lane + 64 * i;
            if (d >= D) continue;
            float acc = 0.f;
            for (int pg = 0; pg < n_pg; ++pg) {
                const int nv = sNv[pg];
                const float *vrow = P.vp + ((int64_t)sPhys[pg] * D + d) * ps + c0;   // V pages are dim-major: [D][ps]
                const float *wp = sw + (LONG_PAGES ? 0 : pg * ps);
                for (int k = 0; k < nv; ++k) acc = fmaf(wp[k], vrow[k], acc);
            }
            o[i] = o[i] * alpha + acc;
        }
        m = m_new;
    };
    const int e_beg = P.row_ptr[r], e_end = P.row_ptr[r + 1];
    if (!LONG_PAGES) {
        // chunks of ppc whole pages; lane t holds key t % ps of page t / ps
        const int ppc = max(1, 64 / ps);
        const int pg = lane / ps, kk = lane % ps;
        for (int e0 = e_beg + wave * ppc; e0 < e_end; e0 += NW * ppc) {
            const int n_pg = min(ppc, e_end - e0);
            bool vis = false;
            int phys = 0, nv = 0;
            if (pg < n_pg) {
                const int4 en = P.entries[e0 + pg];
                if (en.x >= 0 && en.x < P.n_phys) {
                    phys = en.x;
                    nv = max(0, min(en.z, ps));
                    const int pos = en.y + kk;
                    vis = kk < nv && pos <= p && pos > low;
                    if (nv > 0 && (en.y > p || en.y + nv - 1 <= low)) nv = 0;   // no key of the page visible
                }
            }
            const float s = vis ? f32_score(P, phys, kk, sq) : -INFINITY;
            if (kk == 0 && pg < n_pg) {
                sPhys[pg] = phys;
                sNv[pg] = nv;
            }
            step(s, vis, n_pg, 0);
            wave_lds_sync();   // sw, sPhys, sNv are rewritten by the next chunk
        }
    } else {
        for (int e = e_beg + wave; e < e_end; e += NW) {
            const int4 en = P.entries[e];
            if (en.x < 0 || en.x >= P.n_phys) continue;
            const int nv = min(en.z, ps);
            if (nv <= 0 || en.y > p || en.y + nv - 1 <= low) continue;
            for (int k0 = 0; k0 < nv; k0 += 64) {
                const int kk = k0 + lane;
                const int pos = en.y + kk;
                const bool vis = kk < nv && pos <= p && pos > low;
                const float s = vis ? f32_score(P, en.x, kk, sq) : -INFINITY;
                if (lane == 0) {
                    sPhys[0] = en.x;
                    sNv[0] = min(nv - k0, 64);
                }
                step(s, vis, 1, k0);
                wave_lds_sync();
            }
        }
    }
    // merge the waves' (max, sum, unnormalised output) states
    if (lane == 0) {
        sM[wave] = m;
        sL[wave] = l;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        if (d < D) sO[wave][d] = o[i];
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sM[w]);
    float z = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NW; ++w) z += sL[w] * expf(sM[w] - M);   // a wave that saw nothing has l = 0
    }
    const float inv = z > 0.f ? 1.f / z : 0.f;
    float *orow = P.out + ((int64_t)tok * P.Hq + head) * D;
    for (int d = threadIdx.x; d < D; d += 64 * NW) {
        float acc = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < NW; ++w)
                if (sM[w] != -INFINITY) acc += sO[w][d] * expf(sM[w] - M);
        }
        orow[d] = acc * inv;
    }
    if (P.lse && threadIdx.x == 0) P.lse[(int64_t)tok * P.Hq + head] = z > 0.f ? M + logf(z) : -INFINITY;
}

int launch_f32(const AttnArgs &a, int64_t n_tok, const int32_t *tok_ptr, hipStream_t stream) {
    if (a.head_dim > kF32MaxDim || a.head_dim % 4 != 0)
        return fail(SP_EUNSUPPORTED, "fp32 head_dim %d (a multiple of 4, at most %d)", a.head_dim, kF32MaxDim);
    if (n_tok > INT32_MAX) return fail(SP_EINVAL, "too many query tokens");
    F32Params P;
    P.q = (const float *)a.q;
    P.kp = (const float *)a.k_pool;
    P.vp = (const float *)a.v_pool;
    P.out = (float *)a.out;
    P.lse = a.lse;
    P.tok_ptr = tok_ptr;
    P.q_pos = a.d_q_pos;
    P.cls = a.d_cls;
    P.window = a.d_window;
    P.row_ptr = a.d_row_ptr;
    P.entries = (const int4 *)a.d_entries;
    P.n_seq = a.n_seq;
    P.G = a.group;
    P.ps = a.page_size;
    P.Hq = a.n_slot * a.group;
    P.D = a.head_dim;
    P.n_phys = a.n_phys;
    P.scale = a.scale;
    const dim3 grid((unsigned)n_tok, (unsigned)P.Hq);
    if (a.page_size > 64) hipLaunchKernelGGL(attn_f32_kernel<true>, grid, dim3(64 * kF32Waves), 0, stream, P);
    else hipLaunchKernelGGL(attn_f32_kernel<false>, grid, dim3(64 * kF32Waves), 0, stream, P);
    return check_hip(hipGetLastError(), "fp32 attention launch");
}

}  // namespace

int launch_prefill_f32(const AttnArgs &a, int64_t n_tok, hipStream_t stream) {
    return launch_f32(a, n_tok, a.d_tok_ptr, stream);
}

int launch_decode_f32(const AttnArgs &a, hipStream_t stream) { return launch_f32(a, a.n_seq, nullptr, stream); }

}  // namespace sp
