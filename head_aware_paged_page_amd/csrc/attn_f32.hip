// fp32 SegPaged attention (prefill and decode): exact-precision path, VALU only.
//
// Same computation as the bf16 kernels - softmax attention of each query over
// the tokens its head's page table and class make visible (RedKnot product
// profile, section 3) - with fp32 inputs, fp32 arithmetic and fp32 outputs and
// no reduced precision anywhere.  One wave per (query token, query head); keys
// are visited in table order with a running (max, sum) softmax.
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

__global__ __launch_bounds__(64) void attn_f32_kernel(F32Params P) {
    const int lane = threadIdx.x;
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

    float qv[4], o[4];
    const float *qrow = P.q + ((int64_t)tok * P.Hq + head) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        qv[i] = d < D ? qrow[d] : 0.f;
        o[i] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int e = P.row_ptr[r]; e < P.row_ptr[r + 1]; ++e) {
        const int4 en = P.entries[e];
        if (en.x < 0 || en.x >= P.n_phys) continue;
        const int nv = min(en.z, ps);
        if (en.y > p || en.y + nv - 1 <= low) continue;
        for (int tk = 0; tk < nv; ++tk) {
            const int pos = en.y + tk;
            if (!(pos <= p && pos > low)) continue;
            const float *krow = P.kp + ((int64_t)en.x * ps + tk) * D;
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = lane + 64 * i;
                if (d < D) part = fmaf(qv[i], krow[d], part);
            }
            const float s = wave_sum(part) * P.scale;
            const float m_new = fmaxf(m, s);
            const float alpha = expf(m - m_new);
            const float w = expf(s - m_new);
            l = l * alpha + w;
            const float *vcol = P.vp + (int64_t)en.x * D * ps + tk;   // V page is dim-major
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = lane + 64 * i;
                if (d < D) o[i] = fmaf(w, vcol[(int64_t)d * ps], o[i] * alpha);
            }
            m = m_new;
        }
    }
    float *orow = P.out + ((int64_t)tok * P.Hq + head) * D;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        if (d < D) orow[d] = o[i] * inv;
    }
    if (P.lse && lane == 0) P.lse[(int64_t)tok * P.Hq + head] = l > 0.f ? m + logf(l) : -INFINITY;
}

int launch_f32(const AttnArgs &a, int64_t n_tok, const int32_t *tok_ptr, hipStream_t stream) {
    if (a.head_dim > 256) return fail(SP_EUNSUPPORTED, "fp32 head_dim %d > 256", a.head_dim);
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
    hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)n_tok, (unsigned)P.Hq), dim3(64), 0, stream, P);
    return check_hip(hipGetLastError(), "fp32 attention launch");
}

}  // namespace

int launch_prefill_f32(const AttnArgs &a, int64_t n_tok, hipStream_t stream) {
    return launch_f32(a, n_tok, a.d_tok_ptr, stream);
}

int launch_decode_f32(const AttnArgs &a, hipStream_t stream) { return launch_f32(a, a.n_seq, nullptr, stream); }

}  // namespace sp
