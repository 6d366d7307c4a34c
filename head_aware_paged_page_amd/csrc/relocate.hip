// rope_relocate kernel: rotate cached segment keys from their offline to their
// online rotary position, page by page.
//
// Follows the is96.com commentary on the RedKnot paper (RoPE paragraphs: undo
// the cached rotation, apply the online one) and the RedKnot product profile,
// section 3 (reused segment keys are re-aligned with rotary encoding).  The two
// rotations share their planes, so each pair (i, i + D/2) turns once by
// delta * w_i.  The angle is formed and reduced modulo 2*pi in fp64, its
// sine/cosine taken in fp64 and the rotation applied in fp32.
//
// HBM-bound streaming: each thread owns 8 consecutive pairs of one key row
// (16 B + 16 B for bf16), its 8 frequencies are fixed for the whole launch, and
// the 8 (cos, sin) are recomputed only when the page's shift changes - the
// workgroup walks a contiguous run of list entries, so that happens at segment
// boundaries only.
#include "device_common.hpp"

namespace sp {
namespace {

constexpr int kThreads = 256;
constexpr int kPagesPerBlock = 8;
constexpr double kTwoPiHi = 6.283185307179586232;      // 2*pi rounded to fp64
constexpr double kTwoPiLo = 2.4492935982947064e-16;    // 2*pi - kTwoPiHi

template <typename T>
struct Elem;
template <>
struct Elem<float> {
    typedef float4 V8[2];   // 8 fp32
    __device__ static void load(const float *p, float *x) {
        const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    __device__ static void store(float *p, const float *x) {
        *(float4 *)p = make_float4(x[0], x[1], x[2], x[3]);
        *(float4 *)(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
};
template <>
struct Elem<bf16> {
    __device__ static void load(const bf16 *p, float *x) {
        const u32x4 v = *(const u32x4 *)p;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            x[2 * w] = bf16_bits_to_f32(v[w] & 0xffffu);
            x[2 * w + 1] = bf16_bits_to_f32(v[w] >> 16);
        }
    }
    __device__ static void store(bf16 *p, const float *x) {
        u32x4 v;
#pragma unroll
        for (int w = 0; w < 4; ++w) v[w] = pack_bf16x2(x[2 * w], x[2 * w + 1]);
        *(u32x4 *)p = v;
    }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void relocate_kernel(const T *__restrict__ k_in, T *k_out, int ps, int D,
                                                            int64_t n_phys, int n, const int4 *__restrict__ list,
                                                            double log2_theta) {
    const int units_per_row = D / 16;            // a unit = 8 pairs of one key row
    const int ig = threadIdx.x % units_per_row;  // fixed for the launch (kThreads % units_per_row == 0)
    const int units_per_page = ps * units_per_row;
    const int half = D / 2;

    // this thread's 8 frequencies w_i = theta^(-2i/D), i = 8*ig .. 8*ig+7
    double w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = exp2(-(2.0 * (8 * ig + j) / D) * log2_theta);

    float c[8], s[8];
    int cached = 0;
    bool have = false;

    const int64_t first = (int64_t)blockIdx.x * kPagesPerBlock;
    const int pages = (int)min<int64_t>(kPagesPerBlock, n - first);
    const int total = pages * units_per_page;
    for (int u = threadIdx.x; u < total; u += kThreads) {
        const int pl = u / units_per_page;
        const int row = (u % units_per_page) / units_per_row;
        const int4 e = list[first + pl];   // {phys, delta, n_valid, reserved}
        if (row >= min(e.z, ps) || e.x < 0 || e.x >= n_phys) continue;
        if (!have || e.y != cached) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const double a = (double)e.y * w[j];
                const double q = rint(a * (1.0 / kTwoPiHi));
                const double r = fma(-q, kTwoPiLo, fma(-q, kTwoPiHi, a));   // a mod 2*pi, |r| <~ pi
                double sd, cd;
                sincos(r, &sd, &cd);
                c[j] = (float)cd;
                s[j] = (float)sd;
            }
            cached = e.y;
            have = true;
        }
        const int64_t base = ((int64_t)e.x * ps + row) * D + 8 * ig;
        float a[8], b[8];
        Elem<T>::load(k_in + base, a);
        Elem<T>::load(k_in + base + half, b);
        float ya[8], yb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            ya[j] = fmaf(a[j], c[j], -(b[j] * s[j]));
            yb[j] = fmaf(b[j], c[j], a[j] * s[j]);
        }
        Elem<T>::store(k_out + base, ya);
        Elem<T>::store(k_out + base + half, yb);
    }
}

}  // namespace

int launch_relocate(const void *k_in, void *k_out, int dtype, int page_size, int head_dim, int64_t n_phys, int n,
                    const sp_reloc *d_list, double theta, hipStream_t stream) {
    if (kThreads % (head_dim / 16) != 0)
        return fail(SP_EUNSUPPORTED, "rope_relocate head_dim %d (a power of two, 16..256)", head_dim);
    const int64_t blocks = (n + kPagesPerBlock - 1) / kPagesPerBlock;
    if (blocks > INT32_MAX) return fail(SP_EINVAL, "relocation list too long");
    const double l2t = log2(theta);
    if (dtype == SP_F32)
        hipLaunchKernelGGL(relocate_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           (const float *)k_in, (float *)k_out, page_size, head_dim, n_phys, n,
                           (const int4 *)d_list, l2t);
    else
        hipLaunchKernelGGL(relocate_kernel<bf16>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           (const bf16 *)k_in, (bf16 *)k_out, page_size, head_dim, n_phys, n,
                           (const int4 *)d_list, l2t);
    return check_hip(hipGetLastError(), "rope_relocate launch");
}

}  // namespace sp
