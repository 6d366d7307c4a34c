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
// HBM-bound streaming: a workgroup takes a run of list items worth 16 KB of
// keys (4 pages of 16 bf16 keys of 128 dims; staged in LDS) and issues all
// their loads at once (streaming, non-temporal loads and stores:
// every byte is touched once; the table builder lists pages in address order,
// so a run is mostly one contiguous stretch of the pool).  While the loads are
// in flight it builds one (cos, sin) table of D/2 angles per distinct delta of
// the run (a sequence has one delta per segment); then every thread rotates
// units of 8 consecutive pairs of one key row (16 B + 16 B for bf16).
#include "device_common.hpp"

namespace sp {
namespace {

constexpr int kThreads = 256;
constexpr int kBlockKeyBytes = 16384;   // keys one workgroup moves (timed best on MI355X at page 16 and 32)

// Pages per workgroup: kBlockKeyBytes of keys when the page shape is known at
// compile time (PS, DD > 0), else 4.
template <typename T, int PS, int DD>
constexpr int pages_per_block() {
    return (PS && DD) ? (kBlockKeyBytes / (PS * DD * (int)sizeof(T)) > 0 ? kBlockKeyBytes / (PS * DD * (int)sizeof(T)) : 1) : 4;
}
constexpr int kBatch = 4;             // units per thread with loads in flight together
constexpr int kMaxHalf = 128;         // head_dim / 2
constexpr double kTwoPiHi = 6.283185307179586232;      // 2*pi rounded to fp64
constexpr double kTwoPiLo = 2.4492935982947064e-16;    // 2*pi - kTwoPiHi

// 8 consecutive elements of a key row: raw load/store and widening to fp32.
template <typename T>
struct Elem;
template <>
struct Elem<float> {
    struct Raw { f32x4 lo, hi; };
    __device__ static Raw load(const float *p) {
        return Raw{__builtin_nontemporal_load((const f32x4 *)p), __builtin_nontemporal_load((const f32x4 *)(p + 4))};
    }
    __device__ static void widen(const Raw &r, float *x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = r.lo[j];
            x[4 + j] = r.hi[j];
        }
    }
    __device__ static void store(float *p, const float *x) {
        __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, (f32x4 *)p);
        __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, (f32x4 *)(p + 4));
    }
};
template <>
struct Elem<bf16> {
    typedef u32x4 Raw;
    __device__ static Raw load(const bf16 *p) { return __builtin_nontemporal_load((const u32x4 *)p); }
    __device__ static void widen(const Raw &v, float *x) {
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
        __builtin_nontemporal_store(v, (u32x4 *)p);
    }
};

// PS / DD = 0: page size / head dim taken from the arguments (any legal value);
// otherwise compile-time, so the index arithmetic is shifts and masks.
template <typename T, int PS, int DD, int kPagesPerBlock = pages_per_block<T, PS, DD>()>
__global__ __launch_bounds__(kThreads) void relocate_kernel(const T *__restrict__ k_in, T *k_out, int ps_arg,
                                                            int D_arg, int64_t n_phys, int n,
                                                            const int4 *__restrict__ list, double log2_theta) {
    const int ps = PS ? PS : ps_arg;
    const int D = DD ? DD : D_arg;
    __shared__ int4 sL[kPagesPerBlock];
    __shared__ int sSlot[kPagesPerBlock];               // page -> its delta's table
    __shared__ int sDelta[kPagesPerBlock];
    __shared__ int sNd;
    __shared__ float2 sCS[kPagesPerBlock][kMaxHalf];   // (cos, sin) of delta * w_i per distinct delta
    const int units_per_row = D / 16;            // a unit = 8 pairs of one key row
    const int ig = threadIdx.x % units_per_row;  // fixed for the launch (kThreads % units_per_row == 0)
    const int units_per_page = ps * units_per_row;
    const int half = D / 2;

    // this workgroup's run of list items, sanitised (a page outside the pool holds no token)
    const int64_t first = (int64_t)blockIdx.x * kPagesPerBlock;
    const int pages = (int)min<int64_t>(kPagesPerBlock, n - first);
    if (threadIdx.x < pages) {
        int4 e = list[first + threadIdx.x];   // {phys, delta, n_valid, reserved}
        if (e.x < 0 || e.x >= n_phys) e.z = 0;
        e.z = min(e.z, ps);
        sL[threadIdx.x] = e;
    }
    __syncthreads();

    const int total = pages * units_per_page;
    typename Elem<T>::Raw ra[kBatch], rb[kBatch];
    int64_t base[kBatch];
    int pl[kBatch];
    bool ok[kBatch];
    auto issue = [&](int u0) {
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int u = u0 + k * kThreads;
            ok[k] = false;
            base[k] = 0;
            pl[k] = 0;
            if (u < total) {
                pl[k] = u / units_per_page;
                const int4 e = sL[pl[k]];
                const int row = (u % units_per_page) / units_per_row;
                ok[k] = row < e.z;
                base[k] = ((int64_t)e.x * ps + row) * D + 8 * ig;
            }
            if (ok[k]) {
                ra[k] = Elem<T>::load(k_in + base[k]);
                rb[k] = Elem<T>::load(k_in + base[k] + half);
            }
        }
    };
    issue(threadIdx.x);   // the first loads fly while the angle tables are built

    if (threadIdx.x == 0) {   // distinct deltas of the run
        int nd = 0;
        for (int pg = 0; pg < pages; ++pg) {
            int j = 0;
            while (j < nd && sDelta[j] != sL[pg].y) ++j;
            if (j == nd) sDelta[nd++] = sL[pg].y;
            sSlot[pg] = j;
        }
        sNd = nd;
    }
    __syncthreads();
    // (cos, sin) of delta * w_i, w_i = theta^(-2i/D): angle formed and reduced mod 2*pi in fp64
    for (int idx = threadIdx.x; idx < sNd * half; idx += kThreads) {
        const int sl = idx / half, i = idx % half;
        const double w = exp2(-(2.0 * i / D) * log2_theta);
        const double ang = (double)sDelta[sl] * w;
        const double q = rint(ang * (1.0 / kTwoPiHi));
        const double r = fma(-q, kTwoPiLo, fma(-q, kTwoPiHi, ang));   // |r| <~ pi
        double sd, cd;
        sincos(r, &sd, &cd);
        sCS[sl][i] = make_float2((float)cd, (float)sd);
    }
    __syncthreads();

    for (int u0 = threadIdx.x; u0 < total; u0 += kThreads * kBatch) {
        if (u0 != (int)threadIdx.x) issue(u0);
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (!ok[k]) continue;
            const float2 *cs = &sCS[sSlot[pl[k]]][8 * ig];
            float a[8], b[8], ya[8], yb[8];
            Elem<T>::widen(ra[k], a);
            Elem<T>::widen(rb[k], b);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float2 t = cs[j];
                ya[j] = fmaf(a[j], t.x, -(b[j] * t.y));
                yb[j] = fmaf(b[j], t.x, a[j] * t.y);
            }
            Elem<T>::store(k_out + base[k], ya);
            Elem<T>::store(k_out + base[k] + half, yb);
        }
    }
}

}  // namespace

int launch_relocate(const void *k_in, void *k_out, int dtype, int page_size, int head_dim, int64_t n_phys, int n,
                    const sp_reloc *d_list, double theta, hipStream_t stream) {
    if (kThreads % (head_dim / 16) != 0)
        return fail(SP_EUNSUPPORTED, "rope_relocate head_dim %d (a power of two, 16..256)", head_dim);
    const double l2t = log2(theta);
    const dim3 block(kThreads);
#define SP_RELOC(T, PSV, DV)                                                                                   \
    do {                                                                                                       \
        constexpr int ppb = pages_per_block<T, PSV, DV>();                                                    \
        const dim3 grid((unsigned)((n + ppb - 1) / ppb));                                                      \
        hipLaunchKernelGGL((relocate_kernel<T, PSV, DV>), grid, block, 0, stream, (const T *)k_in, (T *)k_out, \
                           page_size, head_dim, n_phys, n, (const int4 *)d_list, l2t);                        \
    } while (0)
#define SP_RELOC_SHAPES(T)                                                                   \
    if (head_dim == 128 && page_size == 16) SP_RELOC(T, 16, 128);                           \
    else if (head_dim == 128 && page_size == 32) SP_RELOC(T, 32, 128);                      \
    else if (head_dim == 128 && page_size == 64) SP_RELOC(T, 64, 128);                      \
    else if (head_dim == 64 && page_size == 16) SP_RELOC(T, 16, 64);                        \
    else if (head_dim == 64 && page_size == 32) SP_RELOC(T, 32, 64);                        \
    else SP_RELOC(T, 0, 0);
    if (dtype == SP_F32) {
        SP_RELOC_SHAPES(float)
    } else {
        SP_RELOC_SHAPES(bf16)
    }
#undef SP_RELOC_SHAPES
#undef SP_RELOC
    return check_hip(hipGetLastError(), "rope_relocate launch");
}

}  // namespace sp
