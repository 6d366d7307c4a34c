// Per-head visible-page pack / unpack: the pages a set of table entries lists,
// gathered in entry order into contiguous K and V buffers, or scattered back.
//
// Follows the RedKnot product profile, section 3, and the is96.com commentary's
// paragraphs on the per-head page table: a head reads only the pages its table
// lists, so when prefill and decode run on different machines only those pages
// move.  This is the single-GPU part: an HBM-bound copy of whole pages (K
// [page_size][head_dim], V [head_dim][page_size], the pools' layouts), 16 bytes
// per lane, consecutive lanes on consecutive bytes of a page, with a run of
// loads in flight per thread before any store.
#include "device_common.hpp"

namespace sp {
namespace {

constexpr int kPackThreads = 256;
constexpr int kPackPages = 2;    // table entries per workgroup (1, 2 and 4 with 4-16 loads measured within 1 %; 4 with 8: 8 % slower)
constexpr int kPackBatch = 4;    // 16-byte chunks per thread in flight together

// UNPACK = false: dst_k/dst_v are the packed buffers, src the pools;
// UNPACK = true: src the packed buffers, dst the pools.  An entry whose page
// id is outside [0, n_phys) packs as zeros and unpacks to nothing.
template <bool UNPACK>
__global__ __launch_bounds__(kPackThreads) void page_copy_kernel(const int4 *__restrict__ entries, int64_t n,
                                                                 const char *src_k, const char *src_v, char *dst_k,
                                                                 char *dst_v, int64_t n_phys, int page_bytes) {
    __shared__ int64_t sPhys[kPackPages];
    const int64_t e0 = (int64_t)blockIdx.x * kPackPages;
    if (threadIdx.x < kPackPages) {
        const int64_t e = e0 + threadIdx.x;
        int64_t p = -1;
        if (e < n) {
            p = entries[e].x;
            if (p < 0 || p >= n_phys) p = -1;
        }
        sPhys[threadIdx.x] = p;
    }
    __syncthreads();
    const int chunks = page_bytes / 16;                     // per page and tensor
    const int total = kPackPages * 2 * chunks;
    for (int c0 = threadIdx.x; c0 < total; c0 += kPackThreads * kPackBatch) {
        u32x4 val[kPackBatch];
        int64_t dst[kPackBatch];
        bool tv[kPackBatch], go[kPackBatch];
#pragma unroll
        for (int k = 0; k < kPackBatch; ++k) {
            const int c = c0 + k * kPackThreads;
            const int pg = c / (2 * chunks), t = (c / chunks) & 1, off = c % chunks;
            const int64_t e = e0 + pg;
            const int64_t p = pg < kPackPages ? sPhys[pg] : -1;
            go[k] = c < total && e < n && (!UNPACK || p >= 0);
            tv[k] = t;
            val[k] = u32x4{0, 0, 0, 0};
            const int64_t s_off = (UNPACK ? e : p) * page_bytes + 16 * off;
            dst[k] = (UNPACK ? p : e) * page_bytes + 16 * off;
            if (go[k] && (UNPACK || p >= 0))
                val[k] = __builtin_nontemporal_load((const u32x4 *)((t ? src_v : src_k) + s_off));
        }
#pragma unroll
        for (int k = 0; k < kPackBatch; ++k)
            if (go[k]) __builtin_nontemporal_store(val[k], (u32x4 *)((tv[k] ? dst_v : dst_k) + dst[k]));
    }
}

}  // namespace

int launch_page_copy(bool unpack, const void *d_entries, int64_t n, const void *src_k, const void *src_v, void *dst_k,
                     void *dst_v, int64_t n_phys, int page_bytes, hipStream_t stream) {
    if (n == 0) return SP_OK;
    const int64_t blocks = (n + kPackPages - 1) / kPackPages;
    if (blocks > INT32_MAX) return fail(SP_EINVAL, "too many entries");
    const dim3 grid((unsigned)blocks), block(kPackThreads);
    if (unpack)
        hipLaunchKernelGGL((page_copy_kernel<true>), grid, block, 0, stream, (const int4 *)d_entries, n,
                           (const char *)src_k, (const char *)src_v, (char *)dst_k, (char *)dst_v, n_phys, page_bytes);
    else
        hipLaunchKernelGGL((page_copy_kernel<false>), grid, block, 0, stream, (const int4 *)d_entries, n,
                           (const char *)src_k, (const char *)src_v, (char *)dst_k, (char *)dst_v, n_phys, page_bytes);
    return check_hip(hipGetLastError(), "page copy launch");
}

}  // namespace sp
