// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "internal.hpp"

namespace sp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kPosInvalid = 0x7fffffff;   // position of a key slot that holds no token

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round-to-nearest-even fp32 -> bf16 (lowers to v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 f32_to_bf16(float x) { return (bf16)x; }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ bf16x8 u4_as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Zeroes the bf16 elements i >= keep of a 16-byte chunk of 8 bf16.
__device__ __forceinline__ u32x4 keep_first_bf16(u32x4 v, int keep) {
    if (keep >= 8) return v;
    u32x4 r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t x = v[w];
        const int e0 = 2 * w, e1 = 2 * w + 1;
        if (e0 >= keep) x &= 0xffff0000u;
        if (e1 >= keep) x &= 0x0000ffffu;
        r[w] = x;
    }
    return r;
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float xor_lane(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Index of the work item's row: the largest r with item_ptr[r] <= b
// (item_ptr ascending, item_ptr[n_rows] > b).  Wave-parallel 64-ary search.
__device__ __forceinline__ int find_row(const int32_t *item_ptr, int n_rows, int b) {
    const int lane = threadIdx.x & 63;
    int lo = 0, hi = n_rows;   // answer in [lo, hi)
    while (hi - lo > 1) {
        const int span = hi - lo;
        const int step = (span + 63) / 64;
        const int idx = lo + lane * step;
        const bool le = idx < hi && item_ptr[idx] <= b;
        const uint64_t m = __ballot(le);
        // lanes 0..k-1 satisfy le (prefix); the answer lies in [lo + (k-1)*step, lo + k*step)
        const int k = __popcll(m);
        const int nlo = lo + (k - 1) * step;
        const int nhi = min(hi, lo + k * step);
        lo = nlo;
        hi = nhi;
        if (step == 1) break;
    }
    return lo;
}

// Launch plan of a call with few rows, built on the host and passed by value
// (kernel arguments), so such calls need no plan kernel: same meaning as the
// workspace arrays of the same names (see item_of).
constexpr int kInlineRows = 192;
struct InlinePlan {
    int32_t item_ptr[kInlineRows + 1], item_ptr2[kInlineRows + 1], part_ptr[kInlineRows + 1];
    int32_t nsplit[kInlineRows];
};

// The prefill's inline plan: the same arrays for up to kPrefillInlineRows
// rows, plus the call's row_ptr and tok_ptr, so that an item's first reads
// of them are kernel arguments too (the struct stays under 4 KB of kernel
// arguments with the prefill's parameters).
constexpr int kPrefillInlineRows = 128;
struct PrefillInlinePlan {
    int32_t item_ptr[kPrefillInlineRows + 1], item_ptr2[kPrefillInlineRows + 1], part_ptr[kPrefillInlineRows + 1];
    int32_t nsplit[kPrefillInlineRows];
    int32_t row_ptr[kPrefillInlineRows + 1], tok_ptr[kPrefillInlineRows + 1];
};

// Host: fills L's item arrays for n_rows rows (at most the struct's capacity),
// with the integer formulas of the plan kernel.  h_tok_ptr: query tokens per
// sequence (prefill; its q-tiles of tpt tokens), or nullptr (decode: one
// q-tile per row).
template <class Plan_>
inline void fill_inline_plan(int n_rows, int n_seq, const int32_t *h_row_ptr, const int32_t *h_tok_ptr, int tpt,
                             int chunk_pages, Plan_ *L) {
    int32_t cl = 0, cs = 0, cp = 0;
    for (int r = 0; r < n_rows; ++r) {
        int nq = 1;
        if (h_tok_ptr) {
            const int q = r % n_seq;
            nq = (h_tok_ptr[q + 1] - h_tok_ptr[q] + tpt - 1) / tpt;
        }
        int ns, it;
        row_items(h_row_ptr[r + 1] - h_row_ptr[r], nq, chunk_pages, &ns, &it);
        L->nsplit[r] = ns;
        L->item_ptr[r] = cl;
        L->item_ptr2[r] = cs;
        L->part_ptr[r] = cp;
        if (ns > 1) {
            cl += it;
            cp += it;
        } else {
            cs += it;
        }
    }
    L->item_ptr[n_rows] = cl;
    L->item_ptr2[n_rows] = cs;
    L->part_ptr[n_rows] = cp;
}

// Row and index within the row of work item b.  Items are numbered long-first:
// [0, item_ptr[n_rows]) are the items of split rows (first item of row r at
// item_ptr[r]), the rest those of unsplit rows (at item_ptr[n_rows] + item_ptr2[r]).
__device__ __forceinline__ void item_of(const int32_t *item_ptr, const int32_t *item_ptr2, int n_rows, int b,
                                        int *row, int *local) {
    const int n_long = item_ptr[n_rows];
    const int32_t *ip = b < n_long ? item_ptr : item_ptr2;
    const int bb = b < n_long ? b : b - n_long;
    const int r = find_row(ip, n_rows, bb);
    *row = r;
    *local = bb - ip[r];
}

// First index e in [a, b) whose key(e) > x, keys ascending in e; b if none.
template <class Key>
__device__ __forceinline__ int first_greater(int a, int b, int x, Key key) {
    const int lane = threadIdx.x & 63;
    while (b - a > 0) {
        const int span = b - a;
        const int step = (span + 63) / 64;
        const int idx = a + lane * step;
        const bool le = idx < b && key(idx) <= x;
        const int k = __popcll(__ballot(le));     // lanes 0..k-1 have key <= x
        if (step == 1) return a + k;
        if (k == 0) return a;
        a = a + (k - 1) * step + 1;               // key(a-1) <= x
        b = min(b, a - 1 + step);
    }
    return a;
}

// Entry range [lo, hi) of a table row [e_beg, e_end) that a query span sees:
// hi = first entry whose first position exceeds p_hi; lo = e_beg, or for a
// local head the first entry whose last position exceeds `bound` (= p_lo - W).
// Entries are in ascending position, so both are prefix counts.  The common
// case (everything of interest within the last 64 entries) takes one round of
// loads; otherwise it falls back to the 64-ary search.
__device__ __forceinline__ void visible_range(const int4 *__restrict__ E, int e_beg, int e_end, int p_hi,
                                              bool is_local, int bound, int *lo_out, int *hi_out) {
    const int lane = threadIdx.x & 63;
    const int a = max(e_beg, e_end - 64);
    const int idx = a + lane;
    const bool valid = idx < e_end;
    int first = 0, last = 0;
    if (valid) {
        const int4 en = E[idx];
        first = en.y;
        last = en.y + en.z - 1;
    }
    const int first_a = __shfl(first, 0, 64), last_a = __shfl(last, 0, 64);
    int hi;
    if (a == e_beg || first_a <= p_hi)
        hi = a + __popcll(__ballot(valid && first <= p_hi));
    else
        hi = first_greater(e_beg, a, p_hi, [&](int e) { return E[e].y; });
    int lo = e_beg;
    if (is_local) {
        if (hi <= a) lo = first_greater(e_beg, hi, bound, [&](int e) { return E[e].y + E[e].z - 1; });
        else if (a == e_beg || last_a <= bound)
            lo = min(hi, a + __popcll(__ballot(valid && last <= bound)));
        else
            lo = first_greater(e_beg, a + 1, bound, [&](int e) { return E[e].y + E[e].z - 1; });
    }
    *lo_out = __builtin_amdgcn_readfirstlane(lo);
    *hi_out = __builtin_amdgcn_readfirstlane(hi);
}

// One 16-byte global->LDS load per lane through a buffer resource (gfx950
// buffer_load_dwordx4 ... lds): lane l reads bytes [voff_l, voff_l + 16) of the
// range [base, base + bytes) and the wave writes LDS bytes [lds, lds + 1024)
// (lds = LDS byte address), lane l at lds + 16 l.  base, bytes and lds must be
// wave-uniform; a lane whose voff_l + 16 passes `bytes` gets zeros (the buffer
// range check).
//
// Two properties matter to the kernels that keep several tiles in flight:
//  * The LDS destination reaches the builtin as a bare byte address that
//    the compiler cannot trace to a variable, so it inserts no waits for the
//    load before later LDS reads: the caller must wait (s_waitcnt vmcnt)
//    before reading what it writes.
//  * It is a buffer (MUBUF) instruction, not a FLAT one.  While a FLAT-encoded
//    load that writes LDS (global_load_lds) is outstanding, the compiler
//    treats the LDS counter as unordered and turns every wait for an LDS read
//    into lgkmcnt(0), which drains the operand reads queued ahead of the
//    matrix instructions; with the buffer form those waits stay exact.
// The builtins exist only for the device target, so the host pass (which must
// still emit the kernel's launch stub) sees a no-op.
#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ void lds_dma16_buf(const void *base, uint32_t bytes, uint32_t voff, uint32_t lds) {
    uint32_t a = __builtin_amdgcn_readfirstlane(lds);   // wave-uniform
    asm volatile("" : "+s"(a));
    // word 3 of the resource: 32-bit data format, the raw-buffer setting of the gfx9 family
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(uintptr_t)a, 16, voff, 0, 0, 0);
}
#else
__device__ __forceinline__ void lds_dma16_buf(const void *, uint32_t, uint32_t, uint32_t) {}
#endif

// Host: the epoch of a call that counts in an epoch-tagged workspace counter
// (ticket_issue / ticket_resolve); never 0, which is what a cleared counter holds.
inline uint32_t next_epoch() {
    static std::atomic<uint32_t> epochs{0};
    uint32_t e = epochs.fetch_add(1) + 1;
    if (e == 0) e = epochs.fetch_add(1) + 1;
    return e;
}

// Work tickets of a persistent kernel from a 64-bit counter in the workspace
// whose high half is the epoch of the call counting in it (a host counter,
// never 0), so no call needs the counter cleared first.  A ticket is issued
// early (ticket_issue: the counter's value before this increment) and
// resolved when it is needed, so that nothing waits for the atomic before
// then.  A value from another epoch means no ticket of this call was handed
// out before: the first such wave installs {epoch, 1} and takes count 0, the
// others then take a count again.  Every failed exchange means another wave
// changed the counter since it was read, and before the install only each
// wave's one increment can do so, so the loop ends.  (Epochs repeat only
// after 2^32 - 1 calls; a workspace would have to sit unused for exactly
// that many calls of the process for its counter to be mistaken as current.)
__device__ __forceinline__ unsigned long long ticket_issue(unsigned long long *ctr) {
    typedef __attribute__((address_space(1))) unsigned long gul;
    return __builtin_amdgcn_atomic_inc64((volatile gul *)(gul *)ctr, ~0ull, __ATOMIC_RELAXED, "agent");
}
__device__ __forceinline__ int ticket_resolve(unsigned long long *ctr, uint32_t epoch, unsigned long long v) {
    if ((uint32_t)(v >> 32) == epoch) return (int)(uint32_t)v;
    const unsigned long long first = ((unsigned long long)epoch << 32) + 1;
    unsigned long long cur = v + 1;      // what this wave's increment left, if nothing moved it since
    for (;;) {
        const unsigned long long seen = atomicCAS(ctr, cur, first);
        if (seen == cur) return 0;
        if ((uint32_t)(seen >> 32) == epoch) return (int)(uint32_t)ticket_issue(ctr);
        cur = seen;
    }
}

}  // namespace sp
