// segpaged_decode_static: segpaged_decode for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts that
// forbid hipMalloc).  Its scratch (launch plan, split partials) lives in one
// file-scope device array per GPU instead of a caller workspace; the kernels
// are those of segpaged_decode.
#include <cstring>
#include <mutex>

#include "internal.hpp"

namespace sp {
constexpr size_t kStaticScratchBytes = size_t(16) << 20;   // SP_STATIC_SCRATCH_BYTES
static_assert(kStaticScratchBytes == SP_STATIC_SCRATCH_BYTES, "header and library disagree");
constexpr int kMaxDevices = 64;
}  // namespace sp

// The array's name is a host-side stand-in in host code: kernels receive the
// device address taken from hipGetSymbolAddress, never `scratch` itself.
static __device__ __align__(256) unsigned char scratch[sp::kStaticScratchBytes];

namespace {

std::mutex g_mu;
void *g_scratch[sp::kMaxDevices] = {};

// Device address of this GPU's copy of `scratch`, looked up once per device
// (with that device current) and kept.
int scratch_of_current_device(void **out) {
    int dev = -1;
    int rc = sp::check_hip(hipGetDevice(&dev), "hipGetDevice");
    if (rc) return rc;
    if (dev < 0 || dev >= sp::kMaxDevices) return sp::fail(SP_EUNSUPPORTED, "device %d (at most %d)", dev,
                                                           sp::kMaxDevices);
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        rc = sp::check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (rc) return rc;
        if (!p || ((uintptr_t)p) % 256) return sp::fail(SP_EHIP, "static scratch at %p is not 256-byte aligned", p);
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SP_OK;
}

}  // namespace

extern "C" int segpaged_decode_static(int dtype, int head_dim, int page_size, int group, int n_seq, int n_slot,
                                      const int32_t *h_row_ptr, const int32_t *d_q_pos, const int32_t *d_cls,
                                      const int32_t *d_window, const int32_t *d_row_ptr, const sp_entry *d_entries,
                                      const void *q, const void *k_pool, const void *v_pool, int64_t n_phys,
                                      float softmax_scale, void *out, float *lse, void *stream) {
    sp::clear_error();
    // the size check comes first and touches no GPU state
    sp::Plan p;
    int rc = sp::make_plan(SP_WS_DECODE, dtype, head_dim, page_size, group, n_seq, n_slot, nullptr, h_row_ptr, &p);
    if (rc) return rc;
    if (p.bytes > sp::kStaticScratchBytes)
        return sp::fail(SP_EWORKSPACE,
                        "segpaged_decode_static: this call needs %zu bytes of scratch, the static scratch holds "
                        "%zu (use segpaged_decode with a workspace)",
                        p.bytes, sp::kStaticScratchBytes);
    void *ws = nullptr;
    rc = scratch_of_current_device(&ws);
    if (rc) return rc;
    return segpaged_decode(dtype, head_dim, page_size, group, n_seq, n_slot, h_row_ptr, d_q_pos, d_cls, d_window,
                           d_row_ptr, d_entries, q, k_pool, v_pool, n_phys, softmax_scale, out, lse, ws,
                           sp::kStaticScratchBytes, stream);
}
