// Internal declarations shared by the host runtime and the kernels of libsegpaged.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "segpaged.h"

namespace sp {

// ---------------------------------------------------------------- errors
// Records a printf-style message for segpaged_last_error() and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int check_hip(hipError_t e, const char *what);

// ---------------------------------------------------------------- launch plan
// Tile shapes of the bf16 MFMA kernels.
constexpr int kPrefillRowsPerWave = 32;   // query rows (token x head) per wave
constexpr int kPrefillKeysPerTile = 64;   // keys staged in LDS per iteration
constexpr int kDecodeKeysPerBlock = 32;   // keys one wave consumes per step
constexpr int kDecodeWaves = 8;

// Split planning: the prefill splits long rows so that their pieces fill the
// 256 CUs of the chip once; decode aims at about one streaming split per CU.
// Every split still streams at least kMinSplitKeysPrefill / kMinSplitKeysDecode keys.
constexpr int kPlanCUs = 256;
constexpr int kPrefillSetupTiles = 6;      // fixed cost of a prefill item (set-up, result, hand-off), in 64-key tiles
constexpr int kPrefillEdgeTiles = 3;       // extra cost of a row end inside an item (bounds, fix-ups), in tiles
constexpr double kMergeTiles = 1.5;        // merge pass per split prefill item, in 64-key tiles of one CU
constexpr int kTargetDecodeItems = 384;
constexpr int kDecodeWgPerCU = 1;          // decode workgroups (of kDecodeWaves waves) per CU the plan aims for
constexpr int kMinSplitKeysPrefill = 64;
constexpr int kMinSplitKeysDecode = 512;
constexpr int kMaxSplits = 1024;
constexpr int kDecodeMaxChunk = 512;       // pages of one decode split (its entries are staged in LDS)
constexpr int kDeepMergeSplits = 32;       // prefill rows split this many ways are merged a row per workgroup

// Number of kv splits and work items of one row; identical on host and device.
__host__ __device__ inline void row_items(int n_entries, int n_qtiles, int chunk_pages,
                                          int *nsplit, int *items) {
    int ns = 1;
    if (n_entries > chunk_pages) {
        ns = (n_entries + chunk_pages - 1) / chunk_pages;
        if (ns > kMaxSplits) ns = kMaxSplits;
    }
    *nsplit = ns;
    *items = ns * n_qtiles;
}

struct Plan {
    int kind = 0;            // SP_WS_PREFILL / SP_WS_DECODE
    int n_rows = 0;
    int waves = 4;           // waves per prefill workgroup
    int rows_per_tile = 0;   // query rows of one work item (prefill BM, decode group)
    int tok_per_tile = 1;    // query tokens of one prefill work item
    int chunk_pages = 0;     // pages per kv split (INT32_MAX = no split)
    int64_t n_items = 0;     // work items (= workgroups of the attention kernel)
    int64_t n_parts = 0;     // work items whose result is a partial to merge
    int merge_rows = 0;      // prefill: most query rows one split item merges (rows split fewer than kDeepMergeSplits ways)
    int merge_rows_deep = 0; // the same for rows split kDeepMergeSplits ways or more
    // Work items are numbered long-first: the items of split rows (row order),
    // then those of unsplit rows.  item_ptr[r] / item_ptr2[r] = first item of
    // row r in the first / second range (zero-length for rows of the other).
    size_t off_item_ptr = 0, off_item_ptr2 = 0, off_part_ptr = 0, off_nsplit = 0, off_zero = 0, off_part_o = 0, off_part_lse = 0;
    size_t bytes = 0;        // workspace bytes
};

int make_plan(int kind, int dtype, int head_dim, int page_size, int group, int n_seq, int n_slot,
              const int32_t *h_tok_ptr, const int32_t *h_row_ptr, Plan *plan);

// ---------------------------------------------------------------- launchers (device code)
int launch_relocate(const void *k_in, void *k_out, int dtype, int page_size, int head_dim,
                    int64_t n_phys, int n, const sp_reloc *d_list, double theta, hipStream_t s);

struct AttnArgs {
    int dtype, head_dim, page_size, group, n_seq, n_slot;
    const int32_t *h_row_ptr;   // host copy of d_row_ptr (launch planning)
    const int32_t *h_tok_ptr;   // host copy of d_tok_ptr (prefill launch planning); decode: nullptr
    const int32_t *d_tok_ptr;   // prefill: [n_seq+1]; decode: nullptr
    const int32_t *d_q_pos;     // prefill: first query position per seq; decode: query position
    const int32_t *d_cls, *d_window, *d_row_ptr;
    const sp_entry *d_entries;
    const void *q, *k_pool, *v_pool;
    int64_t n_phys;
    float scale;
    void *out;
    float *lse;
    void *ws;
};

int launch_prefill(const AttnArgs &a, const Plan &p, int64_t n_tok, hipStream_t s);
int launch_decode(const AttnArgs &a, const Plan &p, hipStream_t s);
// Attention importance (segpaged_token_importance) and token selection.
struct ImportancePlan {
    int n_rows = 0, tpt = 0;
    int64_t n_items = 0, n_part = 0, n_red = 0, e_max = 0;
    size_t off_item_ptr = 0, off_part_ptr = 0, off_red_ptr = 0, off_part = 0;
    size_t bytes = 0;
};
struct ImportanceArgs {
    int dtype, head_dim, page_size, group, n_seq, n_slot;
    const int32_t *h_row_ptr, *h_tok_ptr;
    const int32_t *d_tok_ptr, *d_q_pos0, *d_cls, *d_window, *d_row_ptr, *d_pos_ptr;
    const sp_entry *d_entries;
    const void *q, *k_pool;
    int64_t n_phys;
    float scale;
    const float *lse;
    int64_t n_pos;
    float *imp;
    void *ws;
};
int plan_importance(int dtype, int head_dim, int page_size, int group, int n_seq, int n_slot,
                    const int32_t *h_tok_ptr, const int32_t *h_row_ptr, ImportancePlan *out);
int launch_importance(const ImportanceArgs &a, const ImportancePlan &p, hipStream_t s);
struct SelectArgs {
    int n_layers, slots_per_layer, n_seq, max_len;
    const int32_t *d_pos_ptr, *d_sel_ptr;
    int64_t n_pos, sel_total;
    const float *imp;
    float *score;
    int32_t *sel;
};
int launch_select(const SelectArgs &a, hipStream_t s);

int launch_page_copy(bool unpack, const void *d_entries, int64_t n, const void *src_k, const void *src_v,
                     void *dst_k, void *dst_v, int64_t n_phys, int page_bytes, hipStream_t s);

}  // namespace sp
