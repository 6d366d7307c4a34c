/*
 * segpaged.h - C ABI of libsegpaged.so: SegPagedAttention with head-aware KV
 * reuse on AMD Instinct MI355X (gfx950).
 *
 * What the calls compute (sources named by page title and section):
 *   - RedKnot product profile (tokenfly.club), section 3: each (layer, head) is
 *     classed global, local, retrieval or dense; reusable segments' keys are
 *     cached offline and re-aligned with rotary position encoding when reused;
 *     SegPagedAttention gives every head its own page table over segmented KV
 *     storage so each class reads only its own visible window, on the mask-free
 *     attention path.
 *   - is96.com commentary on the RedKnot paper: the RoPE paragraphs (a cached key
 *     is rotated back by its offline angle and forward by its online angle) and
 *     the SegPagedAttention paragraphs (each head owns pages holding only its
 *     own KV and a table listing the pages it reads).
 *   - "PagedAttention & RadixAttention" (wiki.gxlh.xyz), "The Solution:
 *     Fixed-size blocks": fixed-size blocks, logical->physical block tables, a
 *     global free pool, the last block filled before a new one is claimed.
 *
 * Vocabulary
 *   slot     one (layer, KV head).  It owns its page chains, its class and its
 *            window; its `group` query heads share them.  A call may cover any
 *            number of slots (one layer, or several layers at once).
 *   row      one (slot, sequence) pair, row = slot * n_seq + seq.
 *   page     page_size consecutive token positions of one slot and sequence.
 *   position an online absolute token position (int32, >= 0).
 *
 * Visibility of a query at position p (only tokens with position <= p exist
 * for it): global and dense see every token; local(W) sees tokens with
 * p - W < position; retrieval sees the tokens on its listed segment pages plus
 * every new token.  No mask tensor exists anywhere: the kernels derive bounds
 * from positions.
 *
 * Memory layouts (all row-major, little-endian, no padding between rows)
 *   K pool   [n_phys][page_size][head_dim]   token-major inside a page
 *   V pool   [n_phys][head_dim][page_size]   dim-major inside a page: a run of
 *            consecutive keys at one dim is contiguous, the operand shape the
 *            P.V contraction (over keys) consumes directly.
 *   Q / out  [n_tok][n_slot * group][head_dim]  token-major; query head
 *            h = slot * group + g belongs to slot h / group.
 *   lse      [n_tok][n_slot * group] fp32, natural-log log-sum-exp of the
 *            scaled scores of each (token, head).
 *   dtype    SP_F32 (fp32 in, fp32 arithmetic, fp32 out) or SP_BF16 (bf16 in,
 *            fp32 accumulation, bf16 out rounded to nearest even).
 *
 * Conventions
 *   - Every call returns an int status (SP_OK = 0, negative on error) and
 *     validates all arguments it can see before touching the GPU; no C++
 *     exception crosses the ABI.  On error nothing was enqueued and outputs are
 *     unspecified.
 *   - Ownership: the caller owns every buffer.  The library allocates no host or
 *     device memory in the device calls and keeps no state beyond a call
 *     counter (the epoch that tags the work counters in a workspace) and, for
 *     segpaged_decode_static, each GPU's scratch address; calls are
 *     thread-safe (calls that share a workspace must not overlap).
 *   - Device calls enqueue on `stream` (a hipStream_t; NULL = the null stream)
 *     and return without waiting.  Kernel faults surface at the caller's next
 *     synchronisation.  Physical page ids read from device tables are checked
 *     against n_phys and out-of-range pages are treated as empty.
 *   - Pointers named h_* are host memory, d_* (and the tensors) device memory.
 */
#ifndef SEGPAGED_H
#define SEGPAGED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define SP_OK            0
#define SP_EINVAL       -1   /* bad argument (message via segpaged_last_error) */
#define SP_ENOMEM       -2   /* free list shorter than the pages needed        */
#define SP_EHIP         -3   /* a HIP runtime call or launch failed             */
#define SP_EUNSUPPORTED -4   /* valid but not implemented (dtype/dim/page size) */
#define SP_EWORKSPACE   -5   /* workspace smaller than segpaged_workspace_bytes */

/* head classes */
#define SP_GLOBAL    0
#define SP_LOCAL     1
#define SP_RETRIEVAL 2
#define SP_DENSE     3

/* element types */
#define SP_F32  0
#define SP_BF16 1

/* workspace kinds */
#define SP_WS_PREFILL    0
#define SP_WS_DECODE     1
#define SP_WS_IMPORTANCE 2

/* One reused segment of a sequence: len tokens placed at online positions
 * [online_base, online_base + len), whose cached keys were rotated at
 * [offline_base, offline_base + len).  offline_base may be negative. */
typedef struct { int32_t len, online_base, offline_base; } sp_segment;

/* One page-table entry: physical page, position of its first token, number of
 * its tokens that exist at the call (1..page_size).  16 bytes, host and device. */
typedef struct { int32_t phys, pos_start, n_valid, reserved; } sp_entry;

/* One relocation item: rotate the first n_valid keys of page `phys` by
 * `delta` = online_base - offline_base positions.  16 bytes. */
typedef struct { int32_t phys, delta, n_valid, reserved; } sp_reloc;

/*
 * segpaged_build_tables - segment/page allocation and per-head page tables
 * (host only, pure, deterministic).
 *
 * Defines: the per-head page tables over segmented paged storage of the is96.com
 * SegPagedAttention paragraphs and the product profile's section 3, with
 * block-table allocation from a free pool as in the PagedAttention page's
 * fixed-size-block section.
 *
 * Layout of every (slot, seq) chain, allocated in the order
 * slot -> seq -> segment -> page -> new-token pages, each page popped from the
 * front of free_list: each segment starts on a fresh page (its last page may be
 * partial); the n_new[seq] new tokens (prefill chunk + decode tokens) occupy
 * positions [E, E + n_new) with E = end of the last segment (0 without
 * segments), starting on a fresh page.  Segments must be in ascending,
 * non-overlapping online order.
 *
 * Inputs
 *   n_seq, seg_ptr[n_seq+1], segs[seg_ptr[n_seq]]   sequences (CSR of segments)
 *   n_new[n_seq]             new-token capacity of each sequence (>= 1)
 *   q_lo[n_seq], q_hi[n_seq] the positions this call's queries occupy:
 *                            E <= q_lo <= q_hi < E + n_new
 *   n_slot, cls[n_slot], window[n_slot]   class per slot; window >= 1 for local
 *   ret_ptr[n_slot*n_seq+1], ret_pages    CSR per row of listed segment-page
 *                            ordinals (the k-th page among the sequence's
 *                            segment pages), strictly ascending; non-empty only
 *                            for retrieval rows.  Both may be NULL if no slot
 *                            is retrieval.
 *   page_size >= 1; free_list[n_free] distinct non-negative page ids.
 * Outputs (pass all NULL to only get counts; otherwise all non-NULL)
 *   chain_ptr[n_rows+1]      row r's pages are storage[chain_ptr[r] .. chain_ptr[r+1])
 *   storage[counts[0]]       physical page of every logical page, chain order
 *   row_ptr[n_rows+1], entries[counts[1]]   the call's table per row: the pages
 *                            holding >= 1 token visible to >= 1 of the call's
 *                            queries, ascending position
 *   reloc[counts[2]]         every stored segment page, ascending phys
 *   counts[3]                (always written) pages, entries, reloc items
 * Errors: SP_EINVAL (bad layout, class, window, list, position overflow,
 * duplicate or negative page id), SP_ENOMEM (n_free < pages needed; a count
 * query never fails for it).
 */
int segpaged_build_tables(int n_seq, const int32_t *seg_ptr, const sp_segment *segs,
                          const int32_t *n_new, const int32_t *q_lo, const int32_t *q_hi,
                          int n_slot, const int32_t *cls, const int32_t *window,
                          const int32_t *ret_ptr, const int32_t *ret_pages,
                          int page_size, int64_t n_free, const int32_t *free_list,
                          int32_t *chain_ptr, int32_t *storage, int32_t *row_ptr,
                          sp_entry *entries, sp_reloc *reloc, int64_t counts[3]);

/*
 * The layout every host call below shares: sequences, segments, new-token
 * capacity, slots and their classes, retrieval lists, page size - the same
 * arguments, with the same rules, as segpaged_build_tables takes one by one.
 */
typedef struct {
    int n_seq;
    const int32_t *seg_ptr;        /* [n_seq+1] CSR over segs */
    const sp_segment *segs;
    const int32_t *n_new;          /* [n_seq] new-token capacity (prefill chunk + decode tokens) */
    int n_slot;
    const int32_t *cls, *window;   /* [n_slot] */
    const int32_t *ret_ptr, *ret_pages;   /* retrieval lists per row; NULL if no slot is retrieval */
    int page_size;
} sp_layout;

/*
 * segpaged_build_tables_ex - segpaged_build_tables with window-only storage.
 *
 * Defines: the is96.com commentary's deployment paragraph (local heads store
 * only window-sized KV, so one GPU holds several times more sessions) and its
 * SegPagedAttention paragraphs (a head's pages hold only its own KV).
 *
 * keep_from[n_seq] (or NULL for whole chains, which is segpaged_build_tables):
 * every later query of sequence q is at a position >= keep_from[q]
 * (0 <= keep_from[q] <= q_lo[q]).  A head then stores only the chain pages
 * holding a token that some query at a position in [keep_from, E + n_new) can
 * see: a local(W) head the pages whose last position is >= keep_from - W + 1,
 * a retrieval head its listed segment pages and the new-token pages, global
 * and dense heads every page.  Chains keep their logical layout: storage has
 * one id per chain page, -1 for a page that is not stored; allocation pops the
 * free list in the usual order, skipping pages that are not stored.  The
 * relocation list holds only stored segment pages.
 * counts[4]: chain pages (length of storage), table entries, relocation items,
 * pages taken from the free list.  Other arguments as segpaged_build_tables.
 */
int segpaged_build_tables_ex(const sp_layout *layout, const int32_t *q_lo, const int32_t *q_hi,
                             const int32_t *keep_from, int64_t n_free, const int32_t *free_list,
                             int32_t *chain_ptr, int32_t *storage, int32_t *row_ptr,
                             sp_entry *entries, sp_reloc *reloc, int64_t counts[4]);

/*
 * segpaged_tables_from_chains - the tables of a call over existing chains
 * (host): the same table rule as segpaged_build_tables, with the physical ids
 * read from chain_ptr[n_rows+1] / storage (as built, after any releases).
 * Two-call convention: row_ptr and entries both NULL returns the entry count.
 * Errors: SP_EINVAL also when a page the call's queries read is not stored
 * (-1: released, or outside the window the storage was built for).
 */
int segpaged_tables_from_chains(const sp_layout *layout, const int32_t *q_lo, const int32_t *q_hi,
                                const int32_t *chain_ptr, const int32_t *storage,
                                int32_t *row_ptr, sp_entry *entries, int64_t *n_entries);

/*
 * segpaged_release_pages - return pages no later query can read to the free
 * list (host).
 *
 * Defines: the PagedAttention page's walk-through (at the end of a sequence its
 * blocks return to the free pool) together with window-only storage: once the
 * next query of sequence q is at position p_next[q] (>= its first new
 * position), every stored page that no query at a position in
 * [p_next[q], E + n_new) can see is released: a local head's pages that slid
 * out of its window, a retrieval head's unlisted segment pages, and - once
 * p_next[q] >= E + n_new, i.e. the sequence is over - every page of every head.
 * Released ids are written to released[] in row order, then chain order
 * (capacity: chain_ptr[n_rows] ids), their storage entries become -1, and
 * *n_released is set.  Nothing else changes.
 */
int segpaged_release_pages(const sp_layout *layout, const int32_t *p_next, const int32_t *chain_ptr,
                           int32_t *storage, int32_t *released, int64_t *n_released);

/*
 * rope_relocate - move cached segment keys from their offline to their online
 * rotary position (device).
 *
 * Defines: the is96.com commentary's RoPE paragraphs (rotate back by the cached
 * angle, forward by the new one) and the product profile's section 3 (reused
 * segment KV re-aligned by rotary encoding).  Both rotations act on the same
 * coordinate planes, so they compose into one rotation by delta * w_i; the
 * angle delta * w_i is formed and reduced modulo 2*pi in fp64 before the fp32
 * sine/cosine.  Half-split pairing: coordinate i < D/2 pairs with i + D/2,
 * w_i = rope_theta^(-2i/D):
 *   k'[i]       = k[i] cos(delta w_i) - k[i+D/2] sin(delta w_i)
 *   k'[i+D/2]   = k[i+D/2] cos(delta w_i) + k[i] sin(delta w_i)
 *
 * k_in, k_out  K pools [n_phys][page_size][head_dim] of `dtype`; k_out may equal
 *              k_in (in place: each thread writes back exactly the elements
 *              it read, so the result is bit-identical to out of place) but
 *              must not otherwise overlap it.  Only the first n_valid rows of
 *              each listed page are written.
 * d_list[n]    device relocation items (from segpaged_build_tables, which
 *              lists each stored page once).  A page listed twice is read and
 *              written by two workgroups in no fixed order, in place or out of
 *              place, so its result is undefined: list each page once.
 * head_dim     a power of two, 16..256; page_size 1..1024; rope_theta > 0.
 */
int rope_relocate(const void *k_in, void *k_out, int dtype, int page_size, int head_dim,
                  int64_t n_phys, int n, const sp_reloc *d_list, double rope_theta,
                  void *stream);

/*
 * segpaged_workspace_bytes - device workspace a prefill, decode or importance
 * call needs.
 *
 * kinds SP_WS_PREFILL and SP_WS_IMPORTANCE use h_tok_ptr[n_seq+1] (query tokens
 * of each sequence); SP_WS_DECODE ignores it (one query token per sequence).
 * h_row_ptr is the host copy of the call's row_ptr.  Writes *bytes (> 0).
 *
 * The workspace needs no initialisation: a call neither relies on what it
 * holds before the call nor leaves anything a later call relies on (its work
 * counter is tagged with the call's own epoch).  Calls that use the same
 * workspace must not run concurrently (same stream, or ordered by events).
 */
int segpaged_workspace_bytes(int kind, int dtype, int head_dim, int page_size, int group,
                             int n_seq, int n_slot, const int32_t *h_tok_ptr,
                             const int32_t *h_row_ptr, size_t *bytes);

/*
 * segpaged_prefill - attention of a chunk of new tokens over each head's
 * visible pages (device).
 *
 * Defines: the product profile's section 3 SegPagedAttention (every head reads
 * only its own pages, each class its own visible window, no attention mask);
 * the result is softmax attention restricted to the visible tokens:
 *   out[t, h] = sum_{j in V(h, p_t)} softmax_j(softmax_scale * q[t,h].k_j) v_j
 *   lse[t, h] = ln sum_{j in V(h, p_t)} exp(softmax_scale * q[t,h].k_j)
 *
 * Query tokens of sequence s are rows h_tok_ptr[s] .. h_tok_ptr[s+1]-1 of q,
 * at positions d_q_pos0[s] + (row - tok_ptr[s]).  h_tok_ptr and h_row_ptr are
 * host copies of d_tok_ptr and d_row_ptr, equal to them: they plan the
 * launch, and for calls of few rows the kernels take the bounds from them
 * rather than from the device arrays.  The tables must be those built for
 * this call's query positions.
 * d_cls, d_window: device copies of the per-slot class and window.
 * lse may be NULL.  workspace: device memory of at least
 * segpaged_workspace_bytes(SP_WS_PREFILL, ...) bytes, 256-byte aligned.
 * Supported: SP_BF16 with head_dim 64 or 128, page_size 16, 32 or 64,
 * group 1..16; SP_F32 with head_dim 16..256 (multiple of 16), any page_size.
 */
int segpaged_prefill(int dtype, int head_dim, int page_size, int group, int n_seq, int n_slot,
                     const int32_t *h_tok_ptr, const int32_t *h_row_ptr,
                     const int32_t *d_tok_ptr, const int32_t *d_q_pos0,
                     const int32_t *d_cls, const int32_t *d_window,
                     const int32_t *d_row_ptr, const sp_entry *d_entries,
                     const void *q, const void *k_pool, const void *v_pool, int64_t n_phys,
                     float softmax_scale, void *out, float *lse,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * segpaged_decode - one new token per sequence attends over each head's visible
 * pages, split over the page list and merged by log-sum-exp (device).
 *
 * Defines: the same restricted softmax attention as segpaged_prefill for a
 * single query token per sequence at position d_q_pos[s] (the decode token,
 * already stored); the tutorial page on the RedKnot HotpotQA demo notes the
 * decode side is left essentially unchanged by the method, so decode is the
 * ordinary split-K paged decode walking each head's own table.
 *   q, out [n_seq][n_slot * group][head_dim];  lse [n_seq][n_slot * group].
 * Partial results (m, l, o) of each split go to the workspace and are merged:
 *   O = sum_s e^{lse_s - M} o_s / sum_s e^{lse_s - M},  LSE = M + ln sum_s e^{lse_s - M}.
 * h_row_ptr is the host copy of d_row_ptr, equal to it: it plans the launch.
 * Supported: SP_BF16 with head_dim 64 or 128, page_size 16 or 32, group 1..16;
 * SP_F32 with head_dim 16..256 (multiple of 16), any page_size.
 */
int segpaged_decode(int dtype, int head_dim, int page_size, int group, int n_seq, int n_slot,
                    const int32_t *h_row_ptr, const int32_t *d_q_pos,
                    const int32_t *d_cls, const int32_t *d_window,
                    const int32_t *d_row_ptr, const sp_entry *d_entries,
                    const void *q, const void *k_pool, const void *v_pool, int64_t n_phys,
                    float softmax_scale, void *out, float *lse,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * segpaged_decode_static - segpaged_decode without a caller workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, hosts that forbid hipMalloc.  Same arguments, results
 * and kernels as segpaged_decode, minus the workspace.
 *
 * Scratch: a static device array of SP_STATIC_SCRATCH_BYTES in the library,
 * one per GPU, held until the process ends; its address is looked up on the
 * first call on each device.  The call allocates nothing (no hipMalloc, no
 * allocating library routine).  Every call on one GPU shares that GPU's
 * array, so calls that overlap on one GPU (different streams, or threads
 * without ordering) race and must not be issued; calls on one stream are safe.
 * The scratch needs no clearing: nothing of a previous call's contents is read.
 * Errors: as segpaged_decode; SP_EWORKSPACE (before any GPU work) when the call
 * needs more scratch than SP_STATIC_SCRATCH_BYTES (segpaged_workspace_bytes
 * with SP_WS_DECODE gives the need).
 */
#define SP_STATIC_SCRATCH_BYTES (16u << 20)
int segpaged_decode_static(int dtype, int head_dim, int page_size, int group, int n_seq, int n_slot,
                           const int32_t *h_row_ptr, const int32_t *d_q_pos,
                           const int32_t *d_cls, const int32_t *d_window,
                           const int32_t *d_row_ptr, const sp_entry *d_entries,
                           const void *q, const void *k_pool, const void *v_pool, int64_t n_phys,
                           float softmax_scale, void *out, float *lse, void *stream);

/*
 * segpaged_token_importance - the attention importance every key position
 * receives from a prefill chunk's query rows (device).
 *
 * Defines: the product profile's section 3, third building block (the elastic
 * sparse FFN picks the tokens that run the feed-forward network by attention
 * importance; low-contribution tokens skip it).  The pages give no formula;
 * the importance of key position t in a slot is the softmax probability mass
 * the chunk's rows (its tokens x the slot's group heads) give it:
 *   imp[slot][pos_ptr[s] + t] = sum over rows (i, g) of sequence s that see t of
 *                               exp(softmax_scale * q[i, h] . k_t - lse[i, h]),  h = slot*group + g
 * with lse the natural-log log-sum-exp segpaged_prefill returned for the same
 * call (same q, tables and pools); each row's probabilities then sum to 1.
 * Positions t < pos_ptr[s+1] - pos_ptr[s] of sequence s are written (0 where no
 * row sees t); keys at later positions are skipped.  imp is [n_slot][pos_ptr[n_seq]]
 * fp32.  Other arguments as segpaged_prefill; workspace of
 * segpaged_workspace_bytes(SP_WS_IMPORTANCE, ...) bytes, 256-byte aligned.
 * The result does not depend on the launch (every sum runs in a fixed order).
 * Supported: SP_BF16 with head_dim 64 or 128, page_size 16 or 32, group 1..16;
 * SP_F32 with head_dim 16..256 (multiple of 16), any page_size.
 */
int segpaged_token_importance(int dtype, int head_dim, int page_size, int group, int n_seq, int n_slot,
                              const int32_t *h_tok_ptr, const int32_t *h_row_ptr,
                              const int32_t *d_tok_ptr, const int32_t *d_q_pos0,
                              const int32_t *d_cls, const int32_t *d_window,
                              const int32_t *d_row_ptr, const sp_entry *d_entries,
                              const void *q, const void *k_pool, int64_t n_phys, float softmax_scale,
                              const float *lse, const int32_t *h_pos_ptr, const int32_t *d_pos_ptr, float *imp,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * segpaged_select_tokens - the tokens that run the FFN: in each (layer,
 * sequence) the k positions of highest layer importance (device).
 *
 * Defines: the same sparse-FFN building block (token-level selection by
 * attention importance).  Slots l * slots_per_layer .. (l + 1) * slots_per_layer - 1
 * form layer l.  For sequence s with candidates t in [0, pos_ptr[s+1] - pos_ptr[s])
 * and k = sel_ptr[s+1] - sel_ptr[s]:
 *   score[l][pos_ptr[s] + t] = imp[l*spl][..] + imp[l*spl + 1][..] + ...  (fp32, slot order)
 *   sel[l][sel_ptr[s] .. + k) = the k positions of largest score, equal scores
 *                               taken from the lowest position, in ascending order.
 * imp: [n_layers * slots_per_layer][pos_ptr[n_seq]] fp32 (non-negative, as
 * segpaged_token_importance writes it); score: [n_layers][pos_ptr[n_seq]] fp32
 * (output); sel: [n_layers][sel_ptr[n_seq]] int32 (output).  h_* are host
 * copies of the d_* arrays.  Errors: SP_EINVAL (k outside [0, candidates],
 * bad CSR, NULL pointer).
 */
int segpaged_select_tokens(int n_layers, int slots_per_layer, int n_seq, const int32_t *h_pos_ptr,
                           const int32_t *d_pos_ptr, const float *imp, const int32_t *h_sel_ptr,
                           const int32_t *d_sel_ptr, float *score, int32_t *sel, void *stream);

/* Text of a status code; segpaged_last_error: the calling thread's message for
 * its last failed call ("" if none). */
const char *segpaged_strerror(int status);
const char *segpaged_last_error(void);

/*
 * segpaged_pack_pages / segpaged_unpack_pages - gather the pages that a set of
 * table entries lists, in entry order, into contiguous K and V buffers, and
 * scatter such buffers back into pools (device).
 *
 * Defines: the product profile's section 3 and the is96.com commentary's
 * paragraphs on the per-head page table: a head reads only the pages its
 * table lists, so when prefill and decode run on different machines only
 * those pages need to move; these calls are the single-GPU gather and
 * scatter around such a transfer.  For e = 0 .. n_entries-1, p = d_entries[e].phys:
 *   pack:   k_out[e] = k_pool[p]   ([page_size][head_dim])
 *           v_out[e] = v_pool[p]   ([head_dim][page_size])
 *   unpack: k_pool[p] = k_in[e],  v_pool[p] = v_in[e]
 * Whole pages are copied; a p outside [0, n_phys) packs as zeros and is
 * skipped by unpack.  d_entries is typically a table's entries
 * (d_row_ptr[n_rows] of them).  All buffers are device memory owned by the
 * caller; packed buffers hold n_entries pages.  Unpacking entries that list
 * the same page twice leaves either copy.  dtype SP_BF16 or SP_F32.
 * Errors: SP_EINVAL (bad size, NULL pointer), SP_EUNSUPPORTED (head_dim,
 * page_size); a launch failure returns its HIP error mapped as for the other calls.
 */
int segpaged_pack_pages(int dtype, int head_dim, int page_size, int64_t n_entries, const sp_entry *d_entries,
                        const void *k_pool, const void *v_pool, int64_t n_phys, void *k_out, void *v_out,
                        void *stream);
int segpaged_unpack_pages(int dtype, int head_dim, int page_size, int64_t n_entries, const sp_entry *d_entries,
                          const void *k_in, const void *v_in, void *k_pool, void *v_pool, int64_t n_phys,
                          void *stream);

/* ABI version (major * 100 + minor). */
int segpaged_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEGPAGED_H */
