// segpaged_prefill for bf16: MFMA attention of a chunk of new tokens over each
// head's own page table, with no mask tensor.
//
// Follows the RedKnot product profile, section 3 (SegPagedAttention: every head
// reads only its own pages and each class its own visible window, on the
// mask-free attention path) and the is96.com commentary's SegPagedAttention
// paragraphs (a page table per head listing the pages it reads).  Prefill is the
// compute-bound phase (the Prefill/Decode explainer listed on the
// PagedAttention & RadixAttention page), so the two contractions run on the
// gfx950 matrix cores.
//
// Work item = (row = (slot, seq), q-tile, kv split).  A q-tile holds all
// `group` query heads of up to 32*NW/group consecutive tokens, so each staged
// K/V tile feeds every head of the slot.  Each wave owns 32 query rows.
//
// Per 64-key tile (one to four pages):
//   K  [64 keys][D]        -> LDS, token-major as stored;
//   V^T[page][D][PS keys]  -> LDS, each dim-major V page copied as it is stored;
//   S^T = K Q^T      (v_mfma_f32_32x32x16_bf16: keys x queries), so every lane
//                    holds one query's scores and the row softmax needs a single
//                    cross-lane step;
//   O^T += V^T P^T   (same instruction: dims x queries), P^T taken directly from
//                    the S^T registers.
// The K rows fed to the first product are permuted (sigma below) so that the
// score registers of each lane are exactly the 8 consecutive keys the second
// product's B operand wants - no shuffles between the two products.
// Bounds come from positions and only boundary tiles evaluate them.
#include "device_common.hpp"

namespace sp {
namespace {

constexpr int BN = kPrefillKeysPerTile;   // 64 keys per tile

struct PrefillParams {
    const bf16 *q, *kp, *vp;
    bf16 *out;
    float *lse;
    const int32_t *tok_ptr, *q_pos0, *cls, *window, *row_ptr;
    const int4 *entries;
    const int32_t *item_ptr, *item_ptr2, *part_ptr, *nsplit;
    _Float16 *part_o;   // split partials, normalised, fp16 [part][row][D]
    float *part_lse;
    int n_seq, n_rows, G, ps, tpt, Hq;
    int64_t n_phys;
    float scale_log2;   // softmax_scale * log2(e)
    unsigned long long *work_ctr;   // work tickets: {epoch, count} (ticket_issue / ticket_resolve)
    uint32_t epoch;                 // this call's epoch (never 0)
    int n_items;
};

// Output row m of a 32x32 MFMA tile <- K row sigma(m) of the 32-key block.
// Lane (n, h) holds rows m = (v/4)*8 + 4h + v%4; sigma maps them to keys
// 16*(v/8) + 8h + v%8, i.e. it swaps bits 2 and 3 of m.
__device__ __forceinline__ int sigma(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// s_waitcnt immediate that waits until at most n vector-memory loads are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14, the other counters
// left at their "no wait" maximum).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding global->LDS load); callers wait explicitly.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
    asm volatile("s_barrier" ::: "memory");
}

template <int D, int NW, int PS, int NBUF, bool INL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_bf16_kernel(
    PrefillParams P, PrefillInlinePlan L) {
    constexpr int BM = 32 * NW;
    constexpr int DK = D / 16;     // k-steps of the QK^T product
    constexpr int DT = D / 32;     // 32-dim tiles of the output
    // Tiles arrive by global->LDS loads of 1 KB per wave instruction (lane l
    // writes bytes [16 l, 16 l + 16)), each block inside one page, so a load's
    // source is a wave-uniform page base plus a per-lane offset that is the same
    // for every tile.  K rows (2D bytes) and V^T rows (2*PS bytes, one page's
    // keys of one dim) hold their 16-byte chunks XOR-swizzled by row so that the
    // MFMA operand reads of 32 rows spread over all LDS banks; the swizzle is
    // applied on the source side (lane l fetches the chunk that belongs at l).
    constexpr int KI = BN * D * 2 / 1024, VI = D * BN * 2 / 1024;   // 1 KB blocks per tile
    static_assert(KI % NW == 0 && VI % NW == 0, "tile blocks must split evenly over the waves");
    constexpr int KIW = KI / NW, VIW = VI / NW;                       // per wave and tile
    constexpr int IPW = KIW + VIW;
    constexpr int ppt = BN / PS;                                      // pages per tile
    constexpr int CPK = D / 8, RK = 1024 / (2 * D);                   // K: chunks per row, rows per block
    constexpr int CPV = PS / 8, RV = 1024 / (2 * PS);                 // V^T: chunks per row, rows per block
    constexpr int BPP = D / RV;                                       // V^T blocks per page
    static_assert(RK <= PS && PS % RK == 0, "a 1 KB block of K rows must stay inside one page");
    static_assert(RV <= D && D % RV == 0, "a 1 KB block of V^T rows must stay inside one page");
    __shared__ __attribute__((aligned(1024))) bf16 sK[NBUF][BN * D];
    __shared__ __attribute__((aligned(1024))) bf16 sV[NBUF][D * BN];
    __shared__ int sPos[NBUF][BN];  // key positions of a tile that needs bounds
    __shared__ __attribute__((aligned(16))) int4 sEnt[NW][2][4];   // per wave: page entries of its next tiles
    __shared__ int sNv[NBUF][4];    // tokens held by each page of a tile with empty key slots

    __shared__ int s_item;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, h = lane >> 5;
    auto swz_k = [](int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); };
    auto swz_v = [](int d) { return PS == 16 ? 0 : PS == 32 ? ((d >> 2) & 3) : ((d >> 1) & 7); };

    // This wave's K and V^T blocks of a tile: per-lane source offsets (bytes
    // within a page), the page of the tile they lie in (the same for all of
    // them) and their LDS byte addresses in stage 0.  Fixed for the launch.
    constexpr int BPG = PS * D / 512;                                 // 1 KB blocks per page, K and V^T alike
    static_assert(KIW == VIW && BPG % KIW == 0, "a wave's blocks of a tile must share one page");
    constexpr uint32_t kStageBytes = BN * D * 2, kPageBytes = PS * D * 2;
    uint32_t koff[KIW], voff[VIW];
#pragma unroll
    for (int q = 0; q < KIW; ++q) {
        const int blk = wave * KIW + q;
        const int row = blk * RK + lane / CPK;                    // key row of the tile
        const int c = (lane % CPK) ^ swz_k(row);
        koff[q] = (uint32_t)(((row % PS) * D + 8 * c) * 2);
    }
#pragma unroll
    for (int q = 0; q < VIW; ++q) {
        const int blk = wave * VIW + q;
        const int d = (blk % BPP) * RV + lane / CPV;              // dim row within the page
        const int c = (lane % CPV) ^ swz_v(d);
        voff[q] = (uint32_t)((d * PS + 8 * c) * 2);
    }
    const int pw = __builtin_amdgcn_readfirstlane(wave * KIW / BPG);
    const uint32_t lds_k0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&sK[0][wave * KIW * 512]);
    const uint32_t lds_v0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&sV[0][wave * VIW * 512]);
    const uint32_t lds_e0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&sEnt[wave][0][0]);

    // Persistent workgroups (one per CU) take the work items in their long-first
    // order: the hardware dispatcher places workgroups in order and would hold
    // short items back until a long one ends.  Workgroup w starts with item w;
    // the next item comes from a counter (items gridDim.x, gridDim.x + 1, ...),
    // asked for a few phases before the current item ends, so that the answer
    // is there when it ends and the order of asking still follows the order in
    // which workgroups fall free.
    for (int b = blockIdx.x; b < P.n_items;) {
        unsigned long long ticket = 0;                   // thread 0's counter value, resolved at the item's end

        // ---- work item
        int r, local;
        if constexpr (INL) item_of(L.item_ptr, L.item_ptr2, P.n_rows, b, &r, &local);
        else item_of(P.item_ptr, P.item_ptr2, P.n_rows, b, &r, &local);
        const int ns = INL ? L.nsplit[r] : P.nsplit[r];
        const int qt = local / ns, sp_i = local % ns;
        const int seq = r % P.n_seq, slot = r / P.n_seq;
        const int tok_base = INL ? L.tok_ptr[seq] : P.tok_ptr[seq];
        const int t0 = qt * P.tpt;
        const int ntok = min(P.tpt, (INL ? L.tok_ptr[seq + 1] : P.tok_ptr[seq + 1]) - tok_base - t0);
        const int p0 = P.q_pos0[seq] + t0, p_last = p0 + ntok - 1;
        const int G = P.G;
        const bool is_local = P.cls[slot] == SP_LOCAL;
        const int W = is_local ? P.window[slot] : 0;
        const int nrows = ntok * G;

        // ---- queries of this wave: row = 32*wave + n -> (token, head)
        const int row = 32 * wave + n;
        const bool row_ok = row < nrows;
        const int tq = row / G, g = row % G;
        const int pq = p0 + tq;                    // this lane's query position
        const int lowq = is_local ? pq - W : INT32_MIN;   // visible iff lowq < pos <= pq
        u32x4 qraw[DK];
        // The queries enter the matrix cores as given; each score is scaled by
        // c = scale * log2(e) into the log2 domain of the softmax in fp32 (one
        // FMA with the reference shift).  Pre-multiplying q by c and rounding
        // it to bf16 would save that FMA but add a rounding to every score
        // that grows with |q.k|: at keys four times the unit scale it pushed
        // the log-sum-exp error past 2e-2.
        const float cl = P.scale_log2;
        bf16x8 qf[DK];
        {
            const bf16 *qrow = P.q + ((int64_t)(tok_base + t0 + tq) * P.Hq + (int64_t)slot * G + g) * D;
    #pragma unroll
            for (int s = 0; s < DK; ++s) {
                qraw[s] = u32x4{0, 0, 0, 0};
                if (row_ok) qraw[s] = *(const u32x4 *)(qrow + 16 * s + 8 * h);
            }
        }

        // ---- the q-tile's visible entry range, then this split's share
        const int e_beg = INL ? L.row_ptr[r] : P.row_ptr[r], e_end = INL ? L.row_ptr[r + 1] : P.row_ptr[r + 1];
        const int4 *E = P.entries;
        int lo, hi;
        visible_range(E, e_beg, e_end, p_last, is_local, p0 - W, &lo, &hi);
        int chunk = (hi - lo + ns - 1) / ns;
        chunk = (chunk + ppt - 1) / ppt * ppt;
        const int my_lo = min(hi, lo + sp_i * chunk);
        const int my_hi = min(hi, my_lo + chunk);
        const int n_tiles = (my_hi - my_lo + ppt - 1) / ppt;


        // ---- tile issue: page entries, bounds flags, key positions, and the
        // global->LDS loads of K and V^T.
        // The entries of a tile are read one vector phase ahead of its issue
        // (tiles 0 .. 2: at the start of the item), by a global->LDS load into
        // the wave's own slot (lane l < ppt fetches page l of the tile;
        // entries past the split read the split's last), so their latency
        // hides behind a phase of work and they queue in order with the tile
        // loads; a vector load into registers instead makes the compiler wait
        // for every load in flight before using it.  Tile issue: every wave loads its own 1 KB blocks of K and
        // V^T (all inside page pw of the tile), and derives the tile's flags
        // into its own ring `flr` (8 bits per stage): bit 0 = every key exists
        // and is visible to every query of the q-tile (no bounds needed), bit
        // 1 + pg = page pg has key slots without a token (their V^T cells must
        // be zeroed).  Only for a tile that needs them does one wave (rotating)
        // write the key positions (bounds) or each page's token count
        // (zeroing) to LDS.  Pages past the split or outside the pool count as
        // {phys 0, no tokens}.
        const int n_phys32 = (int)min(P.n_phys, (int64_t)INT32_MAX);
        const int pgi = lane % ppt;                          // page of the entry a lane holds
        auto eload = [&](int t) -> int4 { return E[min(my_lo + t * ppt + pgi, my_hi - 1)]; };
        // entries of tile t into slot t & 1 of this wave, read back (after the
        // wait that covers them) as lane l: page l % ppt
        auto eload_lds = [&](int t) {
            if (lane < ppt)
                lds_dma16_buf(E + my_lo, (uint32_t)(my_hi - my_lo) * 16u,
                              (uint32_t)min(t * ppt + lane, my_hi - my_lo - 1) * 16u, lds_e0 + (t & 1) * 64);
        };
        auto eread_lds = [&](int t) -> int4 {
            asm volatile("" ::: "memory");                   // written by a load the compiler does not see
            return sEnt[wave][t & 1][pgi];
        };
        uint32_t flr = 0;
        // the flags, bounds and page of tile t (entries e) into stage st;
        // returns the byte offset of this wave's page in the pools
        auto prep = [&](int t, int st, const int4 &e) -> uint64_t {
            const bool ok = t * ppt + pgi < my_hi - my_lo && (uint32_t)e.x < (uint32_t)n_phys32;
            const int nv = ok ? min(e.z, PS) : 0;
            const uint32_t pmask = (uint32_t)__ballot(nv < PS) & ((1u << ppt) - 1);
            // A table row ascends by position and a page's positions are
            // consecutive, so with every slot holding a token the tile spans
            // [first position of page 0, last of page ppt-1]: no bounds are
            // needed when that ends at or before the first query and (local)
            // starts inside the last query's window.
            const int pos_first = __builtin_amdgcn_readlane(e.y, 0);
            const int pos_last = __builtin_amdgcn_readlane(e.y, ppt - 1) + (PS - 1);
            const bool full = pmask == 0 && pos_last <= p0 && (!is_local || pos_first > p_last - W);
            const uint32_t fl = (full ? 1u : 0u) | (pmask << 1);
            flr = __builtin_amdgcn_readfirstlane((flr & ~(0xffu << (8 * st))) | (fl << (8 * st)));
            if ((!full || pmask) && wave == t % NW) {
                const int pgl = lane / PS, tk = lane % PS;
                const int nvp = __shfl(nv, pgl, 64), pst = __shfl(e.y, pgl, 64);
                if (!full) sPos[st][lane] = tk < nvp ? pst + tk : kPosInvalid;
                if (pmask && tk == 0) sNv[st][pgl] = nvp;
            }
            const int own = __builtin_amdgcn_readlane(ok ? e.x : 0, pw);
            return (uint64_t)(uint32_t)own * kPageBytes;
        };
        auto dmas = [&](int st, uint64_t poff) {
    #pragma unroll
            for (int q = 0; q < KIW; ++q)
                lds_dma16_buf((const char *)P.kp + poff, kPageBytes, koff[q], lds_k0 + st * kStageBytes + q * 1024);
    #pragma unroll
            for (int q = 0; q < VIW; ++q)
                lds_dma16_buf((const char *)P.vp + poff, kPageBytes, voff[q], lds_v0 + st * kStageBytes + q * 1024);
        };
        // Zero the V^T slots of keys that hold no token (past a page's n_valid, or
        // pages past the split): their weight is zero, but 0 * NaN is not.  The
        // tokens of a page are a prefix of its slots, so a 16-byte cell of 8
        // keys keeps its first clamp(n_valid - 8c, 0, 8) values.
        auto fixup = [&](int st, int pmask, int t0, int nt) {   // threads t0 .. t0+nt-1 of the workgroup
    #pragma unroll
            for (int pg = 0; pg < ppt; ++pg) {
                if (!((pmask >> pg) & 1)) continue;
                const int nv = sNv[st][pg];
                for (int idx = tid - t0; idx < D * CPV; idx += nt) {
                    const int d = idx / CPV, cp = idx % CPV;
                    const int keep = min(max(nv - 8 * (cp ^ swz_v(d)), 0), 8);
                    if (keep < 8) {
                        u32x4 *cell = (u32x4 *)&sV[st][pg * D * PS + d * PS + 8 * cp];
                        *cell = keep > 0 ? keep_first_bf16(*cell, keep) : u32x4{0, 0, 0, 0};
                    }
                }
            }
        };

        // ---- running softmax state (log2 domain) and O^T accumulators.  m_ref is
        // the lane's reference max (-inf until the row's first visible key).
        float m_ref = -INFINITY, l_run = 0.f;
        f32x16 acc[DT];
    #pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{0};

        // per-lane LDS read offsets (bf16 elements); the swizzle of an operand row
        // does not depend on which 32-row tile it sits in
        const int krow0 = sigma(n) * D, kx = swz_k(sigma(n));
        const int vx = swz_v(n);

        // ---- ping-pong schedule.  The waves form two groups of one wave per
        // SIMD (waves 0-3 and 4-7 share SIMDs pairwise).  In each phase one
        // group runs its matrix products
        // (P.V of the previous tile, then S = K Q^T of the next) while the other
        // group runs the softmax of its current tile on the vector ALUs, and the
        // roles swap every phase.  Each SIMD thus has one wave feeding its
        // matrix cores and one keeping its vector ALUs busy at all times; the
        // wave in its matrix phase runs at a raised priority (s_setprio), so
        // that its matrix instructions issue ahead of the other's vector work.
        //   group 0: phase 2j   = MFMA(j): PV(j-1), QK(j);  phase 2j+1 = softmax(j)
        //   group 1: phase 2j+1 = MFMA(j);                  phase 2j+2 = softmax(j)
        // Tile m is issued in phase 2m-4 by group 1 and 2m-3 by group 0 (tiles
        // 0..2 by everyone before phase 0), waited for at the end of phase
        // 2m-1, and its stage is free after phase 2m+3.
        static_assert(NW == 8, "the ping-pong schedule pairs two groups of four waves");
        const int grp = wave >> 2;
        // Operand reads run ahead of the MFMAs that use them (explicit schedule
        // groups): S^T takes its two 32-key blocks' k-steps alternately, with
        // the reads two k-steps ahead, so the LDS latency is paid once per
        // product and few operands are live; P.V reads one k-step ahead.
        auto qk = [&](int st, f32x16 (&S)[2]) {              // S^T = K Q^T of one tile
            constexpr int AH = 2;                            // k-steps read ahead
            bf16x8 a[DK][2];
    #pragma unroll
            for (int s = 0; s < DK; ++s)
    #pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    a[s][kt] = *(const bf16x8 *)(&sK[st][krow0 + 32 * kt * D] + ((2 * s + h) ^ kx) * 8);
    #pragma unroll
            for (int s = 0; s < DK; ++s)
    #pragma unroll
                for (int kt = 0; kt < 2; ++kt) S[kt] = mfma32x32x16(a[s][kt], qf[s], s == 0 ? f32x16{0} : S[kt]);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * AH, 0);       // reads of k-steps 0 .. AH-1
    #pragma unroll
            for (int i = 0; i < 2 * (DK - AH); ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA of k-step i / 2
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // read of k-step i / 2 + AH
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * AH, 0);       // MFMAs of the last AH k-steps
        };
        auto pv = [&](int st, const u32x4 (&Pk)[4]) {       // O^T += V^T P^T over one tile
            bf16x8 a[4][DT];
    #pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int pg = 16 * s2 / PS, c = (16 * s2 % PS) / 8 + h;
                const bf16 *vb = &sV[st][pg * D * PS + n * PS + 8 * (c ^ vx)];
    #pragma unroll
                for (int dt = 0; dt < DT; ++dt) a[s2][dt] = *(const bf16x8 *)(vb + 32 * dt * PS);
            }
    #pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
    #pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma32x32x16(a[s2][dt], u4_as_bf16x8(Pk[s2]), acc[dt]);
            __builtin_amdgcn_sched_group_barrier(0x100, DT, 0);           // reads of k-step 0
    #pragma unroll
            for (int i = 0; i < 3 * DT; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA of k-step i / DT
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // read of k-step i / DT + 1
            }
            __builtin_amdgcn_sched_group_barrier(0x008, DT, 0);           // MFMAs of k-step 3
        };
        // Online softmax with a rarely moved reference (log2 domain).  The weights
        // of a tile are exp2(x - m_ref), x = c * q.k, formed in the score registers; the
        // reference only moves when one of them would exceed 2^16 (the lane's
        // sum of its weights exceeds 2^16, or is inf) or while the row has no
        // reference yet.  Only then are the scores formed again (the tile is
        // still resident), the row max taken and the accumulators rescaled.
        // Weights up to 2^16 are harmless in bf16 and fp32, and once m_ref is a
        // true row max, l >= 1, so weights that underflow are negligible.  The
        // final normalisation by l makes the result independent of m_ref.
        constexpr float kMaxWeight = 65536.f;
        auto mask = [&](int st, f32x16 (&S)[2]) {            // bounds of a boundary tile
    #pragma unroll
            for (int kt = 0; kt < 2; ++kt)
    #pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int kpos = sPos[st][32 * kt + 16 * (v >> 3) + 8 * h + (v & 7)];
                    S[kt][v] = (kpos <= pq && kpos > lowq) ? S[kt][v] : -INFINITY;
                }
        };
        // Weights -> packed bf16 P^T operands, in place over all 32 scores per
        // stage (32 independent operations at a time for the vector ALU); returns
        // the lane's sum of the weights in fp32, before their rounding to bf16
        // (plain adds: a dot-product instruction here waits for the matrix
        // cores that the SIMD's other wave keeps busy).  v_exp_f32 flushes
        // results below 2^-126 to zero, which is harmless.
        auto weights = [&](f32x16 (&S)[2], u32x4 (&Pk)[4]) {
    #pragma unroll
            for (int kt = 0; kt < 2; ++kt)
    #pragma unroll
                for (int v = 0; v < 16; ++v) S[kt][v] = __builtin_amdgcn_exp2f(S[kt][v]);
    #pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
    #pragma unroll
                for (int w = 0; w < 4; ++w)
                    Pk[s2][w] = pack_bf16x2(S[s2 >> 1][8 * (s2 & 1) + 2 * w], S[s2 >> 1][8 * (s2 & 1) + 2 * w + 1]);
            float r4[4] = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
            for (int kt = 0; kt < 2; ++kt)
    #pragma unroll
                for (int v = 0; v < 16; ++v) r4[v & 3] += S[kt][v];
            return (r4[0] + r4[1]) + (r4[2] + r4[3]);
        };
        auto scale_shift = [&](f32x16 (&S)[2], float a, float b) {
    #pragma unroll
            for (int kt = 0; kt < 2; ++kt)
    #pragma unroll
                for (int v = 0; v < 16; ++v) S[kt][v] = fmaf(S[kt][v], a, b);
        };
        auto softmax = [&](int st, bool full, f32x16 (&S)[2], u32x4 (&Pk)[4]) {
            if (!full) mask(st, S);
            const float m_fin = m_ref == -INFINITY ? 0.f : m_ref;
            scale_shift(S, cl, -m_fin);                      // x - m_ref, x = c * q.k
            float rs = weights(S, Pk);
            if (__any(!(rs <= kMaxWeight) || m_ref == -INFINITY)) {
                qk(st, S);                                   // the scores again
                if (!full) mask(st, S);
                float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    #pragma unroll
                for (int kt = 0; kt < 2; ++kt)
    #pragma unroll
                    for (int v = 0; v < 16; ++v) m4[(kt * 16 + v) & 3] = fmaxf(m4[(kt * 16 + v) & 3], S[kt][v]);
                float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
                mx = fmaxf(mx, xor_lane(mx, 32));           // the row's other 32 keys
                const float m_new = fmaxf(m_ref, mx * cl);
                if (m_new != -INFINITY) {
                    // nothing is accumulated while m_ref is -inf
                    const float alpha = m_ref == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
                    l_run *= alpha;
    #pragma unroll
                    for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
                    m_ref = m_new;
                }
                const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
                scale_shift(S, cl, -m_use);
                rs = weights(S, Pk);
            }
            l_run += rs;
        };

        static_assert(NBUF == 4, "tiles m-1 .. m+2 occupy the four stages around phase 2m");
        {
            // tiles 0 .. 2: their entries read together, then issued in order
            int4 e3[NBUF - 1];
    #pragma unroll
            for (int j = 0; j < NBUF - 1; ++j) e3[j] = j < n_tiles ? eload(j) : int4{0, 0, 0, 0};
            if (n_tiles > NBUF - 1) eload_lds(NBUF - 1);   // the first tile the loop issues
    #pragma unroll
            for (int j = 0; j < NBUF - 1; ++j)
                if (j < n_tiles) dmas(j, prep(j, j, e3[j]));
        }
    #pragma unroll
        for (int s = 0; s < DK; ++s) qf[s] = u4_as_bf16x8(qraw[s]);
        if (n_tiles > 0) {
            if (n_tiles > 2) wait_vmcnt<2 * IPW>();
            else if (n_tiles > 1) wait_vmcnt<IPW>();
            else wait_vmcnt<0>();
            lds_barrier();
        }
        f32x16 S[2];
        u32x4 Pk[4];
        // Each group runs its own loop (the branch on the group skips the other
        // loop), so that a phase carries no test of which kind it is.  Both
        // loops run n_it iterations of one workgroup barrier each.
        // Iteration i of a group: its matrix phase (P.V of tile i-1, then S of
        // tile i) and its vector phase (group 0: the softmax of tile i after
        // the matrix phase; group 1: the softmax of tile i-1 before it), then
        // the barrier.  Each vector phase first issues tile i + 2
        // (prepared from the entries read one vector phase earlier) and reads
        // the entries of tile i + 3.  Tile m is issued in iteration m-2 and
        // waited for at the end of iteration m-1; its stage is free after
        // iteration m+1.
        const int n_it = n_tiles > 0 ? n_tiles + 1 : 0;
        // e: the entries of tile i + 2, read back at the start of the
        // iteration (the barrier ending the previous one waited for them: they
        // were loaded before the loads of tile i + 1)
        auto vphase = [&](int i, int js, const int4 &e) {
            const bool act = js >= 0 && js < n_tiles;
            const bool full = act && ((flr >> (8 * (js % NBUF))) & 1);
            if (i >= 1 && i + 2 < n_tiles) {
                // prepare tile i + 2, read the entries of tile i + 3, then
                // issue the loads of tile i + 2
                const uint64_t poff = prep(i + 2, (i + 2) % NBUF, e);
                if (i + 3 < n_tiles) eload_lds(i + 3);
                dmas((i + 2) % NBUF, poff);
            }
            if (act) softmax(js % NBUF, full, S, Pk);
        };
        auto mphase = [&](int i) {
            if (i >= 1) pv((i - 1) % NBUF, Pk);
            if (i < n_tiles) qk(i % NBUF, S);
        };
        auto sync = [&](int i) {                             // tile i+1 is used from the next iteration on
            const int m = i + 1;
            // every wave's loads newer than those of tile m: the loads of tile
            // m + 1, after the entry read of tile m + 2 (from iteration 1 on),
            // which is small and finishes first, so waiting for all but the
            // last IPW also covers it (thread 0's counter ticket, taken late
            // in an item, only makes this wait longer)
            if (m < n_tiles) {
                if (m + 1 < n_tiles) wait_vmcnt<IPW>();
                else wait_vmcnt<0>();
            }
            // it publishes tile m and retires the stage that the next issue reuses
            lds_barrier();
        };
        if (n_it == 0 && tid == 0) ticket = ticket_issue(P.work_ctr);
        if (grp == 0) {
            const int i_ticket = max(0, n_it - 2);
            auto step0 = [&](int i) {
                if (i == i_ticket && tid == 0) ticket = ticket_issue(P.work_ctr);
                const int4 e = eread_lds(i + 2);                 // lands during the matrix phase
                __builtin_amdgcn_s_setprio(2);                   // matrix issue first on the SIMD
                mphase(i);
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(0);
                vphase(i, i, e);
                __builtin_amdgcn_sched_barrier(0);
                sync(i);
            };
            // unrolled by the ring size, so that every stage index is a constant
            for (int j = 0; j < n_it; j += NBUF) {
                step0(j);
                if (j + 1 < n_it) step0(j + 1);
                if (j + 2 < n_it) step0(j + 2);
                if (j + 3 < n_it) step0(j + 3);
            }
        } else {
            auto step1 = [&](int i) {
                const int pm = (flr >> (8 * (i % NBUF) + 1)) & 0x7f;
                if (i < n_tiles && pm) fixup(i % NBUF, pm, 4 * 64, 4 * 64);   // before P.V(i), one iteration on
                vphase(i, i - 1, eread_lds(i + 2));
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(2);
                mphase(i);
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(0);
                sync(i);
            };
            for (int j = 0; j < n_it; j += NBUF) {
                step1(j);
                if (j + 1 < n_it) step1(j + 1);
                if (j + 2 < n_it) step1(j + 2);
                if (j + 3 < n_it) step1(j + 3);
            }
        }

        // The next item, published before the epilogue's stores are issued, so
        // that waiting for the counter's answer (long since arrived) does not
        // also wait for them.
        if (tid == 0) s_item = (int)gridDim.x + ticket_resolve(P.work_ctr, P.epoch, ticket);

        // ---- epilogue
        const float l = l_run + xor_lane(l_run, 32);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const float lse = l > 0.f ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
        if (!row_ok) {
            // a row past the q-tile's tokens: nothing to write
        } else if (ns == 1) {
            bf16 *orow = P.out + ((int64_t)(tok_base + t0 + tq) * P.Hq + (int64_t)slot * G + g) * D;
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt)
    #pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int d = 32 * dt + 8 * q4 + 4 * h;
                    u32x2 w;
                    w[0] = pack_bf16x2(acc[dt][4 * q4 + 0] * inv, acc[dt][4 * q4 + 1] * inv);
                    w[1] = pack_bf16x2(acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv);
                    *(u32x2 *)(orow + d) = w;
                }
            if (P.lse && h == 0) P.lse[(int64_t)(tok_base + t0 + tq) * P.Hq + (int64_t)slot * G + g] = lse;
        } else {
            const int64_t part = (int64_t)(INL ? L.part_ptr[r] : P.part_ptr[r]) + local;
            _Float16 *po = P.part_o + (part * BM + row) * D;
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt)
    #pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int d = 32 * dt + 8 * q4 + 4 * h;
                    const f32x4 v = {acc[dt][4 * q4] * inv, acc[dt][4 * q4 + 1] * inv, acc[dt][4 * q4 + 2] * inv,
                                     acc[dt][4 * q4 + 3] * inv};
                    *(f16x4 *)(po + d) = __builtin_convertvector(v, f16x4);
                }
            if (h == 0) P.part_lse[part * BM + row] = lse;
        }
        // Barriers on LDS only: every wave is done with this item's LDS (its tile
        // loads were all waited for in the last iteration) and s_item is
        // written; the epilogue's global stores stay in flight while the next
        // item starts (nothing in this kernel reads them).
        lds_barrier();
        b = __builtin_amdgcn_readfirstlane(s_item);
        lds_barrier();                       // read before the next item's ticket overwrites it
    }   // work items
}

// Combines the kv splits of every split q-tile: O = sum_s e^{lse_s-M} o_s / sum_s e^{lse_s-M}.
// Launched over the split items (numbered first): item (q-tile, split s) merges
// rows [s * ceil(rows/ns), (s+1) * ceil(rows/ns)) of its q-tile, so all splits
// share the work, and blockIdx.y spreads those rows over workgroups.  A lane
// owns 8 dims of one row and splits g, g + SG, g + 2 SG, ... (D/8 lanes per
// row and split group); it merges them online (running max, rescaled sums)
// with the loads of several splits in flight together, and the SG split
// groups of a row are combined by lane exchanges at the end.  SG = 1 suits
// many rows with few splits each, SG > 1 few rows with many splits.  The
// partials are normalised (|o| <= max |v|), so fp16 keeps them to about
// 5e-4 relative.
// A q-tile cut into kDeepMergeSplits or more kv splits (a small call splits
// its rows finely) is merged one row per workgroup: lane (g, c) of wave w
// merges dims 8c .. 8c+7 of the row over splits w*SGW + g, + 4*SGW, ...
// online (running max, rescaled sums), so 16 lane groups share the splits;
// the groups are combined by lane exchanges within a wave and through LDS
// across the four waves.  Same arithmetic as the per-wave merge below.
template <int D, bool INL>
__device__ __forceinline__ void prefill_merge_deep(const PrefillParams &P, const PrefillInlinePlan &L, int BM, int r,
                                                   int local, int ns) {
    constexpr int CH = D / 8, SGW = 64 / CH, NWm = 4, TG = SGW * NWm;
    __shared__ float smd[NWm][CH], szd[NWm][CH];
    __shared__ float sod[NWm][CH][8];
    const int qt = local / ns, sp_i = local % ns;
    const int per = (BM + ns - 1) / ns;
    if ((int)blockIdx.y >= per) return;                     // the whole workgroup: no row of this split here
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane % CH, g = wave * SGW + lane / CH;
    const int seq = r % P.n_seq, slot = r / P.n_seq;
    const int row = sp_i * per + blockIdx.y;
    const int rl = min(row, BM - 1);
    const int tok_base = INL ? L.tok_ptr[seq] : P.tok_ptr[seq];
    const int t0 = qt * P.tpt;
    const int ntok = min(P.tpt, (INL ? L.tok_ptr[seq + 1] : P.tok_ptr[seq + 1]) - tok_base - t0);
    const int nrows = ntok * P.G;
    const int64_t part0 = (int64_t)(INL ? L.part_ptr[r] : P.part_ptr[r]) + (int64_t)qt * ns;
    const float *lse = P.part_lse + part0 * BM + rl;
    const _Float16 *src = P.part_o + (part0 * BM + rl) * D + 8 * c;
    float m = -INFINITY, z = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    auto add = [&](float x, const f16x8 &v) {
        if (x == -INFINITY) return;                   // a split that sees no key
        if (x > m) {
            const float a = __expf(m - x);            // 0 while m is -inf
            z *= a;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= a;
            m = x;
        }
        const float wgt = __expf(x - m);
        z += wgt;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += wgt * (float)v[e];
    };
    constexpr int kPre = 4;
    float px[kPre];
    f16x8 pv[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
        const int s = g + i * TG;
        px[i] = -INFINITY;
        if (s < ns) {
            px[i] = lse[(int64_t)s * BM];
            pv[i] = *(const f16x8 *)(src + (int64_t)s * BM * D);
        }
    }
#pragma unroll
    for (int i = 0; i < kPre; ++i)
        if (g + i * TG < ns) add(px[i], pv[i]);
#pragma unroll 4
    for (int s = g + kPre * TG; s < ns; s += TG) add(lse[(int64_t)s * BM], *(const f16x8 *)(src + (int64_t)s * BM * D));
    auto combine = [&](float m2, float z2, const float *o2) {   // this state += another, by their max
        const float mm = fmaxf(m, m2);
        const float a = mm == -INFINITY ? 0.f : __expf(m - mm);
        const float b = mm == -INFINITY ? 0.f : __expf(m2 - mm);
        z = z * a + z2 * b;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = o[e] * a + o2[e] * b;
        m = mm;
    };
#pragma unroll
    for (int off = CH; off < 64; off <<= 1) {         // the wave's split groups
        float o2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(o[e], off, 64);
        const float m2 = __shfl_xor(m, off, 64), z2 = __shfl_xor(z, off, 64);
        combine(m2, z2, o2);
    }
    if (lane < CH) {
        smd[wave][c] = m;
        szd[wave][c] = z;
#pragma unroll
        for (int e = 0; e < 8; ++e) sod[wave][c][e] = o[e];
    }
    __syncthreads();
    if (wave != 0 || lane >= CH || row >= min(nrows, (sp_i + 1) * per)) return;
#pragma unroll
    for (int w = 1; w < NWm; ++w) combine(smd[w][c], szd[w][c], sod[w][c]);
    const float inv = z > 0.f ? 1.f / z : 0.f;
    const int tq = row / P.G, gh = row % P.G;
    const int64_t orow = (int64_t)(tok_base + t0 + tq) * P.Hq + (int64_t)slot * P.G + gh;
    u32x4 pk;
#pragma unroll
    for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(o[2 * i] * inv, o[2 * i + 1] * inv);
    *(u32x4 *)(P.out + orow * D + 8 * c) = pk;
    if (P.lse && c == 0) P.lse[orow] = z > 0.f ? m + logf(z) : -INFINITY;
}

template <int D, int SG, bool INL>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillParams P, PrefillInlinePlan L, int BM) {
    constexpr int CH = D / 8, RPW = 64 / (CH * SG), RPB = 4 * RPW;   // rows per wave / workgroup
    static_assert(RPW >= 1 && 64 % (CH * SG) == 0, "a wave holds whole rows");
    int r, local;
    if constexpr (INL) item_of(L.item_ptr, L.item_ptr2, P.n_rows, blockIdx.x, &r, &local);
    else item_of(P.item_ptr, P.item_ptr2, P.n_rows, blockIdx.x, &r, &local);
    const int ns = INL ? L.nsplit[r] : P.nsplit[r];
    if (ns == 1) return;
    if (ns >= kDeepMergeSplits) {
        prefill_merge_deep<D, INL>(P, L, BM, r, local, ns);
        return;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane % CH, g0 = (lane / CH) % SG;
    const int qt = local / ns, sp_i = local % ns;
    const int seq = r % P.n_seq, slot = r / P.n_seq;
    // Split s merges rows [s * per, (s + 1) * per) of the q-tile, per taken
    // from the tile's row count BM (as the grid is), so that the partials'
    // addresses do not wait for the q-tile's token count; rows past it are
    // read (from inside the tile's partials) but not written.
    const int per = (BM + ns - 1) / ns;
    const int row = sp_i * per + blockIdx.y * RPB + wave * RPW + lane / (CH * SG);
    const int rl = min(row, BM - 1);
    const int tok_base = INL ? L.tok_ptr[seq] : P.tok_ptr[seq];
    const int t0 = qt * P.tpt;
    const int ntok = min(P.tpt, (INL ? L.tok_ptr[seq + 1] : P.tok_ptr[seq + 1]) - tok_base - t0);
    const int nrows = ntok * P.G;
    const int64_t part0 = (int64_t)(INL ? L.part_ptr[r] : P.part_ptr[r]) + (int64_t)qt * ns;   // splits part0 .. part0+ns-1
    const float *lse = P.part_lse + part0 * BM + rl;
    const _Float16 *src = P.part_o + (part0 * BM + rl) * D + 8 * c;
    float m = -INFINITY, z = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    auto add = [&](float x, const f16x8 &v) {
        if (x == -INFINITY) return;                   // a split that sees no key
        if (x > m) {
            const float a = __expf(m - x);            // 0 while m is -inf
            z *= a;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= a;
            m = x;
        }
        const float wgt = __expf(x - m);
        z += wgt;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += wgt * (float)v[e];
    };
    // the first kPre splits of the lane's group: every load issued before any is used
    constexpr int kPre = 8;
    float px[kPre];
    f16x8 pv[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
        const int s = g0 + i * SG;
        px[i] = -INFINITY;
        if (s < ns) {
            px[i] = lse[(int64_t)s * BM];
            pv[i] = *(const f16x8 *)(src + (int64_t)s * BM * D);
        }
    }
#pragma unroll
    for (int i = 0; i < kPre; ++i)
        if (g0 + i * SG < ns) add(px[i], pv[i]);
#pragma unroll 4
    for (int s = g0 + kPre * SG; s < ns; s += SG) add(lse[(int64_t)s * BM], *(const f16x8 *)(src + (int64_t)s * BM * D));
#pragma unroll
    for (int off = CH; off < CH * SG; off <<= 1) {    // combine the split groups of the row
        const float m2 = __shfl_xor(m, off, 64);
        const float mm = fmaxf(m, m2);
        const float a = mm == -INFINITY ? 0.f : __expf(m - mm);
        const float b = mm == -INFINITY ? 0.f : __expf(m2 - mm);
        z = z * a + __shfl_xor(z, off, 64) * b;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = o[e] * a + __shfl_xor(o[e], off, 64) * b;
        m = mm;
    }
    if (g0 != 0 || row >= min(nrows, (sp_i + 1) * per)) return;   // whole rows: the exchanges above stay inside one
    const float inv = z > 0.f ? 1.f / z : 0.f;
    const int tq = row / P.G, g = row % P.G;
    const int64_t orow = (int64_t)(tok_base + t0 + tq) * P.Hq + (int64_t)slot * P.G + g;
    u32x4 pk;
#pragma unroll
    for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(o[2 * i] * inv, o[2 * i + 1] * inv);
    *(u32x4 *)(P.out + orow * D + 8 * c) = pk;
    if (P.lse && c == 0) P.lse[orow] = z > 0.f ? m + logf(z) : -INFINITY;
}

// Writes the work-item prefix sums of the launch plan into the workspace; one
// wave, the same integer formulas as the host plan (row_items).  Items of
// split rows are numbered first (item_ptr), those of unsplit rows after them
// (item_ptr2, counted from zero; see item_of).  Rows go 64 at a time through
// wave-wide inclusive scans (no workgroup barriers: the kernel is on the
// critical path of every call).
__device__ __forceinline__ int wave_incl_scan(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(x, off, 64);
        if (lane >= off) x += t;
    }
    return x;
}

__global__ __launch_bounds__(64) void plan_kernel(const int32_t *__restrict__ row_ptr,
                                                  const int32_t *__restrict__ tok_ptr, int n_seq, int n_rows,
                                                  int tpt, int chunk, int32_t *item_ptr, int32_t *item_ptr2,
                                                  int32_t *part_ptr, int32_t *nsplit, int32_t *zero) {
    const int lane = threadIdx.x;
    zero[lane] = 0;
    int carry_l = 0, carry_s = 0, carry_p = 0;
    for (int base = 0; base < n_rows; base += 64) {
        const int r = base + lane;
        int il = 0, is = 0, pt = 0;
        if (r < n_rows) {
            int nq = 1;
            if (tok_ptr) {
                const int q = r % n_seq;
                nq = (tok_ptr[q + 1] - tok_ptr[q] + tpt - 1) / tpt;
            }
            int ns, it;
            row_items(row_ptr[r + 1] - row_ptr[r], nq, chunk, &ns, &it);
            nsplit[r] = ns;
            if (ns > 1) { il = it; pt = it; }
            else is = it;
        }
        const int sl = wave_incl_scan(il), ss = wave_incl_scan(is), sp = wave_incl_scan(pt);
        if (r < n_rows) {
            item_ptr[r] = carry_l + sl - il;
            item_ptr2[r] = carry_s + ss - is;
            part_ptr[r] = carry_p + sp - pt;
        }
        carry_l += __shfl(sl, 63, 64);
        carry_s += __shfl(ss, 63, 64);
        carry_p += __shfl(sp, 63, 64);
    }
    if (lane == 0) {
        item_ptr[n_rows] = carry_l;
        item_ptr2[n_rows] = carry_s;
        part_ptr[n_rows] = carry_p;
    }
}

}  // namespace

int launch_plan(const Plan &p, const int32_t *d_row_ptr, const int32_t *d_tok_ptr, int n_seq, void *ws,
                hipStream_t stream) {
    char *w = (char *)ws;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(64), 0, stream, d_row_ptr, d_tok_ptr, n_seq, p.n_rows,
                       p.tok_per_tile, p.chunk_pages, (int32_t *)(w + p.off_item_ptr),
                       (int32_t *)(w + p.off_item_ptr2), (int32_t *)(w + p.off_part_ptr), (int32_t *)(w + p.off_nsplit), (int32_t *)(w + p.off_zero));
    return check_hip(hipGetLastError(), "plan launch");
}

int launch_prefill_f32(const AttnArgs &a, int64_t n_tok, hipStream_t stream);

template <int D, int PS, bool INL>
void launch_prefill_kernels(const PrefillParams &P, const PrefillInlinePlan &L, const Plan &p, bool merge_wide, dim3 grid,
                            dim3 mgrid, hipStream_t stream) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, 8, PS, 4, INL>), grid, dim3(512), 0, stream, P, L);
    if (p.n_parts && merge_wide)
        hipLaunchKernelGGL((prefill_merge_kernel<D, 4, INL>), mgrid, dim3(256), 0, stream, P, L, p.rows_per_tile);
    else if (p.n_parts)
        hipLaunchKernelGGL((prefill_merge_kernel<D, 1, INL>), mgrid, dim3(256), 0, stream, P, L, p.rows_per_tile);
}

int launch_prefill(const AttnArgs &a, const Plan &p, int64_t n_tok, hipStream_t stream) {
    if (a.dtype == SP_F32) return launch_prefill_f32(a, n_tok, stream);
    // Few rows: the plan goes in the kernel arguments (no plan kernel, and an
    // item's first reads are of kernel arguments); otherwise the plan kernel
    // writes it to the workspace.  Either way the ticket counter needs no
    // clearing: each call counts under its own epoch.
    const bool inl = p.n_rows <= kPrefillInlineRows && a.h_row_ptr != nullptr && a.h_tok_ptr != nullptr;
    PrefillInlinePlan L;
    if (inl) {
        fill_inline_plan(p.n_rows, a.n_seq, a.h_row_ptr, a.h_tok_ptr, p.tok_per_tile, p.chunk_pages, &L);
        for (int r = 0; r <= p.n_rows; ++r) L.row_ptr[r] = a.h_row_ptr[r];
        for (int q = 0; q <= a.n_seq; ++q) L.tok_ptr[q] = a.h_tok_ptr[q];
    } else {
        L.item_ptr[0] = 0;
        const int rc = launch_plan(p, a.d_row_ptr, a.d_tok_ptr, a.n_seq, a.ws, stream);
        if (rc) return rc;
    }
    const uint32_t epoch = next_epoch();
    char *w = (char *)a.ws;
    PrefillParams P;
    P.q = (const bf16 *)a.q;
    P.kp = (const bf16 *)a.k_pool;
    P.vp = (const bf16 *)a.v_pool;
    P.out = (bf16 *)a.out;
    P.lse = a.lse;
    P.tok_ptr = a.d_tok_ptr;
    P.q_pos0 = a.d_q_pos;
    P.cls = a.d_cls;
    P.window = a.d_window;
    P.row_ptr = a.d_row_ptr;
    P.entries = (const int4 *)a.d_entries;
    P.item_ptr = (const int32_t *)(w + p.off_item_ptr);
    P.item_ptr2 = (const int32_t *)(w + p.off_item_ptr2);
    P.part_ptr = (const int32_t *)(w + p.off_part_ptr);
    P.nsplit = (const int32_t *)(w + p.off_nsplit);
    P.part_o = (_Float16 *)(w + p.off_part_o);
    P.part_lse = (float *)(w + p.off_part_lse);
    P.n_seq = a.n_seq;
    P.n_rows = p.n_rows;
    P.G = a.group;
    P.ps = a.page_size;
    P.tpt = p.tok_per_tile;
    P.Hq = a.n_slot * a.group;
    P.n_phys = a.n_phys;
    P.scale_log2 = a.scale * kLog2e;
    P.work_ctr = (unsigned long long *)(w + p.off_zero + 128);
    P.epoch = epoch;
    P.n_items = (int)p.n_items;
    // merge: split groups per row from the rows each split item merges
    // (rows split kDeepMergeSplits ways or more take one row per workgroup)
    const bool merge_wide = p.merge_rows <= 16;
    const int merge_rpb = 4 * 64 / (a.head_dim / 8) / (merge_wide ? 4 : 1);   // rows per merge workgroup
    const dim3 mgrid((unsigned)std::max<int64_t>(1, p.n_parts),
                     (unsigned)std::max(1, std::max((p.merge_rows + merge_rpb - 1) / merge_rpb, p.merge_rows_deep)));
    const dim3 grid_persist((unsigned)std::min<int64_t>(p.n_items, kPlanCUs));
#define SP_PREFILL_CASE(DD, PSV)                                                                     \
    if (a.head_dim == DD && a.page_size == PSV) {                                                    \
        if (inl) launch_prefill_kernels<DD, PSV, true>(P, L, p, merge_wide, grid_persist, mgrid, stream);  \
        else launch_prefill_kernels<DD, PSV, false>(P, L, p, merge_wide, grid_persist, mgrid, stream);     \
    }
    SP_PREFILL_CASE(128, 16) else SP_PREFILL_CASE(128, 32) else SP_PREFILL_CASE(128, 64)
    else SP_PREFILL_CASE(64, 16) else SP_PREFILL_CASE(64, 32) else SP_PREFILL_CASE(64, 64)
    else return fail(SP_EUNSUPPORTED, "bf16 prefill head_dim %d page_size %d", a.head_dim, a.page_size);
#undef SP_PREFILL_CASE
    return check_hip(hipGetLastError(), "prefill launch");
}

}  // namespace sp
