// fa_fwd_mfma_wide.hip -- exact attention forward on the CDNA4 matrix cores,
// for d = dv = 128, d = 64 with dv = 128, and d = dv = 64 over short key
// ranges.
//
// bf16/fp16 inputs, scale > 0; fp32 accumulation.
//
// Method: the FlashAttention-2 loop order of CS349E Lecture 11
// "flash_lab.py", section 3 (flash_fwd, order "fa2"): one block of 256
// query rows per workgroup; the head's K/V tiles (64 keys) stream through
// LDS; per tile the scores of the block are formed on chip, the running row
// maximum and row sum are updated with section 1's online-softmax rescaling,
// and the rescaled output accumulator gains P V.  O is divided by the row
// sum once at the end and LSE = m + ln l is written beside it.  Under the
// causal mask (query i at position Nk - N + i, section 2) tiles past the
// block's last visible key are never loaded and only tiles that straddle
// the diagonal or the end of the keys pay for masking.
//
// gfx950 mapping (8 waves, 32 query rows per wave).  At d = 128 the matrix
// work per score is twice that of d = 64, so the kernel is bound by the
// matrix cores rather than by the softmax arithmetic; it uses the larger
// 32x32 MFMA shape, whose long issue leaves room for the other wave's
// vector-ALU work on the same SIMD:
//  * Products use v_mfma_f32_32x32x16_{bf16,f16}.  Scores are computed
//    transposed, S^T = K Q^T: K is the A operand (ds_read_b128 from LDS),
//    Q^T the B operand (held in registers, read from an LDS copy of the Q
//    block).  The 32x32 result gives each lane one query (lane & 31) and 16
//    of a 32-key block's keys; the other 16 sit in lane ^ 32, so a row max
//    is an in-register max plus one v_permlane32_swap.
//  * The probabilities are rounded to the input type and used straight from
//    registers as the B operand of O^T = V^T P^T: eight consecutive result
//    registers of a score block form the B operand of one 16-key step once
//    the contraction index is read as the key order
//    {4h..4h+3, 8+4h..8+4h+3} (h = lane / 32).  V^T (the A operand) comes
//    from the row-major V tile through two ds_read_b64_tr_b16, each handing
//    a lane four consecutive keys of one value column in that order.
//  * K/V tiles are copied from memory straight into LDS (three stages each)
//    and XOR-swizzled per row (16-byte chunks for K, 64-byte groups for V)
//    so that the operand reads are free of bank conflicts.  The Q block of
//    the next item is copied into LDS while the current one is computed.
//  * The normalised output leaves through LDS: each wave writes its 32 rows
//    into one of the two K/V stages the item's last tile does not occupy
//    and stores whole rows, 1 KiB contiguous per instruction (with d = 64
//    and dv = 128 the stages hold six waves' rows; the other two store
//    their registers directly).
//  * The kernel is persistent: each workgroup walks units of two query
//    blocks of one head whose causal costs add up to a constant, numbered
//    so that workgroups of one XCD share heads (K/V reuse in that L2).
//  * At d = 64 the kernel needs 80 KiB of LDS and 128 registers, so two
//    workgroups share a CU (the launch bounds ask for four waves per SIMD
//    there).  Their items start and end at different times, and one workgroup's
//    item boundary (Q and first tiles in flight, output stores) overlaps
//    the other's tile loop.  That wins over the one-workgroup ping-pong
//    kernel of fa_fwd_mfma.hip while items are short (up to about 48 key
//    tiles); the ping-pong's vector/matrix alternation wins on longer key
//    ranges.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_mfma32.h"

namespace fa {
namespace {

using namespace mfma32;

// Checking build (FA_SERIAL_COPIES=1): every K/V tile and Q block is
// copied between two barriers and waited for before anyone reads it, so no
// copy is in flight while LDS is read.  The arithmetic and its order are
// unchanged, so this build's results must equal the pipelined build's bit
// for bit; only the race-check tests load it.
#ifndef FA_SERIAL_COPIES
#define FA_SERIAL_COPIES 0
#endif
constexpr bool kSerialCopies = FA_SERIAL_COPIES != 0;

// Eight waves; wave w owns query rows [32 w, 32 w + 32) of the block.
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBR = 256;            // query rows per workgroup
constexpr int kQW = 32;             // query rows per wave
constexpr int kBC = 64;             // keys per tile (two 32-key score blocks)

// Position in a workgroup's sequence of work items (see the kernel).
struct Cursor {
    int t, half;        // unit round and which block of the unit's pair
    int head, qblk;     // head < 0: past the end
    int ntiles, j;      // key tiles of the item; next tile to fetch
};
struct Schedule {
    int G, n_units, U, q_blocks, N, Nk;
    bool xcd_map, causal;
};
__device__ __forceinline__ Cursor locate(Cursor cu, const Schedule &s) {
    const int u = (int)blockIdx.x + cu.t * s.G;
    if (u >= s.n_units) {
        cu.head = -1;
        cu.ntiles = 0;
        return cu;
    }
    int pair;
    if (s.xcd_map) {
        const int local = u / 8;
        cu.head = (local / s.U) * 8 + u % 8;
        pair = local % s.U;
    } else {
        cu.head = u / s.U;
        pair = u % s.U;
    }
    cu.qblk = cu.half == 0 ? pair : s.q_blocks - 1 - pair;
    const int key_end =
        s.causal ? min(s.Nk, s.Nk - s.N + min(cu.qblk * kBR + kBR, s.N)) : s.Nk;
    cu.ntiles = key_end > 0 ? (key_end + kBC - 1) / kBC : 0;
    return cu;
}
__device__ __forceinline__ Cursor first_item(const Schedule &s) {
    Cursor cu;
    cu.t = 0;
    cu.half = 0;
    cu.j = 0;
    return locate(cu, s);
}
// The unit's second block, unless the unit is the odd middle block.
__device__ __forceinline__ Cursor next_item(Cursor cu, const Schedule &s) {
    const int pair = cu.half == 0 ? cu.qblk : s.q_blocks - 1 - cu.qblk;
    if (cu.half == 0 && s.q_blocks - 1 - pair != pair) {
        cu.half = 1;
    } else {
        cu.t += 1;
        cu.half = 0;
    }
    cu.j = 0;
    return locate(cu, s);
}


template <typename T, int D, int DV, bool CAUSAL>
// __launch_bounds__' second argument is the minimum number of waves per SIMD:
// 4 (two workgroups per CU, at most 128 registers) at d = dv = 64, else 2.
__global__ __launch_bounds__(kThreads, (D == 64 && DV == 64) ? 4 : 2) void fwd_mfma32_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    T *__restrict__ o, float *__restrict__ lse, int N, int Nk, float c,
    int q_blocks, int n_items) {
    typedef typename Mfma<T>::vec vec8;
    static_assert((D == 128 && DV == 128) || (D == 64 && (DV == 64 || DV == 128)), "(d, dv)");
    constexpr int KLEAD = 2;                    // K tiles fetched ahead of the tile being consumed
    constexpr int KS = D / 16;                  // 16-wide contraction steps of S (d)
    constexpr int DB = DV / 32;                 // 32-wide value blocks of O
    constexpr int CC = kBC / 16;                // 16-key contraction steps of P V
    constexpr int ROWB = D * 2;                 // bytes per key (or query) row
    constexpr int TILE = kBC * ROWB;            // bytes per K tile
    constexpr int ROWBV = DV * 2;               // bytes per value row
    constexpr int TILEV = kBC * ROWBV;          // bytes per V tile
    constexpr int CPRV = ROWBV / 16;            // 16-byte chunks per value row
    constexpr int QTILE = kBR * ROWB;           // bytes of the Q block
    constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
    constexpr int LPT = TILE / 1024 / kWaves;   // 1 KiB wave loads per wave per K tile
    constexpr int LPTV = TILEV / 1024 / kWaves; // ... per V tile
    constexpr int LPQ = QTILE / 1024 / kWaves;  // 1 KiB wave loads per wave per Q block
    static_assert(LPT * 1024 * kWaves == TILE && LPTV * 1024 * kWaves == TILEV &&
                  LPQ * 1024 * kWaves == QTILE, "tile split");
    __shared__ __attribute__((aligned(16))) unsigned char kbuf[3][TILE];
    __shared__ __attribute__((aligned(16))) unsigned char vbuf[3][TILEV];
    __shared__ __attribute__((aligned(16))) unsigned char qbuf[QTILE];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // uniform per wave
    const int lane = tid % 64;
    const int n = lane % 32;    // query column of the 32x32 blocks
    const int h = lane / 32;    // half: which keys of a 32-key block the lane holds

    // Per-lane LDS byte offsets of the MFMA operand reads within a stage; the
    // stage, key-block and step offsets are compile-time constants.
    //  K (A operand of S^T): key row n (+32 kb), 16-byte chunk 2 ks + h.
    //  Q (B operand, read once per item): query row 32 wave + n, chunk 2 ks + h.
    //  V (ds_read_b64_tr_b16, per 16-lane group G = lane/16): key row
    //    4h + (lane%16)/4 (+8, +16 cc), quad 8 db + 4 (G%2) + lane%4.
    uint32_t kofs[KS], vofs[DB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kofs[ks] = n * ROWB + (((2 * ks + h) ^ kswz<D>(n)) * 16);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int li = lane % 16;
        const int r0 = 4 * h + li / 4;
        const int u = 8 * db + 4 * ((lane / 16) % 2) + li % 4;
        vofs[db] = r0 * ROWBV + ((u ^ vswz<DV>(r0)) * 8);
    }
    // Memory-to-LDS copies (buffer_load ... lds): each wave load writes 1 KiB
    // of LDS, lane i's 16 bytes at offset 16 i, so the swizzled layout is
    // produced by choosing which global 16-byte piece each lane fetches.
    // Rows past the end of a head read as zeros (buffer bounds check).
    uint32_t koff[LPT], voff[LPTV];
#pragma unroll
    for (int t = 0; t < LPT; ++t) {
        const int slot = (t * kWaves + wave) * 64 + lane;
        const int row = slot / CPR, pc = slot % CPR;
        koff[t] = ((uint32_t)row * D + (pc ^ kswz<D>(row)) * 8) * 2u;
    }
#pragma unroll
    for (int t = 0; t < LPTV; ++t) {
        const int slot = (t * kWaves + wave) * 64 + lane;
        const int row = slot / CPRV, pc = slot % CPRV;
        voff[t] = ((uint32_t)row * DV + (((2 * pc) ^ vswz<DV>(row)) / 2) * 8) * 2u;
    }
    typedef __attribute__((address_space(3))) void lds_void;
    const uint32_t klds = (uint32_t)(size_t)(lds_void *)&kbuf[0][0];
    const uint32_t vlds = (uint32_t)(size_t)(lds_void *)&vbuf[0][0];
    const uint32_t qlds = (uint32_t)(size_t)(lds_void *)&qbuf[0];
    // Every vector-memory operation of the wave is counted; a wait leaves
    // outstanding only what was issued after a recorded count (operations
    // complete in issue order).
    int issued = 0;
    auto k_words = [&](int head) __attribute__((always_inline)) {
        return rsrc_words(k + (int64_t)head * Nk * D, (uint32_t)Nk * D * 2u);
    };
    auto v_words = [&](int head) __attribute__((always_inline)) {
        return rsrc_words(v + (int64_t)head * Nk * DV, (uint32_t)Nk * DV * 2u);
    };
    auto dma_k_w = [&](const u32x4 &kw, int tile, int stage) __attribute__((always_inline)) {
        const uint32_t tile_off = (uint32_t)tile * kBC * D * 2u;
#pragma unroll
        for (int t = 0; t < LPT; ++t)
            lds_dma16(kw, __builtin_amdgcn_readfirstlane(klds + stage * TILE + (t * kWaves + wave) * 1024),
                      tile_off + koff[t]);
        issued += LPT;
    };
    auto dma_v_w = [&](const u32x4 &vw, int tile, int stage) __attribute__((always_inline)) {
        const uint32_t tile_off = (uint32_t)tile * kBC * DV * 2u;
#pragma unroll
        for (int t = 0; t < LPTV; ++t)
            lds_dma16(vw, __builtin_amdgcn_readfirstlane(vlds + stage * TILEV + (t * kWaves + wave) * 1024),
                      tile_off + voff[t]);
        issued += LPTV;
    };
    auto dma_k = [&](int head, int tile, int stage) __attribute__((always_inline)) {
        dma_k_w(k_words(head), tile, stage);
    };
    auto dma_v = [&](int head, int tile, int stage) __attribute__((always_inline)) {
        dma_v_w(v_words(head), tile, stage);
    };
    // Q block of an item into qbuf, rows swizzled like K rows.
    auto dma_q = [&](int head, int qblk) __attribute__((always_inline)) {
        const u32x4 qw = rsrc_words(q + (int64_t)head * N * D, (uint32_t)N * D * 2u);
        const uint32_t blk_off = (uint32_t)qblk * kBR * D * 2u;
#pragma unroll
        for (int t = 0; t < LPQ; ++t) {
            const int slot = (t * kWaves + wave) * 64 + lane;
            const int row = slot / CPR, pc = slot % CPR;
            const uint32_t off = ((uint32_t)row * D + (pc ^ kswz<D>(row)) * 8) * 2u;
            lds_dma16(qw, __builtin_amdgcn_readfirstlane(qlds + (t * kWaves + wave) * 1024), blk_off + off);
        }
        issued += LPQ;
    };
    // An item's first tiles, K and V tiles 0 and 1, tile 0 first; `t1mark`
    // is the count once tile 0 is issued.
    int t1mark = 0;
    auto first_tiles = [&](int head, int ntiles) __attribute__((always_inline)) {
        if (ntiles > 0) {
            dma_k(head, 0, 0);
            dma_v(head, 0, 0);
        }
        t1mark = issued;
        if (ntiles > 1) {
            dma_k(head, 1, 1);
            dma_v(head, 1, 1);
        }
    };
    auto barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- the workgroup's item sequence ----------------------------------------
    // Persistent loop over units: a unit is a pair of query blocks of one
    // head, p and QB-1-p (the middle block alone when QB is odd): under the
    // causal mask their key counts add up to the same total for every p, so
    // units cost the same and a plain round-robin of units over the G
    // resident workgroups is balanced.  When G and the head count are
    // multiples of 8, units are numbered so that the workgroups of one XCD
    // (ids congruent mod 8) work on the same heads at the same time.
    Schedule sch;
    sch.G = gridDim.x;
    sch.q_blocks = q_blocks;
    sch.U = (q_blocks + 1) / 2;
    const int n_heads = n_items / q_blocks;
    sch.n_units = n_heads * sch.U;
    sch.N = N;
    sch.Nk = Nk;
    sch.xcd_map = (sch.G % 8 == 0) && (n_heads % 8 == 0);
    sch.causal = CAUSAL;

    // ---- per-item state ----------------------------------------------------------
    vec8 qop[KS];
    float m, l;
    float m8, neg_mu;   // m + 8 and -(m, or 0 while m = -inf), updated with m
    f32x16 oacc[DB];
    f32x16 sb[1][2];              // scores of the current tile: [32-key block]
    vec8 pb[CC];                  // probabilities of the current tile (B operands)
    int lim, full_end;

    // ---- S^T = K Q^T for the K tile in stage SK, into score buffer SP -----------
    auto scores = [&](const int sk, auto SP, auto NKBC) __attribute__((always_inline)) {
        constexpr int P = decltype(SP)::value;
        constexpr int NKB = decltype(NKBC)::value;   // 32-key blocks computed (2, or 1 on a half tile)
        const unsigned char *base = kbuf[0] + sk * TILE;
        sb[P][0] = f32x16{};
        sb[P][1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const vec8 a = *reinterpret_cast<const vec8 *>(base + kb * 32 * ROWB + kofs[ks]);
                sb[P][kb] = Mfma<T>::run(a, qop[ks], sb[P][kb]);
            }
        }
    };
    // ---- O^T += V^T P^T for the V tile in stage SV ---------------------------------
    auto accumulate = [&](const int sv, auto NKBC) __attribute__((always_inline)) {
        constexpr int NKB = decltype(NKBC)::value;
        const unsigned char *base = vbuf[0] + sv * TILEV;
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
#pragma unroll
        for (int cc = 0; cc < CC * NKB / 2; ++cc) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const unsigned char *p = base + cc * 16 * ROWBV + vofs[db];
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 8 * ROWBV));
                const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[db] = Mfma<T>::run(__builtin_bit_cast(vec8, both), pb[cc], oacc[db]);
            }
        }
    };
    // ---- masking of tile j (tiles that reach past the keys every row sees) ----
    auto mask = [&](const int j, auto SP, auto NKBC) __attribute__((always_inline)) {
        constexpr int P = decltype(SP)::value;
        constexpr int NKB = decltype(NKBC)::value;
        const int j0 = j * kBC;
        if (__builtin_expect(j0 + 32 * NKB > full_end, 0)) {
            const int t = lim - j0;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sb[P][kb][r] = 32 * kb + 8 * (r / 4) + r % 4 > t ? -INFINITY : sb[P][kb][r];
        }
    };
    // ---- online softmax of score buffer SP with lazy rescaling ---------------------
    // The running max m only moves when a row's tile max exceeds it by more
    // than 8 (base 2); otherwise the stale m is kept, so the probabilities
    // stay <= 2^8 and the accumulator needs no rescale.  The result is
    // unchanged: O and l share the same m.  When m moves, l and the output
    // accumulator are multiplied by the correction factor (exactly 1 in the
    // rows of the wave whose m stays).
    auto softmax = [&](auto SP, auto NKBC) __attribute__((always_inline)) {
        constexpr int P = decltype(SP)::value;
        constexpr int NKB = decltype(NKBC)::value;
        float x = sb[P][0][0];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) x = __builtin_elementwise_maximum(x, sb[P][kb][r]);
        // The row's tile maximum exceeds m + 8 exactly when one of its two
        // lanes' maxima does: the row maximum (a lane exchange) is formed
        // only in the rare case that some row of the wave moves.
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(x * c > m8) != 0, 0)) {
            const float mt = halves_max(x) * c;
            const bool need = mt > m8;
            const float m_new = need ? mt : m;
            const float a = need ? fast_exp2(m - m_new) : 1.f;   // 0 when m = -inf < m_new
            l *= a;
            m = m_new;
            m8 = m + 8.f;
            neg_mu = -((m == -INFINITY) ? 0.f : m);
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= a;
        }
#pragma unroll
        for (int cc = 0; cc < CC * NKB / 2; ++cc) {
            f32x8 pf;
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[e] = fast_exp2(fmaf(sb[P][cc / 2][8 * (cc % 2) + e], c, neg_mu));
            pb[cc] = __builtin_convertvector(pf, vec8);
            l = row_sum_pairs(pb[cc], l);
        }
    };
    // ---- schedule of the copies --------------------------------------------------
    // Tile t of an item lives in stage t % 3.  Before iteration j's barrier
    // each wave waits until only what it issued since the start of iteration
    // j-1 (`mark`) is outstanding; after the barrier (all reads of iteration
    // j-1 done) it fetches K and V tile j + 2 into the stage those reads
    // freed, so a tile is fetched two iterations before it is read.  An
    // item's first two tiles (tile 0 first) are fetched once the previous
    // item's reads are over, its Q block already during the previous item;
    // the item's start waits for the Q block and tile 0 (`t1mark`), and
    // iteration 0 for nothing more.
    Cursor cur = first_item(sch);
    if (cur.head >= 0 && !kSerialCopies) {
        dma_q(cur.head, cur.qblk);
        first_tiles(cur.head, cur.ntiles);
    }
    bool first = true;

    typedef std::integral_constant<int, 0> I0;

    for (; cur.head >= 0;) {
        const Cursor nxt = next_item(cur, sch);
        const int head = cur.head;
        const int q0 = cur.qblk * kBR;
        const int qw0 = q0 + wave * kQW;
        const int ntiles = cur.ntiles;
        int wave_end = Nk;   // keys below are visible to some row of this wave
        full_end = Nk;       // keys below are visible to every row of this wave
        if (CAUSAL) {
            wave_end = min(Nk, Nk - N + min(qw0 + kQW, N));
            full_end = min(Nk, Nk - N + qw0 + 1);
        }
        const int wtiles = (wave_end > 0 && qw0 < N) ? min(ntiles, (wave_end + kBC - 1) / kBC) : 0;
        // Register r of score block kb holds key j0 + 32 kb + 8 (r/4) + 4h + r%4,
        // visible to query qw0 + n iff 32 kb + 8 (r/4) + r%4 <= lim - j0.
        const int qi = qw0 + n;
        lim = (CAUSAL ? min(Nk - 1, Nk - N + qi) : Nk - 1) - 4 * h;
        m = -INFINITY;
        m8 = -INFINITY;
        neg_mu = -0.f;
        l = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
        // The first tiles can only be fetched now that the previous item's
        // reads are over.
        if (!first && !kSerialCopies) {
            barrier();
            first_tiles(head, ntiles);
        }
        first = false;
        // This item's Q block and first tiles have landed everywhere.
        if (kSerialCopies) {
            barrier();
            dma_q(head, cur.qblk);
            wait_pending(0);
        } else {
            const int pend = issued - t1mark;
            if (pend == LPT + LPTV) wait_vmcnt<LPT + LPTV>();
            else wait_pending(pend);
        }
        barrier();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qop[ks] = *reinterpret_cast<const vec8 *>(qbuf + wave * 32 * ROWB + kofs[ks]);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): qbuf is refilled after the next barrier
        // Fetch the next item's Q block after a barrier that follows every
        // wave's Q reads: iteration 0's, or one of its own for an item
        // without tiles.
        auto prefetch_next = [&]() __attribute__((always_inline)) {
            // Opaque copies keep the compiler from computing these copies'
            // addresses ahead of the loop (they would occupy scalar registers
            // for the whole item).
            int hd = nxt.head, qb = nxt.qblk;
            asm volatile("" : "+s"(hd), "+s"(qb));
            if (hd >= 0) dma_q(hd, qb);
        };
        if (ntiles == 0 && !kSerialCopies) {
            barrier();
            prefetch_next();
        }
        int mark = issued;
        // Iteration j: tile j sits in stage st = j % 3.
        auto sync = [&](const int j, const int st) __attribute__((always_inline)) {
            if (kSerialCopies) {
                barrier();
                dma_k(head, j, st);
                dma_v(head, j, st);
                wait_pending(0);
                barrier();
                return;
            }
            // In the steady state the previous iteration issued exactly one
            // K and one V tile: that count gets its own short path.
            if (j > 0) {
                const int pend = issued - mark;
                if (pend == LPT + LPTV) wait_vmcnt<LPT + LPTV>();
                else wait_pending(pend);
            }
            barrier();
            mark = issued;
            static_assert(KLEAD == 2, "stage two ahead");
            const int st2 = st == 0 ? 2 : st - 1;   // (st + 2) mod 3
            if (__builtin_expect(j + 2 < ntiles, 1)) {
                dma_k(head, j + KLEAD, st2);
                dma_v(head, j + 2, st2);
            }
            if (j == 0) prefetch_next();
        };
        // One computed tile: scores, mask, softmax, P V.
        typedef std::integral_constant<int, 2> Full;
        typedef std::integral_constant<int, 1> Half;
        auto compute = [&](const int j, const int st, auto NKBC) __attribute__((always_inline)) {
            sync(j, st);
            scores(st, I0{}, NKBC);
            mask(j, I0{}, NKBC);
            softmax(I0{}, NKBC);
            accumulate(st, NKBC);
        };
        int j = 0, st = 0;
        auto step = [&]() __attribute__((always_inline)) {
            ++j;
            st = st == 2 ? 0 : st + 1;
        };
        // A last tile whose second 32-key block no row of the wave sees is
        // computed as a half tile (its first block only).
        const int jfull = (wtiles > 0 && (wtiles - 1) * kBC + 32 >= wave_end) ? wtiles - 1 : wtiles;
        if constexpr (!(D == 128 && DV == 128 && !CAUSAL)) {
            for (; j < jfull; step()) compute(j, st, Full{});
        } else {
            // Full tiles in threes, each with its stage as a constant, so
            // that every LDS address of a tile is a register plus an
            // immediate.  Measured 4% faster at d = dv = 128 without the
            // mask; 5% slower with it, and at d = dv = 64 it costs the
            // second workgroup per CU its registers.
            for (; j + 3 <= jfull; j += 3) {
                compute(j, 0, Full{});
                compute(j + 1, 1, Full{});
                compute(j + 2, 2, Full{});
            }
            if (j < jfull) compute(j++, 0, Full{});
            if (j < jfull) compute(j++, 1, Full{});
            st = j % 3;
        }
        if (j < wtiles) {
            compute(j, st, Half{});
            step();
        }
        // Tiles past this wave's rows: keep the workgroup's barriers and copies.
        for (; j < ntiles; step()) sync(j, st);

        // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ---------------------
        // Register r of value block db holds O[qi][32 db + 8 (r/4) + 4h + r%4].
        // Buffer stores: rows past N fall outside the view and are dropped.
        const float lt = halves_sum(l);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const auto ors = make_rsrc(o + (int64_t)head * N * DV, (uint32_t)N * DV * 2u);
        typedef T t4 __attribute__((ext_vector_type(4)));
        // (d = 64 with dv = 128: the two free stages hold six waves' blocks,
        // two per V tile and one per K tile; waves 6 and 7 store directly)
        if (D == DV || wave < 6) {
            // The wave's 32 x dv block goes through LDS and leaves as whole
            // rows (16 bytes per lane, 1 KiB contiguous per instruction).
            // Once every wave has passed the item's last barrier, only the
            // stage of the last tile can still be read: the other two
            // stages (st and st + 1) hold the 8 blocks, two per K or V
            // tile.  Chunk c of row r sits at chunk c ^ oswz(r) (conflict
            // free both ways); a wave reads back only what it wrote.
            constexpr int RB = DV * 2;            // bytes per output row
            constexpr int CPRO = RB / 16;         // 16-byte chunks per row
            constexpr int RPI = 64 / CPRO;        // rows per store instruction
            const int st1 = st == 2 ? 0 : st + 1;
            unsigned char *slot;
            if constexpr (D == DV) {
                const int sidx = wave < 4 ? st : st1;
                slot = ((wave / 2) % 2 == 0 ? kbuf[sidx] : vbuf[sidx]) + (wave % 2) * (kQW * RB);
            } else {
                static_assert(TILEV == 2 * kQW * RB && TILE == kQW * RB, "six staged blocks");
                slot = wave < 4 ? vbuf[wave < 2 ? st : st1] + (wave % 2) * (kQW * RB)
                                : kbuf[wave == 4 ? st : st1];
            }
            auto oswz = [](int r) __attribute__((always_inline)) {
                return DV == 64 ? (r >> 1) & 7 : r & 15;
            };
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    t4 out;
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = static_cast<T>(oacc[db][4 * r4 + e] * inv);
                    *reinterpret_cast<t4 *>(slot + n * RB + (((4 * db + r4) ^ oswz(n)) * 16) + 8 * h) = out;
                }
            // (the lane index is re-defined so that this address arithmetic
            // is not hoisted into the tile loops)
            int el = lane;
            asm volatile("" : "+v"(el));
            const int rr = el / CPRO, cc = el % CPRO;
#pragma unroll
            for (int t = 0; t < kQW / RPI; ++t) {
                const int r = t * RPI + rr;
                const u32x4 val = *reinterpret_cast<const u32x4 *>(slot + r * RB + ((cc ^ oswz(r)) * 16));
                // Bounds-checked: rows past N fall outside the view and are dropped.
                __builtin_amdgcn_raw_buffer_store_b128(val, ors, (int)(((uint32_t)(qw0 + r) * DV) * 2u + cc * 16), 0, 0);
            }
        } else {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
                    t4 out;
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = static_cast<T>(oacc[db][4 * r4 + e] * inv);
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, out), ors,
                                                          ((uint32_t)qi * DV + 32 * db + 8 * r4 + 4 * h) * 2u, 0, 0);
                }
        }
        const auto lrs = make_rsrc(lse + (int64_t)head * N, (uint32_t)N * 4u);
        const float lv = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lv), lrs, h == 0 ? (uint32_t)qi * 4u : 0x80000000u, 0, 0);
        cur = nxt;
    }
    // Nothing is left in flight but the stores: every copy was waited for.
}

// Resident workgroups per CU of one kernel instantiation, times the CU count
// of the current device (cached per device).
template <typename T, int D, int DV, bool CAUSAL>
int resident_workgroups() {
    static int cache[64];
    return resident_workgroups_of(reinterpret_cast<const void *>(&fwd_mfma32_kernel<T, D, DV, CAUSAL>),
                                  kThreads, cache);
}

template <typename T, int D, int DV, bool CAUSAL>
hipError_t launch3(const FwdArgs &a) {
    const int q_blocks = (int)((a.N + kBR - 1) / kBR);
    const int64_t n_items = a.B * a.H * q_blocks;
    const int resident = resident_workgroups<T, D, DV, CAUSAL>();
    if (resident <= 0) return hipErrorInvalidDevice;
    const int64_t grid = n_items < resident ? n_items : resident;
    hipLaunchKernelGGL((fwd_mfma32_kernel<T, D, DV, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0,
                       a.stream, static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), static_cast<T *>(a.o), a.lse, (int)a.N,
                       (int)a.Nk, a.scale * kLog2e, q_blocks, (int)n_items);
    return hipGetLastError();
}

template <typename T, int D, int DV>
hipError_t launch2(const FwdArgs &a) {
    return a.causal ? launch3<T, D, DV, true>(a) : launch3<T, D, DV, false>(a);
}

template <typename T>
hipError_t launch1(const FwdArgs &a) {
    if (a.d == 128 && a.dv == 128) return launch2<T, 128, 128>(a);
    if (a.d == 64 && a.dv == 64) return launch2<T, 64, 64>(a);
    if (a.d == 64 && a.dv == 128) return launch2<T, 64, 128>(a);
    return hipErrorInvalidValue;
}

}  // namespace

bool fwd_wide_preferred(int64_t d, int64_t dv, int64_t Nk) {
    // d = 64: crossover measured at Nk = 3072 (B16 x H16, causal, equal times);
    // below it the two-workgroup kernel is 5-20% faster, above it 2-7% slower.
    // d = 64, dv = 128: faster at every length measured (1.46x at 1024 keys,
    // level at 16384).
    return (d == 128 && dv == 128) || (d == 64 && dv == 64 && Nk <= 3072) || (d == 64 && dv == 128);
}

hipError_t launch_fwd_mfma_wide(const FwdArgs &a) {
    return a.dtype == kBF16 ? launch1<bf16_t>(a) : launch1<f16_t>(a);
}

}  // namespace fa
