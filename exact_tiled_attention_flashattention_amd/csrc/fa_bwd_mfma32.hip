// fa_bwd_mfma32.hip -- the dK/dV half of the attention backward on the
// CDNA4 32x32x16 matrix-core instruction (bf16/fp16 inputs, fp32
// accumulation).  The kernel is written for d, dv in {64, 128}; only
// d = dv = 64 is built and dispatched (the other pairs spill registers at
// two waves per SIMD and stay on the 16-key kernel of fa_bwd_mfma.hip).
//
// Method: CS349E Lecture 11 "flash_lab.py", section 3 (flash_bwd, the
// FlashAttention-2 backward), the key-block side: a block of keys keeps
// its dK and dV accumulators on chip while the query rows stream past;
// for each row block the probabilities are recomputed from Q, K and the
// forward's LSE, P = exp(S scale - LSE), and with the row dots
// D_i = rowsum(dO o O):
//     dV += P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dK += dS^T Q (x scale).
// The dQ half runs as its own kernel before this one (fa_bwd_mfma.hip); it
// also writes, per query row, L2 = LSE log2(e) (+inf for a row that sees no
// key) and D into the workspace, which this kernel reads.
//
// gfx950 mapping: a workgroup of 8 waves owns a block of 256 keys of one
// head at a time, 32 per wave as the columns of 32x32 blocks; two waves per
// SIMD.  The wave's K and V rows are B operands held in registers for the
// whole block, and the walk goes over the query rows in steps of 64 (two
// 32-row sub-blocks):
//  * S = Q K^T and dP = dO V^T: Q and dO are A operands read row-major from
//    LDS; the 32x32 results give each lane one key (lane % 32) and 16 of the
//    step's rows, 8 (r/4) + 4h + r%4 for register r (h = lane / 32);
//  * P and dS, rounded to the input type, are the B operands of
//    dV^T += dO^T P and dK^T += Q^T dS straight from registers: eight
//    consecutive result registers form the B operand of one 16-row step
//    once its contraction index is read as the row order
//    {4h..4h+3, 8+4h..8+4h+3}, and dO^T, Q^T are read in that order with
//    ds_read_b64_tr_b16 (the forward's P V mapping with rows for keys);
//  * each step's Q and dO are copied from memory straight into LDS twice,
//    once XOR-swizzled for the row reads and once for the transposing reads
//    (the forward kernel's conflict-free swizzles), together with the
//    step's 64 (L2, D) pairs; three stages, each filled two steps ahead of
//    its use, one barrier per step.
// Schedule: under the causal mask, with more blocks than the GPU holds
// workgroups at once, the grid is persistent and a workgroup walks pairs of
// blocks, k and nblk - 1 - k, whose steps add up to the same count for every
// k; the copies of a block's first two steps are issued during the last two
// steps of the block before, and its K and V operands are loaded into a
// second register set during the first step of the block before, so a
// block starts without waiting on memory.  Otherwise each block has a
// workgroup.
// Under the causal mask (query i at position Nk - N + i) the walk starts at
// the first row that sees the block's first key, a wave skips the steps in
// which none of its keys is visible, and only steps that straddle the
// diagonal pay for the mask.  Rows past N and keys past Nk read as zeros,
// which contribute nothing (dO = 0 and dS = 0 there), and are not stored.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_mfma32.h"

namespace fa {
namespace {

using namespace mfma32;

// Checking build (FA_SERIAL_COPIES=1): each step's copies are issued between
// two barriers and waited for before anyone reads them, so no copy is in
// flight while LDS is read.  The arithmetic and its order are unchanged, so
// this build's gradients must equal the pipelined build's bit for bit; only
// the race-check tests load it.
#ifndef FA_SERIAL_COPIES
#define FA_SERIAL_COPIES 0
#endif
constexpr bool kSerialCopies = FA_SERIAL_COPIES != 0;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kKW = 32;                  // keys per wave
constexpr int kBK = kWaves * kKW;        // keys per workgroup
constexpr int kSB = 32;                  // query rows per sub-block (one 32x32 product)

template <typename T, int D, int DV>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_mfma32_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ ws, const T *__restrict__ dout, T *__restrict__ dk,
    T *__restrict__ dvo, int N, int Nk, int off_c, float c, float scale, int heads, int paired) {
    typedef typename Mfma<T>::vec vec8;
    static_assert((D == 64 || D == 128) && (DV == 64 || DV == 128), "(d, dv)");
    constexpr int KS = D / 16;               // 16-wide contraction steps of S (over d)
    constexpr int KSV = DV / 16;             // ... of dP (over dv)
    constexpr int DBK = D / 32;              // 32-row blocks of dK^T
    constexpr int DBV = DV / 32;             // 32-row blocks of dV^T
    // Query rows per step (one barrier each): two sub-blocks, or one where
    // three stages of two would not fit in LDS.
    constexpr int QS = (D == 128 && DV == 128) ? 32 : 64;
    constexpr int NSB = QS / kSB;
    constexpr int ROWQ = 2 * D, ROWO = 2 * DV;   // bytes per Q / dO row
    constexpr int CPRQ = ROWQ / 16, CPRO = ROWO / 16;
    constexpr int TQ = QS * ROWQ, TO = QS * ROWO;     // bytes of one copy of a step's Q / dO
    constexpr int IQ = TQ / 1024, IO = TO / 1024;     // 1 KiB wave copies per Q / dO copy
    constexpr int NI = 2 * IQ + 2 * IO;               // wave copies per step
    static_assert(NI % kWaves == 0, "copies split evenly over the waves");
    constexpr int LPW = NI / kWaves;                  // per wave per step
    // LDS layout by copy: the three stages of the (L2[QS], D[QS]) strip, then
    // of the Q row-major copy, of the Q transposing copy, of dO row-major and
    // of dO transposing.  A read's address is a per-lane register (copy base
    // + lane offset) plus an immediate (stage, sub-block, step offsets),
    // which stays below the 64 KiB reach of the LDS instructions' offset.
    constexpr int TL = 2 * QS * 4;                    // bytes of one (L2, D) strip
    constexpr int OLD = 0;
    constexpr int OQA = 3 * TL, OQT = OQA + 3 * TQ, OOA = OQA + 6 * TQ, OOT = OOA + 3 * TO;
    constexpr int LDS_BYTES = OOA + 6 * TO;
    static_assert(2 * (TQ > TO ? TQ : TO) + kSB * 2 * (D > DV ? D : DV) < 65536, "immediate reach");
    constexpr int NLD = 2 * QS / 64;                  // 4-byte wave copies of the (L2, D) strip
    __shared__ __attribute__((aligned(16))) unsigned char sbuf[LDS_BYTES];

    // LDS past the step stages: each wave's slice for its 32 output rows.
    constexpr int OUTW = 2 * (D > DV ? D : DV) * kKW;  // bytes per wave slice
    __shared__ __attribute__((aligned(16))) unsigned char obuf[kWaves * OUTW];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;
    const int n = lane % 32;
    const int h = lane / 32;

    // ---- schedule ---------------------------------------------------------------
    // Persistent: workgroup g walks units g, g + G, ...  When `paired`, a
    // unit is a pair of key blocks of one head, k and nblk - 1 - k (the
    // middle block alone when nblk is odd): under the causal mask their
    // query steps add up to the same total for every k, so units cost the
    // same.  Otherwise a unit is one key block.  When G and the head count
    // are multiples of 8, units are numbered so that the workgroups of one
    // XCD (ids congruent mod 8) work on the same heads at the same time and
    // share their Q and dO through its L2.
    const int nblk = (Nk + kBK - 1) / kBK;
    const int U = paired ? (nblk + 1) / 2 : nblk;
    const int n_units = heads * U;
    const int G = gridDim.x;
    const bool xcd_map = (G % 8 == 0) && (heads % 8 == 0);
    const int qsteps = (N + QS - 1) / QS;
    struct Item {
        int t, half;              // unit round and which block of the pair
        int head, j0, s0, nsteps; // head < 0: past the end
    };
    auto locate = [&](Item it) __attribute__((always_inline)) {
        const int u = (int)blockIdx.x + it.t * G;
        if (u >= n_units) {
            it.head = -1;
            it.nsteps = 0;
            return it;
        }
        int pair;
        if (xcd_map) {
            const int local = u / 8;
            it.head = (local / U) * 8 + u % 8;
            pair = local % U;
        } else {
            it.head = u / U;
            pair = u % U;
        }
        const int kblk = it.half == 0 ? pair : nblk - 1 - pair;
        it.j0 = kblk * kBK;
        // Steps over query rows, from the first row that sees key j0.
        it.s0 = max(0, it.j0 - off_c) / QS;
        it.nsteps = max(0, qsteps - it.s0);
        return it;
    };
    auto next_item = [&](Item it) __attribute__((always_inline)) {
        const int pair = it.half == 0 ? it.j0 / kBK : nblk - 1 - it.j0 / kBK;
        if (paired && it.half == 0 && nblk - 1 - pair != pair) {
            it.half = 1;
        } else {
            it.t += 1;
            it.half = 0;
        }
        return locate(it);
    };

    // Memory-to-LDS copies.  Copy i of a step (i = t kWaves + wave) writes
    // 1 KiB of the stage; lane l's 16 bytes land at offset 16 l of it, so the
    // swizzled layouts come from the choice of source piece per lane.  Which
    // tensor and layout a copy has depends only on i, so it is uniform per
    // wave.
    uint32_t goff[LPW], loff[LPW], tstride[LPW];
    bool isq[LPW];
#pragma unroll
    for (int t = 0; t < LPW; ++t) {
        const int i = t * kWaves + wave;
        int x, part, W, CPR, base;
        bool tr;
        if (i < IQ) { x = 0; part = i; }
        else if (i < 2 * IQ) { x = 1; part = i - IQ; }
        else if (i < 2 * IQ + IO) { x = 2; part = i - 2 * IQ; }
        else { x = 3; part = i - 2 * IQ - IO; }
        isq[t] = x < 2;
        tr = x == 1 || x == 3;
        W = isq[t] ? D : DV;
        CPR = isq[t] ? CPRQ : CPRO;
        base = x == 0 ? OQA : x == 1 ? OQT : x == 2 ? OOA : OOT;
        const int slot = part * 64 + lane;
        const int row = slot / CPR, pc = slot % CPR;
        int src;
        if (W == 64) src = tr ? ((2 * pc) ^ vswz<64>(row)) / 2 : pc ^ kswz<64>(row);
        else src = tr ? ((2 * pc) ^ vswz<128>(row)) / 2 : pc ^ kswz<128>(row);
        goff[t] = ((uint32_t)row * W + src * 8) * 2u;
        loff[t] = base + part * 1024;
        tstride[t] = isq[t] ? TQ : TO;
    }
    // The (L2, D) strip, L2 of the step's rows then their D: element
    // e = 64 wave + lane (waves 0 .. NLD-1) is the pair member e / QS of row
    // e % QS.
    const uint32_t ldoff = (uint32_t)(((wave * 64 + lane) % QS) * 2 + (wave * 64 + lane) / QS) * 4u;

    // Per-lane LDS read offsets within a stage.
    //  row reads (A of S and dP): row n, 16-byte chunk 2 ks + h (swizzled);
    //  transposing reads (A of dV^T and dK^T, per 16-lane group G = lane/16):
    //    row 4h + (lane%16)/4 (+8, +16 kk), quad 8 db + 4 (G%2) + lane%4.
    uint32_t aq[KS], ao[KSV], tq[DBK], to[DBV];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) aq[ks] = OQA + n * ROWQ + (((2 * ks + h) ^ kswz<D>(n)) * 16);
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) ao[ks] = OOA + n * ROWO + (((2 * ks + h) ^ kswz<DV>(n)) * 16);
    {
        const int li = lane % 16;
        const int r0 = 4 * h + li / 4;
#pragma unroll
        for (int db = 0; db < DBK; ++db) {
            const int u = 8 * db + 4 * ((lane / 16) % 2) + li % 4;
            tq[db] = OQT + r0 * ROWQ + ((u ^ vswz<D>(r0)) * 8);
        }
#pragma unroll
        for (int db = 0; db < DBV; ++db) {
            const int u = 8 * db + 4 * ((lane / 16) % 2) + li % 4;
            to[db] = OOT + r0 * ROWO + ((u ^ vswz<DV>(r0)) * 8);
        }
    }

    typedef __attribute__((address_space(3))) void lds_void;
    const uint32_t lds0 = (uint32_t)(size_t)(lds_void *)&sbuf[0];
    // Copies issued by this wave per step.
    const int per_step = LPW + (wave < NLD ? 1 : 0);
    // Steps are copied in the order they are consumed, across items, into
    // stages 0, 1, 2, 0, ...: `con` counts the steps consumed, so a step's
    // stage is its position in that stream mod 3.
    // Every vector-memory operation before an item's first step has
    // completed when it starts (the wait after its operand loads); inside
    // the item the only ones are copies, which complete in issue order, so
    // the wait before step s leaves outstanding what the step before issued
    // (`prev` operations: the copies of step s + 1, or of the next item's
    // first steps) and nothing else.
    // (the counters travel as arguments and are written once per step, not
    // in branches: captured by reference, or stored on some paths only,
    // they would stay in memory)
    struct Counts {
        int con, prev, nissued, pf;
    } ps = {0, 0, 0, 0};
    // Buffer resources of one head's Q, dO and (L2, D) pairs.
    struct Src {
        u32x4 qw, ow, lw;
    };
    auto src_of = [=](int head_) __attribute__((always_inline)) {
        Src w;
        w.qw = rsrc_words(q + (int64_t)head_ * N * D, (uint32_t)N * D * 2u);
        w.ow = rsrc_words(dout + (int64_t)head_ * N * DV, (uint32_t)N * DV * 2u);
        w.lw = rsrc_words(ws + (int64_t)head_ * N * 2, (uint32_t)N * 8u);
        return w;
    };
    auto issue = [=](const Src &w, int s0_, int s, int stage) __attribute__((always_inline)) {
        const uint32_t row0 = (uint32_t)__builtin_amdgcn_readfirstlane((s0_ + s) * QS);
#pragma unroll
        for (int t = 0; t < LPW; ++t)
            lds_dma16(isq[t] ? u32x4(w.qw) : u32x4(w.ow), __builtin_amdgcn_readfirstlane(lds0 + loff[t] + stage * tstride[t]),
                      row0 * (isq[t] ? D : DV) * 2u + goff[t]);
        if (wave < NLD)
            lds_dma4(w.lw, __builtin_amdgcn_readfirstlane(lds0 + OLD + stage * TL + wave * 256),
                     row0 * 8u + ldoff);
    };
    auto consumed = [](Counts &c_) __attribute__((always_inline)) { ++c_.con; };
    auto barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // K^T and V^T B operands of an item: lane holds row j0 + 32 wave + n,
    // columns 16 ks + 8h .. +7.
    auto load_kv = [&](int head_, int j0_, vec8 (&ko)[KS], vec8 (&vo)[KSV]) __attribute__((always_inline)) {
        const int key = j0_ + wave * kKW + n;
        const auto krs = make_rsrc(k + (int64_t)head_ * Nk * D, (uint32_t)Nk * D * 2u);
        const auto vrs = make_rsrc(v + (int64_t)head_ * Nk * DV, (uint32_t)Nk * DV * 2u);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            ko[ks] = __builtin_bit_cast(vec8, buffer_load16(krs, ((uint32_t)key * D + ks * 16 + 8 * h) * 2u));
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks)
            vo[ks] = __builtin_bit_cast(vec8, buffer_load16(vrs, ((uint32_t)key * DV + ks * 16 + 8 * h) * 2u));
    };

    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    auto tr_read = [&](const unsigned char *p, int rowb) __attribute__((always_inline)) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 8 * rowb));
        return __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    vec8 kop[KS], vop[KSV];
    vec8 kon[KS], von[KSV];   // the next item's, fetched during the item's first step
    f32x16 dka[DBK], dva[DBV];
    int kw0 = 0, key = 0;

    // Sub-block `sbk` (rows i0 .. i0 + 31, i0 = first row of the step + 32 sbk)
    // of the step in stage `stage`.
    auto sub = [&](int i0, auto SBK, int stage) __attribute__((always_inline)) {
        constexpr int sbk = decltype(SBK)::value;
        if (kw0 > off_c + i0 + kSB - 1) return;   // no row of the sub-block sees the wave's keys
        const unsigned char *sb = sbuf + stage * TQ + sbk * kSB * ROWQ;   // Q copies
        const unsigned char *so = sbuf + stage * TO + sbk * kSB * ROWO;   // dO copies
        const unsigned char *sl = sbuf + OLD + stage * TL + sbk * kSB * 4;   // (L2, D)
        // All of the step's row-read operands and the lane's 16 (L2, D)
        // pairs are read first, so that the products below wait on LDS once.
        typedef float f4 __attribute__((ext_vector_type(4)));
        vec8 qa[KS], oa[KSV];
        f4 L4[4], D4[4];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[ks] = *reinterpret_cast<const vec8 *>(sb + aq[ks]);
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) oa[ks] = *reinterpret_cast<const vec8 *>(so + ao[ks]);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            L4[a] = *reinterpret_cast<const f4 *>(sl + (8 * a + 4 * h) * 4);
            D4[a] = *reinterpret_cast<const f4 *>(sl + QS * 4 + (8 * a + 4 * h) * 4);
        }
        // S and dP as two interleaved accumulation chains.
        f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
        for (int ks = 0; ks < (KS > KSV ? KS : KSV); ++ks) {
            if (ks < KS) S = Mfma<T>::run(qa[ks], kop[ks], S);
            if (ks < KSV) dP = Mfma<T>::run(oa[ks], vop[ks], dP);
        }
        // The scores of the keys a row does not see become -inf, so that
        // their P = 2^(-inf) and dS = P (dP - D) are exactly 0 (dP and D are
        // finite).  Register 4a + b is row 8a + 4h + b, which sees `key` iff
        // 8a + b >= u.  Only a step that straddles the diagonal masks.
        if (kw0 + kKW - 1 > off_c + i0) {
            const int u = key - off_c - i0 - 4 * h;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    S[4 * a + b] = 8 * a + b < u ? -INFINITY : S[4 * a + b];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int r = 4 * a + b;
                const float p = fast_exp2(fmaf(S[r], c, -L4[a][b]));
                S[r] = p;
                dP[r] = p * (dP[r] - D4[a][b]);
            }
#pragma unroll
        for (int kk = 0; kk < kSB / 16; ++kk) {
            f32x8 pf, df;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pf[e] = S[8 * kk + e];
                df[e] = dP[8 * kk + e];
            }
            const vec8 pb = __builtin_convertvector(pf, vec8);
            const vec8 db8 = __builtin_convertvector(df, vec8);
#pragma unroll
            for (int db = 0; db < DBV; ++db)
                dva[db] = Mfma<T>::run(tr_read(so + kk * 16 * ROWO + to[db], ROWO), pb, dva[db]);
#pragma unroll
            for (int db = 0; db < DBK; ++db)
                dka[db] = Mfma<T>::run(tr_read(sb + kk * 16 * ROWQ + tq[db], ROWQ), db8, dka[db]);
        }
    };

    auto compute = [&](int s0_, int s, int stage) __attribute__((always_inline)) {
        sub((s0_ + s) * QS, std::integral_constant<int, 0>{}, stage);
        if constexpr (NSB == 2) sub((s0_ + s) * QS + kSB, std::integral_constant<int, 1>{}, stage);
    };

    // dK = scale (dK^T)^T and dV of an item leave through the wave's slice of
    // obuf: register r of block db holds column 32 db + 8 (r/4) + 4h + r%4 of
    // key n; the wave writes its 32 rows (8-byte pieces, quads XOR-swizzled
    // by the row so that one column's writes spread over the banks), reads
    // them back 16 bytes per lane in row order and stores whole rows
    // (bounds-checked: keys past Nk dropped).  Only this wave uses its slice.
    auto store = [&](int head_, const auto &acc, auto WC, float mul, T *dst) __attribute__((always_inline)) {
        constexpr int W = decltype(WC)::value;
        constexpr int NB = W / 32, ROWB = 2 * W, CPR = ROWB / 16;
        typedef T t4 __attribute__((ext_vector_type(4)));
        unsigned char *buf = obuf + wave * OUTW;
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                t4 x;
#pragma unroll
                for (int b = 0; b < 4; ++b) x[b] = static_cast<T>(acc[db][4 * a + b] * mul);
                const int u = (8 * db + 2 * a + h) ^ (2 * (n & 7));
                *reinterpret_cast<t4 *>(buf + n * ROWB + u * 8) = x;
            }
        const auto rs = make_rsrc(dst + (int64_t)head_ * Nk * W, (uint32_t)Nk * W * 2u);
#pragma unroll
        for (int t = 0; t < kKW * CPR / 64; ++t) {
            const int ch = t * 64 + lane;
            const int r = ch / CPR, pc = ch % CPR;
            const u32x4 x = *reinterpret_cast<const u32x4 *>(buf + r * ROWB + ((2 * pc) ^ (2 * (r & 7))) * 8);
            __builtin_amdgcn_raw_buffer_store_b128(x, rs, (int)((uint32_t)(kw0 + r) * ROWB + pc * 16), 0, 2);
        }
    };

    // ---- the walk ---------------------------------------------------------------
    // At step s of an item, after the barrier (every wave is past the step
    // before, whose stage is the one two steps ahead fills), the wave issues
    // the copies of the step two ahead in the stream, which is the next
    // item's step 0 or 1 near an item's end; before the barrier it waits
    // until only the copies issued after this step's are outstanding.  The
    // next item's first two steps that were not fetched ahead are fetched
    // when it starts, and waited for there.  Its K and V operands are
    // loaded in the first step of the item before (`pf`: NPF loads, issued
    // before that step's copies, so they may stay outstanding through the
    // next step's wait and have landed by the one after).  (Leaving the
    // item before's output stores outstanding at an item's start as well
    // measured slower.)
    constexpr int NPF = KS + KSV;
    auto wait_prev = [&](int prev, int pf) __attribute__((always_inline)) {
        if (prev == 0) {
            if (pf == 0) wait_vmcnt<0>();
            else wait_vmcnt<NPF>();
        } else if (pf == 0) {
            if (wave < NLD) wait_vmcnt<LPW + 1>();
            else wait_vmcnt<LPW>();
        } else {
            if (wave < NLD) wait_vmcnt<LPW + 1 + NPF>();
            else wait_vmcnt<LPW + NPF>();
        }
    };
    auto start = [&](const Item &it, bool prefetched) __attribute__((always_inline)) {
        if (prefetched) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kop[ks] = kon[ks];
#pragma unroll
            for (int ks = 0; ks < KSV; ++ks) vop[ks] = von[ks];
        } else {
            load_kv(it.head, it.j0, kop, vop);
        }
        wait_vmcnt<0>();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(kop[ks]));
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) asm volatile("" : "+v"(vop[ks]));
    };
    Item cur;
    cur.t = 0;
    cur.half = 0;
    cur = locate(cur);
    if (cur.head < 0) return;
    {
        const Src w = src_of(cur.head);
        if (!kSerialCopies)
            for (int s = 0; s < 2 && s < cur.nsteps; ++s) issue(w, cur.s0, s, s);
        start(cur, false);
    }
    for (;;) {
        const Item nxt = next_item(cur);
        const Src cw = src_of(cur.head);
        ps.prev = 0;
        ps.pf = 0;
        ps.nissued = 0;   // steps of nxt already fetched
        kw0 = cur.j0 + wave * kKW;
        key = kw0 + n;
#pragma unroll
        for (int db = 0; db < DBK; ++db) dka[db] = f32x16{};
#pragma unroll
        for (int db = 0; db < DBV; ++db) dva[db] = f32x16{};
        // One step in stage ST (a compile-time constant, so that every LDS
        // address of the step is an immediate offset); the stage cycles
        // 0, 1, 2 in the order of the stream.
        auto step = [&](Counts &ps_, const Item cur_, const Item nxt_, int s, auto ST) __attribute__((always_inline)) {
            constexpr int st = decltype(ST)::value;
            if (kSerialCopies) {
                barrier();
                issue(cw, cur_.s0, s, st);
                wait_vmcnt<0>();
                barrier();
            } else {
                wait_prev(ps_.prev, ps_.pf);
                barrier();
                const bool pf = s == 0 && nxt_.head >= 0;
                if (pf) {
                    int hd = nxt_.head, j0n = nxt_.j0;
                    asm volatile("" : "+s"(hd), "+s"(j0n));
                    load_kv(hd, j0n, kon, von);
                }
                ps_.pf = pf ? 1 : 0;
                const int jn = s + 2 - cur_.nsteps;   // >= 0: the next item's step
                const bool ahead_next = jn >= 0 && nxt_.head >= 0 && jn == ps_.nissued && jn < nxt_.nsteps;
                if (jn < 0) {
                    issue(cw, cur_.s0, s + 2, (st + 2) % 3);
                } else if (ahead_next) {
                    // (an opaque copy keeps the compiler from holding the
                    // next head's resources across the whole loop)
                    int hd = nxt_.head;
                    asm volatile("" : "+s"(hd));
                    issue(src_of(hd), nxt_.s0, jn, (st + 2) % 3);
                }
                ps_.nissued += ahead_next ? 1 : 0;
                ps_.prev = jn < 0 || ahead_next ? per_step : 0;
            }
            compute(cur_.s0, s, st);
            consumed(ps_);
        };
        typedef std::integral_constant<int, 0> S0;
        typedef std::integral_constant<int, 1> S1;
        typedef std::integral_constant<int, 2> S2;
        // The item's first steps up to the next stage 0, then steps in
        // threes (stages 0, 1, 2), then the last one or two.
        const int n_ = cur.nsteps, ph = ps.con % 3;
        int s = 0;
        if (ph == 1 && s < n_) step(ps, cur, nxt, s++, S1{});
        if (ph >= 1 && s < n_) step(ps, cur, nxt, s++, S2{});
        for (; s + 3 <= n_; s += 3) {
            step(ps, cur, nxt, s, S0{});
            step(ps, cur, nxt, s + 1, S1{});
            step(ps, cur, nxt, s + 2, S2{});
        }
        if (s < n_) step(ps, cur, nxt, s, S0{});
        if (s + 1 < n_) step(ps, cur, nxt, s + 1, S1{});
        store(cur.head, dka, std::integral_constant<int, D>{}, scale, dk);
        store(cur.head, dva, std::integral_constant<int, DV>{}, 1.f, dvo);
        if (nxt.head < 0) break;
        const Src nw = src_of(nxt.head);
        if (!kSerialCopies)
            for (int s = ps.nissued; s < 2 && s < nxt.nsteps; ++s) issue(nw, nxt.s0, s, (ps.con + s) % 3);
        start(nxt, !kSerialCopies && cur.nsteps > 0);
        cur = nxt;
    }
}

// Resident workgroups of one instantiation on the current device (cached).
template <typename T, int D, int DV>
int resident_workgroups() {
    static int cache[64];
    return resident_workgroups_of(reinterpret_cast<const void *>(&bwd_dkdv_mfma32_kernel<T, D, DV>),
                                  kThreads, cache);
}

template <typename T, int D, int DV>
hipError_t launch(const BwdArgs &b) {
    const FwdArgs &a = b.a;
    const unsigned heads = (unsigned)(a.B * a.H);
    const int off_c = a.causal ? (int)(a.Nk - a.N) : (int)a.Nk;
    const int64_t nblk = (a.Nk + kBK - 1) / kBK;
    const int resident = resident_workgroups<T, D, DV>();
    if (resident <= 0) return hipErrorInvalidDevice;
    // Under the causal mask: pairs of blocks, where there are more blocks
    // than resident workgroups, and a persistent grid.  Without it every
    // block costs the same, and one workgroup per block measured faster
    // than walking them.
    const int paired = a.causal && (int64_t)heads * nblk > resident ? 1 : 0;
    const int64_t units = (int64_t)heads * (paired ? (nblk + 1) / 2 : nblk);
    const dim3 grid((unsigned)(a.causal && units > resident ? resident : units));
    hipLaunchKernelGGL((bwd_dkdv_mfma32_kernel<T, D, DV>), grid, dim3(kThreads), 0, a.stream,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), b.Dsum, static_cast<const T *>(b.dout),
                       static_cast<T *>(b.dk), static_cast<T *>(b.dv), (int)a.N, (int)a.Nk, off_c,
                       a.scale * kLog2e, a.scale, (int)heads, paired);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const BwdArgs &b) {
    const int64_t d = b.a.d, dv = b.a.dv;
    if (d == 64 && dv == 64) return launch<T, 64, 64>(b);
    return hipErrorInvalidValue;
}

}  // namespace

bool bwd_dkdv_mfma32_supported(int dtype, int64_t d, int64_t dv) {
    return (dtype == kBF16 || dtype == kF16) && d == 64 && dv == 64;
}

// Under the causal mask with fewer 256-key blocks than resident workgroups
// the 16-key kernel of fa_bwd_mfma.hip, whose blocks are half as long, keeps
// more of the GPU busy (B1 x H16 x 1024: 47 us against 54 us).
bool bwd_dkdv_mfma32_preferred(const BwdArgs &b) {
    const FwdArgs &a = b.a;
    if (!bwd_dkdv_mfma32_supported(a.dtype, a.d, a.dv)) return false;
    if (!a.causal) return true;
    const int resident = a.dtype == kBF16 ? resident_workgroups<bf16_t, 64, 64>()
                                          : resident_workgroups<f16_t, 64, 64>();
    return a.B * a.H * ((a.Nk + kBK - 1) / kBK) >= resident;
}

hipError_t launch_bwd_dkdv_mfma32(const BwdArgs &b) {
    if (!bwd_dkdv_mfma32_supported(b.a.dtype, b.a.d, b.a.dv)) return hipErrorInvalidValue;
    return b.a.dtype == kBF16 ? launch_t<bf16_t>(b) : launch_t<f16_t>(b);
}

}  // namespace fa
