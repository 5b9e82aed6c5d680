// fa_bwd_dq_mfma32.hip -- the dQ half of the attention backward on the
// CDNA4 32x32x16 matrix-core instruction (bf16/fp16 inputs, fp32
// accumulation), d = dv in {64, 128} and d = 64 with dv = 128.
//
// Method: CS349E Lecture 11 "flash_lab.py", section 3 (flash_bwd, the
// FlashAttention-2 backward), the query-block side: a block of query rows
// keeps its dQ accumulators on chip while the keys stream past; for each
// key block the probabilities are recomputed from Q, K and the forward's
// LSE, P = exp(S scale - LSE), and with the row dots D_i = rowsum(dO o O):
//     dP = dO V^T,  dS = P o (dP - D),  dQ += dS K (x scale).
// This kernel runs first: it also computes D_i from the dO and O rows it
// loads anyway and writes, per query row, L2 = LSE log2(e) (+inf for a row
// that sees no key) and D into the workspace for the dK/dV kernel.
//
// gfx950 mapping (the forward's 32x32 kernel with keys and rows of the
// score block exchanged, as the dK/dV kernel of fa_bwd_mfma32.hip has them
// the other way round): a workgroup of 8 waves owns a block of 256 query
// rows of one head at a time, 32 per wave as the columns of 32x32 blocks;
// two waves per SIMD.  The wave's Q and dO rows are B operands held in
// registers for the whole block, and its rows' L2 and D one register each.
// The walk goes over the keys in steps of 64 (two 32-key sub-blocks; one at
// d = 128, where three stages of two would not fit in LDS):
//  * S^T = K Q^T and dP^T = V dO^T: K and V are A operands read row-major
//    from LDS; the 32x32 results give each lane one query row (lane % 32)
//    and 16 of the sub-block's keys, 8 (r/4) + 4h + r%4 for register r
//    (h = lane / 32);
//  * dS^T, rounded to the input type, is the B operand of dQ^T += K^T dS^T
//    straight from registers: eight consecutive result registers form the
//    B operand of one 16-key step once its contraction index is read as the
//    key order {4h..4h+3, 8+4h..8+4h+3}, and K^T is read in that order with
//    ds_read_b64_tr_b16 from a second, transposing-swizzled copy of K;
//  * each step's K (twice) and V are copied from memory straight into LDS,
//    three stages, each filled two steps ahead of its use, one barrier per
//    step.
// Schedule: with more blocks than the GPU holds workgroups at once, the
// grid is persistent and a workgroup walks several blocks (under the causal
// mask pairs of row blocks, p and nblk - 1 - p, whose key steps add up to
// the same count for every p); the copies of a block's first two steps are
// issued during the last two steps of the block before.
// Under the causal mask (query i at position Nk - N + i) a block walks the
// keys up to its last row's diagonal, a wave skips the sub-blocks in which
// none of its rows sees any key, and only sub-blocks that reach past a row's
// diagonal (or past Nk) pay for the mask.  Rows past N read as zeros and
// have L2 = +inf, so they contribute nothing, and are not stored.
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
constexpr int kQW = 32;                  // query rows per wave
constexpr int kBQ = kWaves * kQW;        // query rows per workgroup
constexpr int kSB = 32;                  // keys per sub-block (one 32x32 product)

template <typename T, int D, int DV>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_mfma32_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ lse, const T *__restrict__ dout, const T *__restrict__ o,
    float *__restrict__ ws, T *__restrict__ dq, int N, int Nk, int off_c, float c, float scale,
    int heads, int paired) {
    typedef typename Mfma<T>::vec vec8;
    static_assert(((D == 64 || D == 128) && DV == D) || (D == 64 && DV == 128), "(d, dv)");
    constexpr int KST = D == 64 ? 64 : 32;   // keys per step
    constexpr int KS = D / 16;               // 16-wide contraction steps of S^T (over d)
    constexpr int KSV = DV / 16;             // ... of dP^T (over dv)
    constexpr int DB = D / 32;               // 32-row blocks of dQ^T
    constexpr int NSB = KST / kSB;
    constexpr int ROWK = 2 * D, ROWV = 2 * DV;   // bytes per K / V row
    constexpr int CPRK = ROWK / 16, CPRV = ROWV / 16;
    constexpr int TK = KST * ROWK, TV = KST * ROWV;   // bytes of one copy of a step's K / V
    constexpr int IK = TK / 1024, IV = TV / 1024;     // 1 KiB wave copies per K / V copy
    constexpr int NI = 2 * IK + IV;                   // wave copies per step
    static_assert(NI % kWaves == 0, "copies split evenly over the waves");
    constexpr int LPW = NI / kWaves;                  // per wave per step
    // LDS layout by copy: the three stages of the K row-major copy, of the K
    // transposing copy and of V row-major.  A read's address is a per-lane
    // register (copy base + lane offset) plus an immediate (stage, sub-block
    // offsets) below the 64 KiB reach of the LDS instructions' offset.
    constexpr int OKA = 0, OKT = 3 * TK, OVA = 6 * TK;
    constexpr int LDS_BYTES = OVA + 3 * TV;
    static_assert(2 * (TK > TV ? TK : TV) + KST * ROWK < 65536, "immediate reach");
    __shared__ __attribute__((aligned(16))) unsigned char sbuf[LDS_BYTES];

    // LDS past the step stages: each wave's slice for its 32 output rows.
    constexpr int OUTW = 2 * D * kQW;   // bytes per wave slice
    __shared__ __attribute__((aligned(16))) unsigned char obuf[kWaves * OUTW];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;
    const int n = lane % 32;
    const int h = lane / 32;

    // ---- schedule ---------------------------------------------------------------
    // Persistent: workgroup g walks units g, g + G, ...  When `paired`, a
    // unit is a pair of row blocks of one head, p and nblk - 1 - p (the
    // middle block alone when nblk is odd): under the causal mask their key
    // steps add up to the same total for every p, so units cost the same.
    // Otherwise a unit is one row block.  When G and the head count are
    // multiples of 8, units are numbered so that the workgroups of one XCD
    // (ids congruent mod 8) work on the same heads at the same time and
    // share their K and V through its L2.
    const int nblk = (N + kBQ - 1) / kBQ;
    const int U = paired ? (nblk + 1) / 2 : nblk;
    const int n_units = heads * U;
    const int G = gridDim.x;
    const bool xcd_map = (G % 8 == 0) && (heads % 8 == 0);
    struct Item {
        int t, half;              // unit round and which block of the pair
        int head, i0, nsteps;     // head < 0: past the end
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
        const int qblk = it.half == 0 ? pair : nblk - 1 - pair;
        it.i0 = qblk * kBQ;
        // Key steps up to the block's last row's diagonal.
        const int key_end = min(Nk, off_c + min(it.i0 + kBQ, N));
        it.nsteps = key_end > 0 ? (key_end + KST - 1) / KST : 0;
        return it;
    };
    auto next_item = [&](Item it) __attribute__((always_inline)) {
        const int pair = it.half == 0 ? it.i0 / kBQ : nblk - 1 - it.i0 / kBQ;
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
    uint32_t goff[LPW], loff[LPW];
    bool isk[LPW];
#pragma unroll
    for (int t = 0; t < LPW; ++t) {
        const int i = t * kWaves + wave;
        int x, part;
        if (i < IK) { x = 0; part = i; }
        else if (i < 2 * IK) { x = 1; part = i - IK; }
        else { x = 2; part = i - 2 * IK; }
        isk[t] = x < 2;
        const bool tr = x == 1;
        const int W = isk[t] ? D : DV;
        const int CPR = isk[t] ? CPRK : CPRV;
        const int base = x == 0 ? OKA : x == 1 ? OKT : OVA;
        const int slot = part * 64 + lane;
        const int row = slot / CPR, pc = slot % CPR;
        const int src = tr ? ((2 * pc) ^ vswz<D>(row)) / 2 : pc ^ (isk[t] ? kswz<D>(row) : kswz<DV>(row));
        goff[t] = ((uint32_t)row * W + src * 8) * 2u;
        loff[t] = base + part * 1024;
    }

    // Per-lane LDS read offsets within a stage.
    //  row reads (A of S^T and dP^T): row n, 16-byte chunk 2 ks + h (swizzled);
    //  transposing reads (A of dQ^T, per 16-lane group G = lane/16):
    //    row 4h + (lane%16)/4 (+8, +16 kk), quad 8 db + 4 (G%2) + lane%4.
    uint32_t ak[KS], av[KSV], tk[DB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ak[ks] = OKA + n * ROWK + (((2 * ks + h) ^ kswz<D>(n)) * 16);
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) av[ks] = OVA + n * ROWV + (((2 * ks + h) ^ kswz<DV>(n)) * 16);
    {
        const int li = lane % 16;
        const int r0 = 4 * h + li / 4;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int u = 8 * db + 4 * ((lane / 16) % 2) + li % 4;
            tk[db] = OKT + r0 * ROWK + ((u ^ vswz<D>(r0)) * 8);
        }
    }

    typedef __attribute__((address_space(3))) void lds_void;
    const uint32_t lds0 = (uint32_t)(size_t)(lds_void *)&sbuf[0];
    // Copies issued by this wave per step.
    constexpr int per_step = LPW;
    // Steps are copied in the order they are consumed, across items, into
    // stages 0, 1, 2, 0, ...: `con` counts the steps consumed, so a step's
    // stage is its position in that stream mod 3.
    // Every vector-memory operation before an item's first step has
    // completed when it starts (the wait after its row loads); inside the
    // item the only ones are copies, which complete in issue order, so the
    // wait before step s leaves outstanding what the step before issued
    // (`prev` operations: the copies of step s + 1, or of the next item's
    // first steps) and nothing else.
    // (the counters travel as arguments and are written once per step, not
    // in branches: captured by reference, or stored on some paths only,
    // they would stay in memory)
    struct Counts {
        int con, prev, nissued;
    } ps = {0, 0, 0};
    // Buffer resources of one head's K and V.
    struct Src {
        u32x4 kw, vw;
    };
    auto src_of = [=](int head_) __attribute__((always_inline)) {
        Src w;
        w.kw = rsrc_words(k + (int64_t)head_ * Nk * D, (uint32_t)Nk * D * 2u);
        w.vw = rsrc_words(v + (int64_t)head_ * Nk * DV, (uint32_t)Nk * DV * 2u);
        return w;
    };
    auto issue = [=](const Src &w, int s, int stage) __attribute__((always_inline)) {
        const uint32_t key0 = (uint32_t)__builtin_amdgcn_readfirstlane(s * KST);
#pragma unroll
        for (int t = 0; t < LPW; ++t)
            lds_dma16(isk[t] ? u32x4(w.kw) : u32x4(w.vw),
                      __builtin_amdgcn_readfirstlane(lds0 + loff[t] + stage * (isk[t] ? TK : TV)),
                      key0 * (isk[t] ? D : DV) * 2u + goff[t]);
    };
    auto consumed = [](Counts &c_) __attribute__((always_inline)) { ++c_.con; };
    auto barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    vec8 qop[KS], dop[KSV];
    f32x16 dqa[DB];
    float lse2 = INFINITY, Drow = 0.f;
    int qw0 = 0;

    // Q^T and dO^T B operands of an item (lane: row qw0 + n, columns
    // 16 ks + 8h .. +7), the row's D from the same column slices of O
    // (summed over the two lane halves), and its L2; the (L2, D) pair goes
    // to the workspace for the dK/dV kernel.
    auto load_rows = [&](int head_, int i0_) __attribute__((always_inline)) {
        const int row = i0_ + wave * kQW + n;
        const auto qrs = make_rsrc(q + (int64_t)head_ * N * D, (uint32_t)N * D * 2u);
        const auto drs = make_rsrc(dout + (int64_t)head_ * N * DV, (uint32_t)N * DV * 2u);
        const auto ors = make_rsrc(o + (int64_t)head_ * N * DV, (uint32_t)N * DV * 2u);
        float dpart = 0.f;
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) {
            const uint32_t off = ((uint32_t)row * DV + ks * 16 + 8 * h) * 2u;
            dop[ks] = __builtin_bit_cast(vec8, buffer_load16(drs, off));
            const vec8 ov = __builtin_bit_cast(vec8, buffer_load16(ors, off));
#pragma unroll
            for (int j = 0; j < 8; ++j) dpart = fmaf(to_f32(ov[j]), to_f32(dop[ks][j]), dpart);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qop[ks] = __builtin_bit_cast(vec8, buffer_load16(qrs, ((uint32_t)row * D + ks * 16 + 8 * h) * 2u));
        Drow = dpart + swap32(dpart);
        lse2 = INFINITY;
        if (row < N) {
            const float L = lse[(int64_t)head_ * N + row];
            lse2 = L == -INFINITY ? INFINITY : L * kLog2e;
            if (h == 0) {
                ws[((int64_t)head_ * N + row) * 2] = lse2;
                ws[((int64_t)head_ * N + row) * 2 + 1] = Drow;
            }
        }
    };

    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    auto tr_read = [&](const unsigned char *p, int rowb) __attribute__((always_inline)) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 8 * rowb));
        return __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // Sub-block `sbk` (keys j0 .. j0 + 31, j0 = first key of the step + 32 sbk)
    // of the step in stage `stage`.
    auto sub = [&](int j0, auto SBK, int stage) __attribute__((always_inline)) {
        constexpr int sbk = decltype(SBK)::value;
        // no row of the wave sees a key of the sub-block (or it is past Nk,
        // or the wave's rows are past N)
        if (j0 >= Nk || j0 > off_c + qw0 + kQW - 1 || qw0 >= N) return;
        const unsigned char *sk = sbuf + stage * TK + sbk * kSB * ROWK;   // K copies
        const unsigned char *sv = sbuf + stage * TV + sbk * kSB * ROWV;   // V copy
        // All of the sub-block's row-read operands are read first, so that
        // the products below wait on LDS once.
        vec8 ka[KS], va[KSV];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ka[ks] = *reinterpret_cast<const vec8 *>(sk + ak[ks]);
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) va[ks] = *reinterpret_cast<const vec8 *>(sv + av[ks]);
        // S^T and dP^T as two interleaved accumulation chains.
        f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
        for (int ks = 0; ks < (KS > KSV ? KS : KSV); ++ks) {
            if (ks < KS) S = Mfma<T>::run(ka[ks], qop[ks], S);
            if (ks < KSV) dP = Mfma<T>::run(va[ks], dop[ks], dP);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(S[r], c, -lse2));
            dP[r] = p * (dP[r] - Drow);
        }
        // dS of the keys a row does not see (or past Nk) is set to 0 (after
        // the arithmetic, whose values there are meaningless and may be inf
        // or NaN).  Register 4a + b is key j0 + 8a + 4h + b, which row
        // qw0 + n sees iff 8a + b <= lim.  Only a sub-block that reaches
        // past some row's diagonal, or past Nk, masks.
        if (j0 + kSB - 1 > off_c + qw0 || j0 + kSB > Nk) {
            const int lim = min(off_c + qw0 + n, Nk - 1) - j0 - 4 * h;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    dP[4 * a + b] = 8 * a + b > lim ? 0.f : dP[4 * a + b];
        }
#pragma unroll
        for (int kk = 0; kk < kSB / 16; ++kk) {
            f32x8 df;
#pragma unroll
            for (int e = 0; e < 8; ++e) df[e] = dP[8 * kk + e];
            const vec8 db8 = __builtin_convertvector(df, vec8);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                dqa[db] = Mfma<T>::run(tr_read(sk + kk * 16 * ROWK + tk[db], ROWK), db8, dqa[db]);
        }
    };

    // A step whose 64 keys every row of the wave sees (the common case off
    // the diagonal): both sub-blocks' products S^T and dP^T are issued
    // before either's exponentials, in one straight-line block, so that the
    // second sub-block's products run on the matrix cores while the first
    // one's vector work issues.
    auto full_step = [&](int stage) __attribute__((always_inline)) {
        vec8 ka[NSB][KS], va[NSB][KSV];
        f32x16 S[NSB], dP[NSB];
#pragma unroll
        for (int b = 0; b < NSB; ++b) {
            const unsigned char *sk = sbuf + stage * TK + b * kSB * ROWK;
            const unsigned char *sv = sbuf + stage * TV + b * kSB * ROWV;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) ka[b][ks] = *reinterpret_cast<const vec8 *>(sk + ak[ks]);
#pragma unroll
            for (int ks = 0; ks < KSV; ++ks) va[b][ks] = *reinterpret_cast<const vec8 *>(sv + av[ks]);
        }
#pragma unroll
        for (int b = 0; b < NSB; ++b) {
            S[b] = f32x16{};
            dP[b] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < (KS > KSV ? KS : KSV); ++ks) {
                if (ks < KS) S[b] = Mfma<T>::run(ka[b][ks], qop[ks], S[b]);
                if (ks < KSV) dP[b] = Mfma<T>::run(va[b][ks], dop[ks], dP[b]);
            }
        }
#pragma unroll
        for (int b = 0; b < NSB; ++b) {
            const unsigned char *sk = sbuf + stage * TK + b * kSB * ROWK;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(S[b][r], c, -lse2));
                dP[b][r] = p * (dP[b][r] - Drow);
            }
#pragma unroll
            for (int kk = 0; kk < kSB / 16; ++kk) {
                f32x8 df;
#pragma unroll
                for (int e = 0; e < 8; ++e) df[e] = dP[b][8 * kk + e];
                const vec8 db8 = __builtin_convertvector(df, vec8);
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    dqa[db] = Mfma<T>::run(tr_read(sk + kk * 16 * ROWK + tk[db], ROWK), db8, dqa[db]);
            }
        }
    };

    auto compute = [&](int s, int stage) __attribute__((always_inline)) {
        const int j0 = s * KST;
        if (NSB == 2 && qw0 < N && j0 + KST <= Nk && j0 + KST - 1 <= off_c + qw0) {
            full_step(stage);
        } else {
            sub(j0, std::integral_constant<int, 0>{}, stage);
            if constexpr (NSB == 2) sub(j0 + kSB, std::integral_constant<int, 1>{}, stage);
        }
    };

    // dQ = scale (dQ^T)^T of an item leaves through the wave's slice of obuf:
    // register r of block db holds column 32 db + 8 (r/4) + 4h + r%4 of row
    // n; the wave writes its 32 rows (8-byte pieces, quads XOR-swizzled by
    // the row so that one column's writes spread over the banks), reads them
    // back 16 bytes per lane in row order and stores whole rows
    // (bounds-checked: rows past N dropped).  Only this wave uses its slice.
    auto store = [&](int head_) __attribute__((always_inline)) {
        constexpr int W = D;
        constexpr int NB = W / 32, ROWB = 2 * W, CPR = ROWB / 16;
        typedef T t4 __attribute__((ext_vector_type(4)));
        unsigned char *buf = obuf + wave * OUTW;
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                t4 x;
#pragma unroll
                for (int b = 0; b < 4; ++b) x[b] = static_cast<T>(dqa[db][4 * a + b] * scale);
                const int u = (8 * db + 2 * a + h) ^ (2 * (n & 7));
                *reinterpret_cast<t4 *>(buf + n * ROWB + u * 8) = x;
            }
        const auto rs = make_rsrc(dq + (int64_t)head_ * N * W, (uint32_t)N * W * 2u);
#pragma unroll
        for (int t = 0; t < kQW * CPR / 64; ++t) {
            const int ch = t * 64 + lane;
            const int r = ch / CPR, pc = ch % CPR;
            const u32x4 x = *reinterpret_cast<const u32x4 *>(buf + r * ROWB + ((2 * pc) ^ (2 * (r & 7))) * 8);
            __builtin_amdgcn_raw_buffer_store_b128(x, rs, (int)((uint32_t)(qw0 + r) * ROWB + pc * 16), 0, 2);
        }
    };

    // ---- the walk ---------------------------------------------------------------
    // At step s of an item, after the barrier (every wave is past the step
    // before, whose stage is the one two steps ahead fills), the wave issues
    // the copies of the step two ahead in the stream, which is the next
    // item's step 0 or 1 near an item's end; before the barrier it waits
    // until only the copies issued after this step's are outstanding.  The
    // next item's first two steps that were not fetched ahead, and its
    // rows, are fetched when it starts, and waited for there.
    auto wait_prev = [&](int prev) __attribute__((always_inline)) {
        if (prev == 0) wait_vmcnt<0>();
        else wait_vmcnt<LPW>();
    };
    auto start = [&](const Item &it) __attribute__((always_inline)) {
        load_rows(it.head, it.i0);
        wait_vmcnt<0>();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qop[ks]));
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) asm volatile("" : "+v"(dop[ks]));
        asm volatile("" : "+v"(lse2), "+v"(Drow));
    };
    Item cur;
    cur.t = 0;
    cur.half = 0;
    cur = locate(cur);
    if (cur.head < 0) return;
    {
        const Src w = src_of(cur.head);
        if (!kSerialCopies)
            for (int s = 0; s < 2 && s < cur.nsteps; ++s) issue(w, s, s);
        start(cur);
    }
    for (;;) {
        const Item nxt = next_item(cur);
        const Src cw = src_of(cur.head);
        ps.prev = 0;
        ps.nissued = 0;   // steps of nxt already fetched
        qw0 = cur.i0 + wave * kQW;
#pragma unroll
        for (int db = 0; db < DB; ++db) dqa[db] = f32x16{};
        // One step in stage ST (a compile-time constant, so that every LDS
        // address of the step is an immediate offset); the stage cycles
        // 0, 1, 2 in the order of the stream.
        auto step = [&](Counts &ps_, const Item cur_, const Item nxt_, int s, auto ST) __attribute__((always_inline)) {
            constexpr int st = decltype(ST)::value;
            if (kSerialCopies) {
                barrier();
                issue(cw, s, st);
                wait_vmcnt<0>();
                barrier();
            } else {
                wait_prev(ps_.prev);
                barrier();
                const int jn = s + 2 - cur_.nsteps;   // >= 0: the next item's step
                const bool ahead_next = jn >= 0 && nxt_.head >= 0 && jn == ps_.nissued && jn < nxt_.nsteps;
                if (jn < 0) {
                    issue(cw, s + 2, (st + 2) % 3);
                } else if (ahead_next) {
                    // (an opaque copy keeps the compiler from holding the
                    // next head's resources across the whole loop)
                    int hd = nxt_.head;
                    asm volatile("" : "+s"(hd));
                    issue(src_of(hd), jn, (st + 2) % 3);
                }
                ps_.nissued += ahead_next ? 1 : 0;
                ps_.prev = jn < 0 || ahead_next ? per_step : 0;
            }
            compute(s, st);
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
        store(cur.head);
        if (nxt.head < 0) break;
        const Src nw = src_of(nxt.head);
        if (!kSerialCopies)
            for (int s = ps.nissued; s < 2 && s < nxt.nsteps; ++s) issue(nw, s, (ps.con + s) % 3);
        start(nxt);
        cur = nxt;
    }
}

// Resident workgroups of one instantiation on the current device (cached).
template <typename T, int D, int DV>
int resident_workgroups() {
    static int cache[64];
    return resident_workgroups_of(reinterpret_cast<const void *>(&bwd_dq_mfma32_kernel<T, D, DV>),
                                  kThreads, cache);
}

template <typename T, int D, int DV>
hipError_t launch(const BwdArgs &b) {
    const FwdArgs &a = b.a;
    const unsigned heads = (unsigned)(a.B * a.H);
    const int off_c = a.causal ? (int)(a.Nk - a.N) : (int)a.Nk;
    const int64_t nblk = (a.N + kBQ - 1) / kBQ;
    const int resident = resident_workgroups<T, D, DV>();
    if (resident <= 0) return hipErrorInvalidDevice;
    // A persistent grid where there are more blocks than resident
    // workgroups, walking pairs of blocks under the causal mask.
    const int paired = a.causal && (int64_t)heads * nblk > resident ? 1 : 0;
    const int64_t units = (int64_t)heads * (paired ? (nblk + 1) / 2 : nblk);
    const dim3 grid((unsigned)(units > resident ? resident : units));
    hipLaunchKernelGGL((bwd_dq_mfma32_kernel<T, D, DV>), grid, dim3(kThreads), 0, a.stream,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), a.lse, static_cast<const T *>(b.dout),
                       static_cast<const T *>(a.o), b.Dsum, static_cast<T *>(b.dq), (int)a.N,
                       (int)a.Nk, off_c, a.scale * kLog2e, a.scale, (int)heads, paired);
    return hipGetLastError();
}

}  // namespace

bool bwd_dq_mfma32_supported(int dtype, int64_t d, int64_t dv) {
    return (dtype == kBF16 || dtype == kF16) &&
           ((d == dv && (d == 64 || d == 128)) || (d == 64 && dv == 128));
}

// Measured against the 16x16 dQ kernel of fa_bwd_mfma.hip (whole fa_bwd,
// bf16, paired HIP-event timings).  d = 64: 3.7% faster at causal
// B64 x H16 x 1024 and 4-5% at causal 2048 to 8192 rows, level or 1% slower
// at causal 512 and 1000 rows, slower below one block per resident
// workgroup (B1 x H16 x 1024: 56 against 47 us) and without the mask at
// 1024 rows (1124 against 1086 us).  d = 128, and d = 64 with dv = 128:
// 8-13% faster on every measured shape with at least one block per
// resident workgroup, with and without the mask, 512 to 8192 rows.
bool bwd_dq_mfma32_preferred(const BwdArgs &b) {
    const FwdArgs &a = b.a;
    if (!bwd_dq_mfma32_supported(a.dtype, a.d, a.dv)) return false;
    if (a.d == 64 && a.dv == 64 && (!a.causal || a.N < 1024)) return false;
    const bool bf = a.dtype == kBF16;
    const int resident =
        a.d == 128   ? (bf ? resident_workgroups<bf16_t, 128, 128>() : resident_workgroups<f16_t, 128, 128>())
        : a.dv == 128 ? (bf ? resident_workgroups<bf16_t, 64, 128>() : resident_workgroups<f16_t, 64, 128>())
                      : (bf ? resident_workgroups<bf16_t, 64, 64>() : resident_workgroups<f16_t, 64, 64>());
    return a.B * a.H * ((a.N + kBQ - 1) / kBQ) >= resident;
}

hipError_t launch_bwd_dq_mfma32(const BwdArgs &b) {
    if (!bwd_dq_mfma32_supported(b.a.dtype, b.a.d, b.a.dv)) return hipErrorInvalidValue;
    const bool bf = b.a.dtype == kBF16;
    if (b.a.d == 128) return bf ? launch<bf16_t, 128, 128>(b) : launch<f16_t, 128, 128>(b);
    if (b.a.dv == 128) return bf ? launch<bf16_t, 64, 128>(b) : launch<f16_t, 64, 128>(b);
    return bf ? launch<bf16_t, 64, 64>(b) : launch<f16_t, 64, 64>(b);
}

}  // namespace fa
