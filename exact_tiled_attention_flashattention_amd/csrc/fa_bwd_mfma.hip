// fa_bwd_mfma.hip -- attention backward on the CDNA4 matrix cores
// (bf16/fp16 inputs, d and dv in {32, 64, 128, 256}, fp32 accumulation).
//
// Method: CS349E Lecture 11 "flash_lab.py", section 3 (flash_bwd, the
// FlashAttention-2 backward).  The probabilities are recomputed from Q, K
// and the forward's LSE, P = exp(S - LSE) (here exp2 of S scale log2(e) -
// LSE log2(e)); with D_i = rowsum(dO o O) (computed by the dQ kernel, which
// runs first, from the dO rows it holds anyway):
//     dV += P^T dO,  dP = dO V^T,  dS = P o (dP - D),
//     dK += dS^T Q (times scale),  dQ += dS K (times scale).
// As in fa_bwd.hip the two halves run as separate kernels (no location is
// written by two workgroups; deterministic).
//
// All products use v_mfma_f32_16x16x32_{bf16,f16}; P and dS are rounded to
// the input type before the products that take them.  Lane layouts (lane l,
// g = l / 16, i = l % 16): A operand A[i][8g + j], B operand B[8g + j][i],
// result D[4g + r][i] in register r.
//
// dK/dV kernel: a workgroup of 8 waves owns 128 keys of one head, 16 per
// wave as the MFMA columns; it walks the head's query rows in steps of 32.
//  * S = Q K^T and dP = dO V^T per 16-row block: Q and dO are A operands
//    read row-major from LDS; K^T and V^T are B operands held in registers
//    for the whole walk (a lane's 16 bytes are one row of K or V).
//  * The two 16-row result blocks of S (rows 4g + r and 16 + 4g + r of the
//    lane's key) are a B operand over the row order {4g..4g+3,
//    16+4g..16+4g+3}; so dV^T += dO^T P and dK^T += Q^T dS take P and dS
//    straight from registers, and dO^T, Q^T are read in that order with
//    ds_read_b64_tr_b16.
//  * Q and dO of a step are stored twice in LDS, once swizzled for the
//    row-major reads and once for the transposing reads (each swizzle
//    conflict-free for its pattern, as in the forward kernels); LDS holds
//    two steps and each step's loads are issued two steps ahead.
// dQ kernel: a workgroup of 8 waves owns 128 query rows, 16 per wave as the
// MFMA columns, and walks the keys in tiles of 64 (computed transposed):
//  * S^T = K Q^T and dP^T = V dO^T with K and V row-major from LDS and Q^T,
//    dO^T in registers; each lane holds one query row, so LSE and D are
//    one register each;
//  * dQ^T += K^T dS^T with dS^T from registers (the same key-order trick)
//    and K^T read with ds_read_b64_tr_b16 from a second copy of the K tile.
// Workgroups of one head are placed on one XCD (see work_item) so that they
// share the head's tensors through its L2.
// Under the causal mask (query i at position Nk - N + i) each kernel walks
// only the blocks some of its rows or keys can see, and a wave skips the
// steps in which none of its own rows or keys is visible.  The kernels take
// the offset of that diagonal (off_c = Nk - N); without the mask they run
// with off_c = Nk, which makes every key visible to every row.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
    typedef bf16x8 vec;
    static __device__ __forceinline__ f32x4 run(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<f16_t> {
    typedef f16x8 vec;
    static __device__ __forceinline__ f32x4 run(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
// __launch_bounds__' second argument is the minimum waves per SIMD: 4 (two
// resident workgroups per CU, at most 128 registers) for d = 64, 2 for d = 128.

// LDS swizzles (the forward kernels' conflict-free ones; both have period 16
// in the row, so a 32- or 64-row tile repeats them).  Row-major copy: 16-byte
// chunk c of row r at chunk c ^ kswz(r), for reads of rows i, chunks 4 ks +
// g.  Transposing copy: 8-byte quad u of row r at quad u ^ vswz(r), for
// ds_read_b64_tr_b16 of rows 4g + i/4, quads 4 db + i%4.
template <int D> __device__ __forceinline__ int kswz(int r) {
    if constexpr (D == 64)
        return ((r >> 2) & 1) | ((__builtin_popcount(r & 15) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
    else if constexpr (D == 32) return r & 3;
    else return r & 15;
}
template <int D> __device__ __forceinline__ int vswz(int r) {
    if constexpr (D == 64) return 4 * ((r & 3) ^ ((r >> 2) & 1));
    else if constexpr (D == 32) return 0;
    else return 4 * (r & 7);
}

// This workgroup's (head, block) in a 1-D grid of nblk * heads workgroups.
// Workgroup ids are dealt to the 8 XCDs round-robin; when heads is a
// multiple of 8 the blocks of one head get ids congruent mod 8, so they run
// on one XCD and share the head's Q, dO (or K, V) through its L2.
__device__ __forceinline__ void work_item(int nblk, int heads, int &head, int &blk) {
    const int L = blockIdx.x;
    if (heads % 8 == 0) {
        const int local = L / 8;
        head = (local / nblk) * 8 + L % 8;
        blk = local % nblk;
    } else {
        head = L / nblk;
        blk = L % nblk;
    }
}

// Sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float rows4_sum(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = __int_as_float(a[0]) + __int_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(b[0]) + __int_as_float(b[1]);
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::vec as_vec(u32x4 x) {
    return __builtin_bit_cast(typename Mma<T>::vec, x);
}

// A operand of 16 rows x 32 columns from a row-major (kswz) LDS copy.
__device__ __forceinline__ u32x4 lds_row16(const unsigned char *base) {
    return *reinterpret_cast<const u32x4 *>(base);
}

// A operand of 16 columns x 32 rows (rows in the order {4g..4g+3,
// 16+4g..16+4g+3}) from a transposing (vswz) LDS copy; `p` is the lane's
// address in rows 0..15 of the 32-row block.
template <typename T, int ROWB>
__device__ __forceinline__ typename Mma<T>::vec lds_tr32(const unsigned char *p) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 16 * ROWB));
    return __builtin_bit_cast(typename Mma<T>::vec,
                              __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Two 16x16 result blocks (f32) -> one B operand in the input type.
template <typename T>
__device__ __forceinline__ typename Mma<T>::vec pack_b(f32x4 a, f32x4 b) {
    typename Mma<T>::vec r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        r[j] = static_cast<T>(a[j]);
        r[4 + j] = static_cast<T>(b[j]);
    }
    return r;
}

// Waves per SIMD the launch bounds ask for: 4 (two resident workgroups per
// CU, at most 128 registers) for the small head dimensions, 2 otherwise.
template <int D, int DV> constexpr int bwd_waves_per_simd() { return D + DV <= 128 ? 4 : 2; }

// =============================================================================
// dK, dV
// =============================================================================
template <typename T, int D, int DV>
__global__ __launch_bounds__(kThreads, (bwd_waves_per_simd<D, DV>())) void bwd_dkdv_mfma_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ lse, const T *__restrict__ dout, const float *__restrict__ Dsum,
    T *__restrict__ dk, T *__restrict__ dvo, int N, int Nk, int off_c, float c, float scale,
    int heads) {
    typedef typename Mma<T>::vec vec8;
    constexpr int KS = D / 32;              // contraction steps of S = Q K^T (over d)
    constexpr int KSV = DV / 32;            // contraction steps of dP = dO V^T (over dv)
    constexpr int DBK = D / 16;             // 16-column blocks of dK^T
    constexpr int DBV = DV / 16;            // 16-column blocks of dV^T
    constexpr int ROWQ = 2 * D, ROWO = 2 * DV;   // bytes per Q / dO row
    constexpr int CPRQ = ROWQ / 16, CPRO = ROWO / 16;
    constexpr int QS = 32;                  // query rows per step
    constexpr int TQ = QS * ROWQ, TO = QS * ROWO;   // bytes of one copy of a step's Q / dO
    constexpr int CHQ = QS * CPRQ, CHO = QS * CPRO; // 16-byte chunks of Q / dO per step
    constexpr int NL = (CHQ + CHO + kThreads - 1) / kThreads;   // chunks per thread per step

    // Per stage: Q row-major, Q transposing, dO row-major, dO transposing.
    __shared__ __attribute__((aligned(16))) unsigned char bq[2][2][TQ];
    __shared__ __attribute__((aligned(16))) unsigned char bo[2][2][TO];
    __shared__ float s_lse[2][QS];
    __shared__ float s_D[2][QS];

    int head, kblk;
    work_item((Nk + kWaves * 16 - 1) / (kWaves * 16), heads, head, kblk);
    const int j0 = kblk * (kWaves * 16);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;
    const int g = lane / 16;
    const int li = lane % 16;
    const int kw0 = j0 + wave * 16;
    const int key = kw0 + li;               // this lane's key (MFMA column)

    const T *qh = q + (int64_t)head * N * D;
    const T *dh = dout + (int64_t)head * N * DV;
    const float *Wh = Dsum + (int64_t)head * N * 2;   // (LSE log2 e, D) per row
    const auto qrs = make_rsrc(qh, (uint32_t)N * D * 2u);
    const auto drs = make_rsrc(dh, (uint32_t)N * DV * 2u);
    const auto krs = make_rsrc(k + (int64_t)head * Nk * D, (uint32_t)Nk * D * 2u);
    const auto vrs = make_rsrc(v + (int64_t)head * Nk * DV, (uint32_t)Nk * DV * 2u);

    // K^T and V^T B operands: lane holds the row of `key`, columns 32 ks + 8g .. +7.
    vec8 kop[KS], vop[KSV];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        kop[ks] = as_vec<T>(buffer_load16(krs, ((uint32_t)key * D + ks * 32 + 8 * g) * 2u));
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks)
        vop[ks] = as_vec<T>(buffer_load16(vrs, ((uint32_t)key * DV + ks * 32 + 8 * g) * 2u));

    // Steps over query rows, from the first row that sees key j0.
    const int first = max(0, j0 - off_c);
    const int s0 = first / QS;
    const int nsteps = (N + QS - 1) / QS - s0;

    // Per-thread load slots: chunk t * kThreads + tid of [Q chunks | dO chunks].
    // CHQ and CHQ + CHO are multiples of 64, so whether a slot is used and
    // which tensor it reads is the same for a whole wave: derived from the
    // wave index, the choice of buffer resource stays scalar.
    static_assert(CHQ % 64 == 0 && (CHQ + CHO) % 64 == 0, "wave-uniform chunk roles");
    uint32_t gofs[NL], wA[NL], wT[NL];
    bool isdo[NL], used[NL];
#pragma unroll
    for (int t = 0; t < NL; ++t) {
        const int cidx = t * kThreads + tid;
        const int cwave = t * kThreads + wave * 64;
        used[t] = cwave < CHQ + CHO;
        isdo[t] = cwave >= CHQ;
        if constexpr (D == DV) {   // one layout for both tensors
            // chunk (t kThreads + tid) mod CHQ: the part from t is zero or a
            // whole number of 16-row swizzle periods, so the offsets are
            // t = 0's plus a constant (fewer registers at d = 256)
            static_assert(CHQ <= kThreads ? kThreads % CHQ == 0
                                          : CHQ % kThreads == 0 && (kThreads / CPRQ) % 16 == 0,
                          "chunk offsets periodic in t");
            const int ch = tid % CHQ;
            const int row = ch / CPRQ, cc = ch % CPRQ;
            const uint32_t add = (uint32_t)(((t * kThreads) % CHQ) / CPRQ) * ROWQ;
            gofs[t] = ((uint32_t)row * D + cc * 8) * 2u + add;
            wA[t] = row * ROWQ + ((cc ^ kswz<D>(row)) * 16) + add;
            wT[t] = row * ROWQ + (((2 * cc) ^ vswz<D>(row)) * 8) + add;
            continue;
        }
        gofs[t] = wA[t] = wT[t] = 0;
        if (!used[t]) continue;
        if (!isdo[t]) {
            const int row = cidx / CPRQ, cc = cidx % CPRQ;
            gofs[t] = ((uint32_t)row * D + cc * 8) * 2u;
            wA[t] = row * ROWQ + ((cc ^ kswz<D>(row)) * 16);
            wT[t] = row * ROWQ + (((2 * cc) ^ vswz<D>(row)) * 8);
        } else {
            const int ch = cidx - CHQ;
            const int row = ch / CPRO, cc = ch % CPRO;
            gofs[t] = ((uint32_t)row * DV + cc * 8) * 2u;
            wA[t] = row * ROWO + ((cc ^ kswz<DV>(row)) * 16);
            wT[t] = row * ROWO + (((2 * cc) ^ vswz<DV>(row)) * 8);
        }
    }
    // Per-lane read offsets.
    // The swizzles flip at most the low 4 bits of a 16-byte chunk index and
    // the low 3 bits of a quad's 4-quad group, so past 16 chunks (4 read
    // steps) or 8 column blocks the offsets repeat 256 bytes further on:
    // only the first period is kept per lane (fewer registers at d = 256)
    // and the rest is an immediate.
    constexpr int NAQ = KS < 4 ? KS : 4, NAO = KSV < 4 ? KSV : 4;
    constexpr int NTQ = DBK < 8 ? DBK : 8, NTO = DBV < 8 ? DBV : 8;
    uint32_t rAq[NAQ], rAo[NAO], rTq[NTQ], rTo[NTO];
#pragma unroll
    for (int ks = 0; ks < NAQ; ++ks) rAq[ks] = li * ROWQ + (((ks * 4 + g) ^ kswz<D>(li)) * 16);
#pragma unroll
    for (int ks = 0; ks < NAO; ++ks) rAo[ks] = li * ROWO + (((ks * 4 + g) ^ kswz<DV>(li)) * 16);
    auto aq = [&](int ks) { return rAq[ks % NAQ] + (ks / NAQ) * 256; };
    auto ao = [&](int ks) { return rAo[ks % NAO] + (ks / NAO) * 256; };
    auto tq = [&](int db) { return rTq[db % NTQ] + (db / NTQ) * 256; };
    auto to = [&](int db) { return rTo[db % NTO] + (db / NTO) * 256; };
    const int r0 = 4 * g + li / 4;
#pragma unroll
    for (int db = 0; db < NTQ; ++db) rTq[db] = r0 * ROWQ + (((4 * db + li % 4) ^ vswz<D>(r0)) * 8);
#pragma unroll
    for (int db = 0; db < NTO; ++db) rTo[db] = r0 * ROWO + (((4 * db + li % 4) ^ vswz<DV>(r0)) * 8);

    // Steps are fetched two ahead: step x's data waits in register set x % 2
    // until it is stored to LDS stage x % 2 at the end of step x - 1.  The
    // step's (LSE log2 e, D) pairs are fetched the same way (bounds-checked:
    // rows past N read 0; wave 0 stores them), so that nothing waits on the
    // loads just issued.  Where the dK and dV accumulators leave no room for
    // two register sets (d + dv >= 384) steps are fetched one ahead through
    // one set, which is stored to LDS and then refilled after each barrier.
    constexpr bool kOneSet = D + DV >= 384;
    const auto wrs = make_rsrc(Wh, (uint32_t)N * 8u);
    u32x4 regs0[NL], regs1[kOneSet ? 1 : NL];
    float vl0 = 0.f, vd0 = 0.f, vl1 = 0.f, vd1 = 0.f;
    auto load_step = [&](u32x4 (&rg)[NL], float &vl, float &vd, int s) {   // global -> registers
        const uint32_t baseq = (uint32_t)((s0 + s) * QS) * D * 2u;
        const uint32_t baseo = (uint32_t)((s0 + s) * QS) * DV * 2u;
        // One load per slot with a (wave-uniform) choice of tensor; an unused
        // slot fetches a harmless chunk that is never stored.
#pragma unroll
        for (int t = 0; t < NL; ++t)
            rg[t] = buffer_load16(isdo[t] ? drs : qrs, (isdo[t] ? baseo : baseq) + gofs[t]);
        // (every wave issues these two small loads, so that the count of
        // loads per step, and with it every wait, is the same on all paths)
        const uint32_t off = (uint32_t)((s0 + s) * QS + lane % QS) * 8u;
        vl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wrs, (int)off, 0, 0));
        vd = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wrs, (int)off + 4, 0, 0));
    };
    auto store_step = [&](const u32x4 (&rg)[NL], float vl, float vd, int s, int st) {   // registers -> LDS
#pragma unroll
        for (int t = 0; t < NL; ++t) {
            if (!used[t]) continue;
            unsigned char *a = isdo[t] ? bo[st][0] : bq[st][0];
            unsigned char *b = isdo[t] ? bo[st][1] : bq[st][1];
            *reinterpret_cast<u32x4 *>(a + wA[t]) = rg[t];
            *reinterpret_cast<u32x4 *>(b + wT[t]) = rg[t];
        }
        if (tid < QS) {
            const int row = (s0 + s) * QS + tid;
            s_lse[st][tid] = row >= N ? INFINITY : vl;   // +inf: no weight
        } else if (tid < 2 * QS) {
            s_D[st][tid - QS] = vd;
        }
    };

    f32x4 dka[DBK], dva[DBV];
#pragma unroll
    for (int db = 0; db < DBK; ++db) dka[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < DBV; ++db) dva[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int s, int st) {
        const int i0 = (s0 + s) * QS;
        // Skip when no row of this step sees any of the wave's keys.
        const bool active = kw0 <= off_c + i0 + QS - 1;
        if (active) {
            const unsigned char *qa = bq[st][0], *qt = bq[st][1];
            const unsigned char *da = bo[st][0], *dt = bo[st][1];
            f32x4 S[2], dP[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                S[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
                dP[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
                if constexpr (D == DV) {   // the two products interleaved step by step
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        S[rb] = Mma<T>::run(as_vec<T>(lds_row16(qa + rb * 16 * ROWQ + aq(ks))), kop[ks], S[rb]);
                        dP[rb] = Mma<T>::run(as_vec<T>(lds_row16(da + rb * 16 * ROWO + aq(ks))), vop[ks], dP[rb]);
                    }
                } else {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        S[rb] = Mma<T>::run(as_vec<T>(lds_row16(qa + rb * 16 * ROWQ + aq(ks))), kop[ks], S[rb]);
#pragma unroll
                    for (int ks = 0; ks < KSV; ++ks)
                        dP[rb] = Mma<T>::run(as_vec<T>(lds_row16(da + rb * 16 * ROWO + ao(ks))), vop[ks], dP[rb]);
                }
            }
            // P and dS of rows rb*16 + 4g + r, key `key`.  Only steps where
            // some of the wave's keys are hidden from some row (the diagonal,
            // or keys past Nk) pay for the mask.
            const bool masked = kw0 + 15 >= Nk || kw0 + 15 > off_c + i0;
            if (masked) {
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int rl = rb * 16 + 4 * g + r;
                        const bool vis = key < Nk && key <= off_c + i0 + rl;
                        const float p = vis ? fast_exp2(fmaf(S[rb][r], c, -s_lse[st][rl])) : 0.f;
                        S[rb][r] = p;
                        dP[rb][r] = p * (dP[rb][r] - s_D[st][rl]);
                    }
            } else {
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int rl = rb * 16 + 4 * g + r;
                        const float p = fast_exp2(fmaf(S[rb][r], c, -s_lse[st][rl]));
                        S[rb][r] = p;
                        dP[rb][r] = p * (dP[rb][r] - s_D[st][rl]);
                    }
            }
            const vec8 pb = pack_b<T>(S[0], S[1]);
            const vec8 sb = pack_b<T>(dP[0], dP[1]);
            if constexpr (D == DV) {
#pragma unroll
                for (int db = 0; db < DBK; ++db) {
                    dva[db] = Mma<T>::run(lds_tr32<T, ROWO>(dt + tq(db)), pb, dva[db]);
                    dka[db] = Mma<T>::run(lds_tr32<T, ROWQ>(qt + tq(db)), sb, dka[db]);
                }
            } else {
#pragma unroll
                for (int db = 0; db < DBV; ++db)
                    dva[db] = Mma<T>::run(lds_tr32<T, ROWO>(dt + to(db)), pb, dva[db]);
#pragma unroll
                for (int db = 0; db < DBK; ++db)
                    dka[db] = Mma<T>::run(lds_tr32<T, ROWQ>(qt + tq(db)), sb, dka[db]);
            }
        }
    };

    // The prefetches are issued unconditionally (loads past the last step are
    // bounds-checked and never stored), so that every path through the loop
    // issues the same loads and each wait covers exactly what it needs.
    if (nsteps > 0) {
        load_step(regs0, vl0, vd0, 0);
        store_step(regs0, vl0, vd0, 0, 0);
    }
    if constexpr (kOneSet) load_step(regs0, vl0, vd0, 1);
    else load_step(regs1, vl1, vd1, 1);
    // Re-define the K^T and V^T operands (landed by now) so that the step
    // loop carries no dependence on their loads: it would otherwise wait on
    // the vector-memory counter, and so on the steps' own prefetch loads.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(kop[ks]));
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) asm volatile("" : "+v"(vop[ks]));
    __syncthreads();
    if constexpr (kOneSet) {
        for (int s = 0; s < nsteps; s += 2) {
            compute(s, 0);
            if (s + 1 < nsteps) store_step(regs0, vl0, vd0, s + 1, 1);
            __syncthreads();
            load_step(regs0, vl0, vd0, s + 2);
            if (s + 1 >= nsteps) break;
            compute(s + 1, 1);
            if (s + 2 < nsteps) store_step(regs0, vl0, vd0, s + 2, 0);
            __syncthreads();
            load_step(regs0, vl0, vd0, s + 3);
        }
    } else {
        for (int s = 0; s < nsteps; s += 2) {
            load_step(regs0, vl0, vd0, s + 2);
            compute(s, 0);
            if (s + 1 < nsteps) store_step(regs1, vl1, vd1, s + 1, 1);
            __syncthreads();
            if (s + 1 >= nsteps) break;
            load_step(regs1, vl1, vd1, s + 3);
            compute(s + 1, 1);
            if (s + 2 < nsteps) store_step(regs0, vl0, vd0, s + 2, 0);
            __syncthreads();
        }
    }

    // dK^T, dV^T result blocks: lane holds columns 16 db + 4g + r of `key`.
    // They leave through LDS (the step buffers are idle after the loop's last
    // barrier: the Q buffer holds the workgroup's 128 dK rows exactly, the dO
    // buffer its dV rows), read back row-major and stored as whole rows.
    store_rows<T, D, ROWQ>(&bq[0][0][0] + wave * 16 * ROWQ, lane, dka, scale,
                           make_rsrc(dk + (int64_t)head * Nk * D, (uint32_t)Nk * D * 2u), kw0);
    store_rows<T, DV, ROWO>(&bo[0][0][0] + wave * 16 * ROWO, lane, dva, 1.f,
                            make_rsrc(dvo + (int64_t)head * Nk * DV, (uint32_t)Nk * DV * 2u), kw0);
}

// =============================================================================
// dQ
// =============================================================================
template <typename T, int D, int DV>
__global__ __launch_bounds__(kThreads, (bwd_waves_per_simd<D, DV>())) void bwd_dq_mfma_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ lse, const T *__restrict__ dout, const T *__restrict__ o,
    float *__restrict__ Dsum, T *__restrict__ dq, int N, int Nk, int off_c, float c, float scale,
    int heads) {
    typedef typename Mma<T>::vec vec8;
    constexpr int KS = D / 32;              // contraction steps of S^T = K Q^T (over d)
    constexpr int KSV = DV / 32;            // contraction steps of dP^T = V dO^T (over dv)
    constexpr int DB = D / 16;              // 16-column blocks of dQ^T
    constexpr int ROWK = 2 * D, ROWV = 2 * DV;   // bytes per K / V row
    constexpr int CPRK = ROWK / 16, CPRV = ROWV / 16;
    constexpr int BC = D + DV <= 256 ? 64 : 32;     // keys per step (LDS: 2 stages of 3 copies)
    constexpr int KB = BC / 16;             // 16-key score blocks per step
    constexpr int PC = BC / 32;             // 32-key contraction steps of dQ^T
    constexpr int TK = BC * ROWK, TV = BC * ROWV;
    constexpr int CHK = BC * CPRK, CHV = BC * CPRV;
    constexpr int NL = (CHK + CHV + kThreads - 1) / kThreads;   // chunks per thread per step

    // Per stage: K row-major, K transposing, V row-major.
    __shared__ __attribute__((aligned(16))) unsigned char bk[2][2][TK];
    __shared__ __attribute__((aligned(16))) unsigned char bv[2][TV];

    int head, qblk;
    work_item((N + kWaves * 16 - 1) / (kWaves * 16), heads, head, qblk);
    const int i0 = qblk * (kWaves * 16);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;
    const int g = lane / 16;
    const int li = lane % 16;
    const int qw0 = i0 + wave * 16;
    const int row = qw0 + li;               // this lane's query row (MFMA column)

    const auto qrs = make_rsrc(q + (int64_t)head * N * D, (uint32_t)N * D * 2u);
    const auto drs = make_rsrc(dout + (int64_t)head * N * DV, (uint32_t)N * DV * 2u);
    const auto ors = make_rsrc(o + (int64_t)head * N * DV, (uint32_t)N * DV * 2u);
    const auto krs = make_rsrc(k + (int64_t)head * Nk * D, (uint32_t)Nk * D * 2u);
    const auto vrs = make_rsrc(v + (int64_t)head * Nk * DV, (uint32_t)Nk * DV * 2u);

    // Q^T and dO^T B operands, and this row's D = sum_c dO_c O_c from the same
    // column slices of O (summed over the four lane groups); D and the row's
    // LSE log2 e are also written for the dK/dV kernel, which runs after this
    // one.
    vec8 qop[KS], dop[KSV];
    float dpart = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) {
        const uint32_t off = ((uint32_t)row * DV + ks * 32 + 8 * g) * 2u;
        if (D == DV) qop[ks] = as_vec<T>(buffer_load16(qrs, off));
        dop[ks] = as_vec<T>(buffer_load16(drs, off));
        const vec8 ov = as_vec<T>(buffer_load16(ors, off));
#pragma unroll
        for (int j = 0; j < 8; ++j) dpart = fmaf(to_f32(ov[j]), to_f32(dop[ks][j]), dpart);
    }
    if (D != DV) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qop[ks] = as_vec<T>(buffer_load16(qrs, ((uint32_t)row * D + ks * 32 + 8 * g) * 2u));
    }
    const float Drow = rows4_sum(dpart);
    float lse2 = INFINITY;
    if (row < N) {
        const float L = lse[(int64_t)head * N + row];
        lse2 = L == -INFINITY ? INFINITY : L * kLog2e;
        if (g == 0) {
            Dsum[((int64_t)head * N + row) * 2] = lse2;
            Dsum[((int64_t)head * N + row) * 2 + 1] = Drow;
        }
    }

    const int key_end = min(Nk, off_c + min(i0 + kWaves * 16, N));
    const int nsteps = key_end > 0 ? (key_end + BC - 1) / BC : 0;

    // Chunk roles are uniform per wave (CHK and CHK + CHV are multiples of 64).
    static_assert(CHK % 64 == 0 && (CHK + CHV) % 64 == 0, "wave-uniform chunk roles");
    uint32_t gofs[NL], wA[NL], wT[NL];
    bool isv[NL], used[NL];
#pragma unroll
    for (int t = 0; t < NL; ++t) {
        const int cidx = t * kThreads + tid;
        const int cwave = t * kThreads + wave * 64;
        used[t] = cwave < CHK + CHV;
        isv[t] = cwave >= CHK;
        if constexpr (D == DV) {   // one layout for both tensors
            const int ch = cidx % CHK;
            const int r = ch / CPRK, cc = ch % CPRK;
            gofs[t] = ((uint32_t)r * D + cc * 8) * 2u;
            wA[t] = r * ROWK + ((cc ^ kswz<D>(r)) * 16);
            wT[t] = r * ROWK + (((2 * cc) ^ vswz<D>(r)) * 8);
            continue;
        }
        gofs[t] = wA[t] = wT[t] = 0;
        if (!used[t]) continue;
        if (!isv[t]) {
            const int r = cidx / CPRK, cc = cidx % CPRK;
            gofs[t] = ((uint32_t)r * D + cc * 8) * 2u;
            wA[t] = r * ROWK + ((cc ^ kswz<D>(r)) * 16);
            wT[t] = r * ROWK + (((2 * cc) ^ vswz<D>(r)) * 8);
        } else {
            const int ch = cidx - CHK;
            const int r = ch / CPRV, cc = ch % CPRV;
            gofs[t] = ((uint32_t)r * DV + cc * 8) * 2u;
            wA[t] = r * ROWV + ((cc ^ kswz<DV>(r)) * 16);
        }
    }
    uint32_t rAk[KS], rAv[KSV], rT[DB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) rAk[ks] = li * ROWK + (((ks * 4 + g) ^ kswz<D>(li)) * 16);
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) rAv[ks] = li * ROWV + (((ks * 4 + g) ^ kswz<DV>(li)) * 16);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int r0 = 4 * g + li / 4;
        rT[db] = r0 * ROWK + (((4 * db + li % 4) ^ vswz<D>(r0)) * 8);
    }

    u32x4 regs0[NL], regs1[NL];
    auto load_step = [&](u32x4 (&rg)[NL], int s) {
        const uint32_t basek = (uint32_t)(s * BC) * D * 2u;
        const uint32_t basev = D == DV ? basek : (uint32_t)(s * BC) * DV * 2u;
#pragma unroll
        for (int t = 0; t < NL; ++t)
            rg[t] = buffer_load16(isv[t] ? vrs : krs, (isv[t] ? basev : basek) + gofs[t]);
    };
    auto store_step = [&](const u32x4 (&rg)[NL], int st) {
#pragma unroll
        for (int t = 0; t < NL; ++t) {
            if (!used[t]) continue;
            if (isv[t]) {
                *reinterpret_cast<u32x4 *>(bv[st] + wA[t]) = rg[t];
            } else {
                *reinterpret_cast<u32x4 *>(bk[st][0] + wA[t]) = rg[t];
                *reinterpret_cast<u32x4 *>(bk[st][1] + wT[t]) = rg[t];
            }
        }
    };

    f32x4 dqa[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dqa[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int s, int st) {
        const int j0 = s * BC;
        const bool active = qw0 < N && j0 <= off_c + qw0 + 15;
        if (active) {
            const unsigned char *ka = bk[st][0], *kt = bk[st][1], *va = bv[st];
            f32x4 S[KB], dP[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                S[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
                dP[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
                if constexpr (D == DV) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        S[kb] = Mma<T>::run(as_vec<T>(lds_row16(ka + kb * 16 * ROWK + rAk[ks])), qop[ks], S[kb]);
                        dP[kb] = Mma<T>::run(as_vec<T>(lds_row16(va + kb * 16 * ROWV + rAk[ks])), dop[ks], dP[kb]);
                    }
                } else {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        S[kb] = Mma<T>::run(as_vec<T>(lds_row16(ka + kb * 16 * ROWK + rAk[ks])), qop[ks], S[kb]);
#pragma unroll
                    for (int ks = 0; ks < KSV; ++ks)
                        dP[kb] = Mma<T>::run(as_vec<T>(lds_row16(va + kb * 16 * ROWV + rAv[ks])), dop[ks], dP[kb]);
                }
            }
            // As in the dK/dV kernel, only steps that reach past some row's
            // last visible key (or past Nk) apply the mask.
            const bool masked = j0 + BC > Nk || j0 + BC - 1 > off_c + qw0;
            if (masked) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int kk = j0 + kb * 16 + 4 * g + r;
                        const bool vis = kk < Nk && kk <= off_c + row;
                        const float p = vis ? fast_exp2(fmaf(S[kb][r], c, -lse2)) : 0.f;
                        dP[kb][r] = p * (dP[kb][r] - Drow);
                    }
            } else {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float p = fast_exp2(fmaf(S[kb][r], c, -lse2));
                        dP[kb][r] = p * (dP[kb][r] - Drow);
                    }
            }
#pragma unroll
            for (int pc = 0; pc < PC; ++pc) {
                const vec8 sb = pack_b<T>(dP[2 * pc], dP[2 * pc + 1]);
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    dqa[db] = Mma<T>::run(lds_tr32<T, ROWK>(kt + pc * 32 * ROWK + rT[db]), sb, dqa[db]);
            }
        }
    };

    // Steps fetched two ahead, unconditionally, as in the dK/dV kernel.
    if (nsteps > 0) {
        load_step(regs0, 0);
        store_step(regs0, 0);
    }
    load_step(regs1, 1);
    // As in the dK/dV kernel: the row's operands carry no load dependence
    // into the step loop.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qop[ks]));
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) asm volatile("" : "+v"(dop[ks]));
    __syncthreads();
    for (int s = 0; s < nsteps; s += 2) {
        load_step(regs0, s + 2);
        compute(s, 0);
        if (s + 1 < nsteps) store_step(regs1, 1);
        __syncthreads();
        if (s + 1 >= nsteps) break;
        load_step(regs1, s + 3);
        compute(s + 1, 1);
        if (s + 2 < nsteps) store_step(regs0, 0);
        __syncthreads();
    }

    // dQ^T leaves through LDS like dK and dV (the K buffer is idle after the
    // loop's last barrier and holds the workgroup's 128 rows).
    static_assert(sizeof(bk) >= kWaves * 16 * ROWK, "dQ staging fits");
    store_rows<T, D, ROWK>(&bk[0][0][0] + wave * 16 * ROWK, lane, dqa, scale,
                           make_rsrc(dq + (int64_t)head * N * D, (uint32_t)N * D * 2u), qw0);
}

// Query i sees keys up to off_c + i: off_c = Nk - N under the causal mask
// (bottom-right), and off_c = Nk (every key) without it, so one kernel per
// shape serves both.
template <typename T, int D, int DV>
hipError_t launch2(const BwdArgs &b) {
    const FwdArgs &a = b.a;
    const unsigned heads = (unsigned)(a.B * a.H);
    const float c = a.scale * kLog2e;
    const int off_c = a.causal ? (int)(a.Nk - a.N) : (int)a.Nk;
    // dQ first: it also writes the (LSE log2 e, D) pairs the dK/dV kernels read.
    hipError_t e;
    if (bwd_dq_mfma32_preferred(b)) {
        e = launch_bwd_dq_mfma32(b);
    } else {
        const dim3 gq((unsigned)((a.N + kWaves * 16 - 1) / (kWaves * 16)) * heads);
        hipLaunchKernelGGL((bwd_dq_mfma_kernel<T, D, DV>), gq, dim3(kThreads), 0, a.stream,
                           static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                           static_cast<const T *>(a.v), a.lse, static_cast<const T *>(b.dout),
                           static_cast<const T *>(a.o), b.Dsum, static_cast<T *>(b.dq), (int)a.N,
                           (int)a.Nk, off_c, c, a.scale, (int)heads);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    if (bwd_dkdv_mfma32_preferred(b)) return launch_bwd_dkdv_mfma32(b);
    const dim3 gk((unsigned)((a.Nk + kWaves * 16 - 1) / (kWaves * 16)) * heads);
    hipLaunchKernelGGL((bwd_dkdv_mfma_kernel<T, D, DV>), gk, dim3(kThreads), 0, a.stream,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), a.lse, static_cast<const T *>(b.dout),
                       b.Dsum, static_cast<T *>(b.dk), static_cast<T *>(b.dv), (int)a.N,
                       (int)a.Nk, off_c, c, a.scale, (int)heads);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dv(const BwdArgs &b) {
    switch (b.a.dv) {
        case 32: return launch2<T, D, 32>(b);
        case 64: return launch2<T, D, 64>(b);
        case 128: return launch2<T, D, 128>(b);
        case 256: return launch2<T, D, 256>(b);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch1(const BwdArgs &b) {
    switch (b.a.d) {
        case 32: return launch_dv<T, 32>(b);
        case 64: return launch_dv<T, 64>(b);
        case 128: return launch_dv<T, 128>(b);
        case 256: return launch_dv<T, 256>(b);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool bwd_mfma_supported(int dtype, int64_t d, int64_t dv) {
    auto ok = [](int64_t x) { return x == 32 || x == 64 || x == 128 || x == 256; };
    return (dtype == kBF16 || dtype == kF16) && ok(d) && ok(dv);
}

hipError_t launch_bwd_mfma(const BwdArgs &b) {
    if (!bwd_mfma_supported(b.a.dtype, b.a.d, b.a.dv)) return hipErrorInvalidValue;
    return b.a.dtype == kBF16 ? launch1<bf16_t>(b) : launch1<f16_t>(b);
}

}  // namespace fa
