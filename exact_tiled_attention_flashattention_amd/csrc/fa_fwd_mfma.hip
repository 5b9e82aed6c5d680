// fa_fwd_mfma.hip -- exact attention forward on the CDNA4 matrix cores.
//
// bf16/fp16 inputs, (d, dv) in {(64, 64), (128, 64)}, scale > 0; fp32
// accumulation.  (d = dv = 128, d = 64 with dv = 128, and d = dv = 64 with
// at most 3072 keys run on the 32x32 variant in fa_fwd_mfma_wide.hip.)
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
// gfx950 mapping (8 waves in two groups of four, 32 query rows per wave):
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_{bf16,f16}: K is the A operand (read from LDS with
//    ds_read_b128), Q^T the B operand (loaded once into registers).  The
//    16x16 result puts one query per lane column (lane & 15) and four
//    consecutive keys per lane, so a query's 64 scores of a tile sit in 16
//    registers of each of 4 lane groups: the row max needs only
//    in-register max plus v_permlane16_swap and v_permlane32_swap.
//  * The probabilities are rounded to the input type and used straight from
//    registers as the B operand of O^T = V^T P^T: the result layout of one
//    pair of 16-key score blocks is a legal B operand once the contraction
//    index is read as the key order {4g..4g+3, 16+4g..16+4g+3}.  V^T (the
//    A operand) is read from the row-major V tile with ds_read_b64_tr_b16,
//    which hands each lane four consecutive keys of one value column, in
//    that same key order.  An all-ones A operand yields the row sums.
//  * The two wave groups alternate between matrix-core work and softmax
//    work in intervals separated by barriers (ping-pong), so the two waves
//    of a SIMD (w and w + 4) overlap the matrix core and the vector ALU.
//  * K/V tiles are copied from memory straight into LDS (three stages each)
//    and XOR-swizzled per row (16-byte chunks for K, 32-byte groups for V)
//    so that the A-operand reads of K and the transposing reads of V are
//    free of bank conflicts; the loop is unrolled over the three stages so
//    that every LDS address is a register plus an immediate.
//  * The kernel is persistent: each workgroup walks units of two query
//    blocks of one head whose causal costs add up to a constant, numbered
//    so that workgroups of one XCD share heads (K/V reuse in that L2).
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// Eight waves in two groups of four; waves w and w + 4 share a SIMD.  Group
// gamma owns query rows [128 gamma, 128 gamma + 128) of the block, 32 per wave.
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBR = 256;            // query rows per workgroup
constexpr int kQW = 32;             // query rows per wave (two 16-row blocks)
constexpr int kBC = 64;             // keys per tile
template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
    typedef bf16x8 vec;
    static __device__ __forceinline__ f32x4 run(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<f16_t> {
    typedef f16x8 vec;
    static __device__ __forceinline__ f32x4 run(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).
// The maximum propagates NaN and needs no operand canonicalisation.
__device__ __forceinline__ float rows_max(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = __builtin_elementwise_maximum(__int_as_float(a[0]), __int_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __builtin_elementwise_maximum(__int_as_float(b[0]), __int_as_float(b[1]));
}
// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left at their "no wait" maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16-byte buffer load into registers, issued as inline assembly so that the
// compiler does not track it: the caller waits for it with an explicit
// s_waitcnt vmcnt before the first use of the result.  Out-of-range offsets
// read zeros.
__device__ __forceinline__ u32x4 load16_untracked(u32x4 rsrc, uint32_t voff) {
    u32x4 r;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(r) : "v"(voff), "s"(rsrc) : "memory");
    return r;
}

// LDS swizzles.  K: 16-byte chunk c of key row r is stored at chunk
// c ^ kswz(r).  V: 8-byte quad u of row r is stored at quad u ^ vswz(r)
// (a multiple of 4, so 16-byte chunks stay whole).
template <int D> __device__ __forceinline__ int kswz(int r) {
    if constexpr (D == 64)
        return ((r >> 2) & 1) | ((__builtin_popcount(r & 15) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
    else return r & 15;
}
template <int D> __device__ __forceinline__ int vswz(int r) {
    if constexpr (D == 64) return 4 * ((r & 3) ^ ((r >> 2) & 1));
    else return 4 * (r & 7);
}

template <typename T, int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_mfma_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    T *__restrict__ o, float *__restrict__ lse, int N, int Nk, float c,
    int q_blocks, int n_items) {
    typedef typename Mfma<T>::vec vec8;
    constexpr int KS = D / 32;                  // contraction steps of S (d)
    constexpr int DB = DV / 16;                 // 16-wide value blocks of O
    constexpr int KB = kBC / 16;                // 16-key blocks of S per tile
    constexpr int PC = kBC / 32;                // contraction steps of P V (keys)
    constexpr int ROWB = D * 2;                 // bytes per K row
    constexpr int ROWBV = DV * 2;               // bytes per V row
    constexpr int TILE = kBC * ROWB;            // bytes per K tile
    constexpr int TILEV = kBC * ROWBV;          // bytes per V tile
    constexpr int CPR = ROWB / 16;              // 16-byte chunks per K row
    constexpr int CPRV = ROWBV / 16;            // 16-byte chunks per V row
    constexpr int NK = 3, NV = 3;               // LDS stages of K and of V
    constexpr int LPT = TILE / 1024 / kWaves;   // 1 KiB wave loads per wave per K tile
    constexpr int LPTV = TILEV / 1024 / kWaves; // ... per V tile
    static_assert(LPT * 1024 * kWaves == TILE && LPTV * 1024 * kWaves == TILEV, "tile split");
    // K stages, then V stages, in one array.  After an item's tile loop
    // (whose last barrier every wave has passed, with no copy in flight) the
    // same memory holds each wave's normalised output rows on the way out,
    // so that every store instruction writes whole rows (1 KiB contiguous at
    // dv = 64) instead of 8-byte pieces of 16 rows.  Those rows are padded by
    // 16 bytes, which spreads the 8-byte writes of one column over the banks.
    constexpr int OPITCH = DV * 2 + 16;
    static_assert(kWaves * kQW * OPITCH <= NK * TILE + NV * TILEV, "output staging fits");
    __shared__ __attribute__((aligned(16))) unsigned char kvbuf[NK * TILE + NV * TILEV];
    unsigned char(*kbuf)[TILE] = reinterpret_cast<unsigned char(*)[TILE]>(kvbuf);
    unsigned char(*vbuf)[TILEV] = reinterpret_cast<unsigned char(*)[TILEV]>(kvbuf + NK * TILE);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // uniform per wave
    const int grp = wave / 4;   // 0: group A, 1: group B
    const int lane = tid % 64;
    const int g = lane / 16;    // lane row (0..3)
    const int li = lane % 16;   // lane column

    // Per-lane LDS byte offsets of the MFMA operand reads within a tile; the
    // rest of each address (stage, key block) is a compile-time constant.
    //  K (A operand of S^T): key row kb*16 + li, 16-byte chunk ks*4 + g.
    //  V (ds_read_b64_tr_b16): key row 4g + li/4 (+16, +32 pc), quad 4 db + li%4.
    uint32_t kofs[KS], vofs[DB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kofs[ks] = li * ROWB + (((ks * 4 + g) ^ kswz<D>(li)) * 16);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int r0 = 4 * g + li / 4;
        vofs[db] = r0 * ROWBV + (((4 * db + li % 4) ^ vswz<DV>(r0)) * 8);
    }
    vec8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = static_cast<T>(1.0f);

    // ---- persistent loop over work units ---------------------------------------
    // A unit is a pair of query blocks of one head, p and QB-1-p (the middle
    // block alone when QB is odd): under the causal mask their key counts add
    // up to the same total for every p, so units cost the same and a plain
    // round-robin of units over the G resident workgroups is balanced.  The
    // two blocks of a unit reuse the head's K/V from L2.  When G and the head
    // count are multiples of 8, units are numbered so that the workgroups of
    // one XCD (ids congruent mod 8) work on the same heads at the same time.
    const int G = gridDim.x;
    const int n_heads = n_items / q_blocks;
    const int U = (q_blocks + 1) / 2;   // units per head
    const int n_units = n_heads * U;
    const bool xcd_map = (G % 8 == 0) && (n_heads % 8 == 0);
    for (int u = blockIdx.x; u < n_units; u += G)
    for (int half = 0; half < 2; ++half) {
    int head, pair;
    if (xcd_map) {
        const int local = u / 8;
        head = (local / U) * 8 + u % 8;
        pair = local % U;
    } else {
        head = u / U;
        pair = u % U;
    }
    const int qblk = half == 0 ? pair : q_blocks - 1 - pair;
    if (half == 1 && qblk == pair) break;   // odd middle block: single item
    // The previous item's LDS reads and copies are finished everywhere.
    __syncthreads();

    const int q0 = qblk * kBR;
    const int qw0 = q0 + grp * (kBR / 2) + (wave % 4) * kQW;

    // Bounds-checked views of this head's Q, K, V (reads past the end give 0).
    const u32x4 qw = rsrc_words(q + (int64_t)head * N * D, (uint32_t)N * D * 2u);

    // ---- Q^T operands: lane holds Q[qw0 + qb*16 + li][ks*32 + 8g .. +7] ---
    // (untracked loads: the first wait below covers them, so that the tile
    // loop does not start with a wait for every load in flight)
    vec8 qop[2][KS];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int row = qw0 + qb * 16 + li;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint32_t off = ((uint32_t)row * D + ks * 32 + 8 * g) * 2u;
            qop[qb][ks] = __builtin_bit_cast(vec8, load16_untracked(qw, off));
        }
    }

    // ---- key ranges ---------------------------------------------------------
    // The block streams the tiles up to its last visible key; a wave computes
    // only the tiles its own rows can see and masks those that reach past
    // the keys every one of its rows sees (none if all its rows are past N).
    int key_end = Nk;        // block
    int wave_end = Nk;       // this wave: keys below are visible to some row
    int full_end = Nk;       // this wave: keys below are visible to every row
    if (CAUSAL) {
        key_end = min(Nk, Nk - N + min(q0 + kBR, N));
        wave_end = min(Nk, Nk - N + min(qw0 + kQW, N));
        full_end = min(Nk, Nk - N + qw0 + 1);
    }
    const int ntiles = key_end > 0 ? (key_end + kBC - 1) / kBC : 0;
    const int wtiles = (wave_end > 0 && qw0 < N) ? (wave_end + kBC - 1) / kBC : 0;

    // K/V tiles go straight from memory to LDS (buffer_load ... lds): each
    // wave load writes 1 KiB of LDS, lane i's 16 bytes at offset 16 i, so the
    // swizzled layout is produced by choosing which global 16-byte piece each
    // lane fetches.  Rows past Nk read as zeros (buffer bounds check).
    typedef __attribute__((address_space(3))) void lds_void;
    uint32_t koff[LPT], voff[LPTV];   // per-lane global byte offsets within a tile
#pragma unroll
    for (int t = 0; t < LPT; ++t) {
        const int slot = (t * kWaves + wave) * 64 + lane;   // 16-byte slot in the tile
        const int row = slot / CPR, pc = slot % CPR;
        koff[t] = ((uint32_t)row * D + (pc ^ kswz<D>(row)) * 8) * 2u;
    }
#pragma unroll
    for (int t = 0; t < LPTV; ++t) {
        const int slot = (t * kWaves + wave) * 64 + lane;
        const int row = slot / CPRV, pc = slot % CPRV;
        voff[t] = ((uint32_t)row * DV + (((2 * pc) ^ vswz<DV>(row)) / 2) * 8) * 2u;
    }
    const u32x4 kw = rsrc_words(k + (int64_t)head * Nk * D, (uint32_t)Nk * D * 2u);
    const u32x4 vw = rsrc_words(v + (int64_t)head * Nk * DV, (uint32_t)Nk * DV * 2u);
    const uint32_t klds = (uint32_t)(size_t)(lds_void *)&kbuf[0][0];
    const uint32_t vlds = (uint32_t)(size_t)(lds_void *)&vbuf[0][0];
    auto issue_k = [&](int j) {
        if (j >= ntiles) return;
        const uint32_t tile_off = (uint32_t)j * kBC * D * 2u;
#pragma unroll
        for (int t = 0; t < LPT; ++t) {
            const uint32_t dst = klds + (j % NK) * TILE + (t * kWaves + wave) * 1024;
            lds_dma16(kw, __builtin_amdgcn_readfirstlane(dst), tile_off + koff[t]);
        }
    };
    auto issue_v = [&](int j) {
        if (j >= ntiles) return;
        const uint32_t tile_off = (uint32_t)j * kBC * DV * 2u;
#pragma unroll
        for (int t = 0; t < LPTV; ++t) {
            const uint32_t dst = vlds + (j % NV) * TILEV + (t * kWaves + wave) * 1024;
            lds_dma16(vw, __builtin_amdgcn_readfirstlane(dst), tile_off + voff[t]);
        }
    };

    // Per-lane mask bound: key j0 + kb*16 + 4g + r is visible to query qi iff
    // kb*16 + r <= lim[qb] - j0, with lim = (last key qi sees) - 4g.
    int lim[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int qi = qw0 + qb * 16 + li;
        lim[qb] = (CAUSAL ? min(Nk - 1, Nk - N + qi) : Nk - 1) - 4 * g;
    }

    float m[2] = {-INFINITY, -INFINITY};   // running max of scaled scores (base 2)
    // Kept with m, changed only when m moves: the exponent offset (0 while
    // m = -inf) and the rescale threshold m + 8.
    float mu[2] = {0.f, 0.f}, m8[2] = {-INFINITY, -INFINITY};
    f32x4 lacc[2];                         // row sums (every register holds the sum)
    f32x4 oacc[DB][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        lacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    f32x4 s[KB][2];      // scores of the current tile
    vec8 pb[PC][2];      // probabilities of the previous tile (B operands)
    // Empty asm that claims to modify its operands: the values must be
    // computed before this point and are not moved (sunk) past it, which
    // keeps each phase's work inside its interval.
    auto pin_scores = [&]() {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) asm volatile("" : "+v"(s[kb][0]), "+v"(s[kb][1]));
    };
    auto pin_acc = [&]() {
#pragma unroll
        for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(oacc[db][0]), "+v"(oacc[db][1]));
        asm volatile("" : "+v"(lacc[0]), "+v"(lacc[1]));
    };
    auto pin_probs = [&]() {
#pragma unroll
        for (int pc = 0; pc < PC; ++pc) asm volatile("" : "+v"(pb[pc][0]), "+v"(pb[pc][1]));
        asm volatile("" : "+v"(m[0]), "+v"(m[1]));
    };

    // ---- S^T = K Q^T for the K tile in stage SK ---------------------------------
    auto scores = [&](auto SK) {
        const unsigned char *base = kbuf[0] + decltype(SK)::value * TILE;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            s[kb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
            s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const vec8 a = *reinterpret_cast<const vec8 *>(base + kb * 16 * ROWB + kofs[ks]);
                s[kb][0] = Mfma<T>::run(a, qop[0][ks], s[kb][0]);
                s[kb][1] = Mfma<T>::run(a, qop[1][ks], s[kb][1]);
            }
        }        pin_scores();
    };

    // ---- O^T += V^T P^T for the V tile in stage SV -----------------------------
    // The row sums come from the matrix core too: an all-ones A operand turns
    // P^T into its column sums.
    auto accumulate = [&](auto SV) {
        const unsigned char *base = vbuf[0] + decltype(SV)::value * TILEV;
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
#pragma unroll
        for (int pc = 0; pc < PC; ++pc) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const unsigned char *p = base + pc * 32 * ROWBV + vofs[db];
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 16 * ROWBV));
                const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                const vec8 a = __builtin_bit_cast(vec8, both);
                oacc[db][0] = Mfma<T>::run(a, pb[pc][0], oacc[db][0]);
                oacc[db][1] = Mfma<T>::run(a, pb[pc][1], oacc[db][1]);
            }
            lacc[0] = Mfma<T>::run(ones, pb[pc][0], lacc[0]);
            lacc[1] = Mfma<T>::run(ones, pb[pc][1], lacc[1]);
        }        pin_acc();
    };

    // ---- online softmax of tile j with lazy rescaling ----------------------------
    // The running max m only moves when a row's tile max exceeds it by more
    // than 8 (base 2); otherwise the stale m is kept, so the probabilities
    // stay <= 2^8 and the accumulator needs no rescale.  The result is
    // unchanged: O and l share the same m.
    auto softmax = [&](const int j) {
        const int j0 = j * kBC;
        if (j0 + kBC > full_end) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int t = lim[qb] - j0;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (kb * 16 + r > t) s[kb][qb][r] = -INFINITY;
            }
        }
        // A row's tile maximum exceeds m + 8 exactly when the maximum over one
        // of its four lanes' scores does, so the wave tests its lanes' own
        // maxima and forms the row maxima (a cross-lane reduction) only in
        // the rare case that some row moves.
        float xl[2];
        bool any[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float x = s[0][qb][0];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) x = __builtin_elementwise_maximum(x, s[kb][qb][r]);
            xl[qb] = x;
            any[qb] = x * c > m8[qb];
        }
        if (__builtin_amdgcn_ballot_w64(any[0] || any[1])) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const float mt = rows_max(xl[qb]) * c;
                const bool need = mt > m[qb] + 8.f;
                const float m_new = need ? mt : m[qb];
                const float alpha = fast_exp2(m[qb] - m_new);   // 0 when m = -inf < m_new
                const float a = need ? alpha : 1.f;
                lacc[qb] *= a;
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db][qb] *= a;
                m[qb] = m_new;
                mu[qb] = m_new == -INFINITY ? 0.f : m_new;
                m8[qb] = m_new + 8.f;
            }
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float m_use = mu[qb];
#pragma unroll
            for (int pc = 0; pc < PC; ++pc) {
                f32x8 pf;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        pf[4 * h + r] = fast_exp2(fmaf(s[2 * pc + h][qb][r], c, -m_use));
                pb[pc][qb] = __builtin_convertvector(pf, vec8);
            }
        }        pin_probs();
        pin_acc();
    };

    // ---- ping-pong schedule ------------------------------------------------------
    // Time is cut into intervals by workgroup barriers.  Group A forms the
    // scores of tile j and adds P V of tile j-1 (matrix cores) while group B
    // turns the scores of tile j-1 into probabilities (vector ALU); in the
    // next interval the roles swap.  The two waves sharing a SIMD thus keep
    // the matrix core and the vector ALU busy at the same time.  Both groups
    // pass the same number of barriers: B starts with one, A ends with one.
    //
    // Loads: K tiles 0-2 and V tiles 0-1 are fetched up front.  Load step i
    // (the barrier after group A's softmax of tile i) waits until K tile
    // i+1 and V tile i have landed, then fetches K tile i+3 and V tile i+2
    // into the stages of K tile i and V tile i-1, whose last readers (group
    // B's interval before that barrier) are done.  Only tiles below ntiles
    // are loaded, so nothing is in flight once the item ends.
    // Workgroup barrier that the compiler may not schedule work across, so
    // that each phase's instructions stay inside its interval.
    auto phase_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto load_step = [&](const int i) {
        if (i + 2 < ntiles) wait_vmcnt<LPT + LPTV>();
        else if (i + 1 < ntiles) wait_vmcnt<LPTV>();
        else wait_vmcnt<0>();
        phase_barrier();
        issue_k(i + 3);
        issue_v(i + 2);
    };
    // The stage of tile j is j % 3 for K and V alike; the loop bodies are
    // specialised per stage so that every LDS address is a per-lane register
    // plus an immediate offset.
    typedef std::integral_constant<int, 0> S0;
    typedef std::integral_constant<int, 1> S1;
    typedef std::integral_constant<int, 2> S2;
    auto with_stage = [&](const int j, auto f) {
        const int r = j % 3;
        if (r == 0) f(S0{});
        else if (r == 1) f(S1{});
        else f(S2{});
    };
    issue_k(0);
    issue_k(1);
    issue_v(0);
    issue_k(2);
    issue_v(1);
    // Wait for Q and K tile 0 only: the copies issued after K tile 0 may
    // still be in flight (loads complete in order, so at most that many
    // outstanding means everything before them has landed).  The first
    // load step waits for K tile 1 and V tile 0.
    if (ntiles >= 3) wait_vmcnt<2 * LPT + 2 * LPTV>();
    else if (ntiles == 2) wait_vmcnt<LPT + 2 * LPTV>();
    else if (ntiles == 1) wait_vmcnt<LPTV>();
    else wait_vmcnt<0>();
    // Re-define the Q operands here so that they are read only after that
    // wait and the loops carry no dependence on their loads.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qop[qb][ks]));
    phase_barrier();
    if (grp == 0) {
        if (wtiles > 0) scores(S0{});
        phase_barrier();
        if (wtiles > 0) softmax(0);
        load_step(0);
        // Steady state, tile j in stage j % 3 (j starts at 1): unrolled by
        // three so that no stage switch merges register assignments.
        auto body = [&](const int j, auto R) {
            accumulate(std::integral_constant<int, (decltype(R)::value + 2) % 3>{});
            scores(R);
            phase_barrier();
            softmax(j);
            load_step(j);
        };
        int j = 1;
        for (; j + 3 <= wtiles; j += 3) {
            body(j, S1{});
            body(j + 1, S2{});
            body(j + 2, S0{});
        }
        if (j < wtiles) body(j++, S1{});
        if (j < wtiles) body(j++, S2{});
        for (; j <= ntiles; ++j) {
            if (j == wtiles) with_stage(j - 1, [&](auto R) { accumulate(R); });
            phase_barrier();
            load_step(j);
        }
    } else {
        phase_barrier();
        if (wtiles > 0) scores(S0{});
        load_step(0);
        if (wtiles > 0) softmax(0);
        auto body = [&](const int j, auto R) {
            phase_barrier();
            accumulate(std::integral_constant<int, (decltype(R)::value + 2) % 3>{});
            scores(R);
            load_step(j);
            softmax(j);
        };
        int j = 1;
        for (; j + 3 <= wtiles; j += 3) {
            body(j, S1{});
            body(j + 1, S2{});
            body(j + 2, S0{});
        }
        if (j < wtiles) body(j++, S1{});
        if (j < wtiles) body(j++, S2{});
        for (; j <= ntiles; ++j) {
            phase_barrier();
            if (j == wtiles) with_stage(j - 1, [&](auto R) { accumulate(R); });
            load_step(j);
        }
    }

    const auto ors = make_rsrc(o + (int64_t)head * N * DV, (uint32_t)N * DV * 2u);
    // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----------------------
    // The wave's 32 x dv tile is written to its LDS slice (lane: row
    // qb*16 + li, columns 16 db + 4g .. +3), read back row-major 16 bytes per
    // lane, and stored as whole rows.
    // (The lane index is re-defined through an empty asm so that none of the
    // epilogue's address arithmetic is hoisted into the tile loops, where it
    // would hold registers.)
    unsigned char *ow = kvbuf + wave * (kQW * OPITCH);
    int elane = lane;
    asm volatile("" : "+v"(elane));
    const int eli = elane % 16, eg = elane / 16;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float lt = lacc[qb][0];
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            typedef T t4 __attribute__((ext_vector_type(4)));
            t4 out;
#pragma unroll
            for (int r = 0; r < 4; ++r) out[r] = static_cast<T>(oacc[db][qb][r] * inv);
            *reinterpret_cast<t4 *>(ow + (qb * 16 + eli) * OPITCH + (db * 16 + 4 * eg) * 2) = out;
        }
        const int qi = qw0 + qb * 16 + eli;
        if (eg == 0 && qi < N)
            lse[(int64_t)head * N + qi] = lt > 0.f ? (m[qb] + fast_log2(lt)) * kLn2 : -INFINITY;
    }
    {
        constexpr int CPRO = DV * 2 / 16;            // 16-byte chunks per output row
        constexpr int RPI = 64 / CPRO;               // rows per store instruction
        const int rr = elane / CPRO, cc = elane % CPRO;
#pragma unroll
        for (int t = 0; t < kQW / RPI; ++t) {
            const int row = t * RPI + rr;
            const u32x4 val = *reinterpret_cast<const u32x4 *>(ow + row * OPITCH + cc * 16);
            const int qi = qw0 + row;
            // Bounds-checked store (rows past N fall outside the buffer and
            // are dropped) with the non-temporal hint: O is not read again.
            __builtin_amdgcn_raw_buffer_store_b128(val, ors, (int)(((uint32_t)qi * DV) * 2u + cc * 16), 0, 2);
        }
    }
    }   // item loop
}

// Resident workgroups per CU of one kernel instantiation, times the CU count
// of the current device (cached per device).
template <typename T, int D, int DV, bool CAUSAL>
int resident_workgroups() {
    static int cache[64];
    return resident_workgroups_of(reinterpret_cast<const void *>(&fwd_mfma_kernel<T, D, DV, CAUSAL>),
                                  kThreads, cache);
}

template <typename T, int D, int DV, bool CAUSAL>
hipError_t launch3(const FwdArgs &a) {
    const int q_blocks = (int)((a.N + kBR - 1) / kBR);
    const int64_t n_items = a.B * a.H * q_blocks;
    const int resident = resident_workgroups<T, D, DV, CAUSAL>();
    if (resident <= 0) return hipErrorInvalidDevice;
    const int64_t grid = n_items < resident ? n_items : resident;
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, DV, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0,
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
    if (a.d == 64 && a.dv == 64) return launch2<T, 64, 64>(a);
    if (a.d == 128 && a.dv == 64) return launch2<T, 128, 64>(a);
    return hipErrorInvalidValue;
}

}  // namespace

bool fwd_mfma_supported(int dtype, int64_t d, int64_t dv, float scale) {
    const bool dims = (d == 64 || d == 128) && (dv == 64 || dv == 128);
    return (dtype == kBF16 || dtype == kF16) && dims && scale > 0.f;
}

hipError_t launch_fwd_mfma16(const FwdArgs &a) {
    return a.dtype == kBF16 ? launch1<bf16_t>(a) : launch1<f16_t>(a);
}

}  // namespace fa
