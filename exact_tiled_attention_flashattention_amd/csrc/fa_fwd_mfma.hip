// fa_fwd_mfma.hip -- exact attention forward on the CDNA4 matrix cores.
//
// bf16/fp16 inputs, d == dv in {64, 128}, scale > 0; fp32 accumulation.
//
// Method: the FlashAttention-2 loop order of CS349E Lecture 11
// "flash_lab.py", section 3 (flash_fwd, order "fa2"): one block of 128
// query rows per workgroup; the head's K/V tiles (64 keys) stream through
// LDS; per tile the scores of the block are formed on chip, the running row
// maximum and row sum are updated with section 1's online-softmax rescaling,
// and the rescaled output accumulator gains P V.  O is divided by the row
// sum once at the end and LSE = m + ln l is written beside it.  Under the
// causal mask (query i at position Nk - N + i, section 2) tiles past the
// block's last visible key are never loaded and only tiles that straddle
// the diagonal or the end of the keys pay for masking.
//
// gfx950 mapping (4 waves, 32 query rows per wave):
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
//    that same key order.
//  * LDS tiles are XOR-swizzled per row (16-byte chunks for K, 32-byte
//    groups for V) so that the A-operand reads of K and the transposing
//    reads of V hit distinct banks.  Two buffers: while tile j is consumed,
//    tile j+1 is fetched with 16-byte global loads into registers and
//    written to the other buffer afterwards; one barrier per tile.
//  * The row sum is kept per lane (over that lane's keys) and reduced
//    across the 4 lane groups only in the epilogue.
//  * Workgroups are numbered so that consecutive work of one head lands on
//    one XCD (the hardware deals workgroup ids round-robin over the 8 XCDs),
//    keeping a head's K/V hot in that XCD's L2; under the causal mask the
//    longest query blocks of each head are issued first.
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

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBR = 128;            // query rows per workgroup
constexpr int kQW = kBR / kWaves;   // query rows per wave (two 16-row blocks)
constexpr int kBC = 64;             // keys per tile
// A buffer offset beyond any head's K/V extent (at most 2^31 bytes).
constexpr uint32_t kOutOfRange = 0xC0000000u;

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
__device__ __forceinline__ float rows_sum(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = __int_as_float(a[0]) + __int_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(b[0]) + __int_as_float(b[1]);
}

// acc + sum of the 8 probabilities of a B operand, as rounded for the MFMA
// (v_dot2 against (1, 1) pairs), so numerator and denominator see the same P.
__device__ __forceinline__ float row_sum_pairs(bf16x8 t, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(t, t, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(t, t, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(t, t, 4, 5), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(t, t, 6, 7), one, acc, false);
    return acc;
}
__device__ __forceinline__ float row_sum_pairs(f16x8 t, float acc) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(t, t, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(t, t, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(t, t, 4, 5), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(t, t, 6, 7), one, acc, false);
    return acc;
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left at their "no wait" maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS swizzles.  K: 16-byte chunk c of key row r is stored at chunk
// c ^ kswz(r).  V: 8-byte quad u of row r is stored at quad u ^ vswz(r)
// (a multiple of 4, so 16-byte chunks stay whole).
template <int D> __device__ __forceinline__ int kswz(int r) {
    if constexpr (D == 64) return (r & 7) ^ ((r >> 3) & 1);
    else return r & 15;
}
template <int D> __device__ __forceinline__ int vswz(int r) {
    if constexpr (D == 64) return 4 * ((r & 3) ^ ((r >> 2) & 1));
    else return 4 * (r & 7);
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, (D == 64 ? 2 : 1)) void fwd_mfma_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    T *__restrict__ o, float *__restrict__ lse, int N, int Nk, float c,
    int q_blocks, int num_wg) {
    typedef typename Mfma<T>::vec vec8;
    constexpr int KS = D / 32;                  // contraction steps of S (d)
    constexpr int DB = D / 16;                  // 16-wide value blocks of O
    constexpr int KB = kBC / 16;                // 16-key blocks of S per tile
    constexpr int PC = kBC / 32;                // contraction steps of P V (keys)
    constexpr int ROWB = D * 2;                 // bytes per key row
    constexpr int TILE = kBC * ROWB;            // bytes per K (or V) tile
    constexpr int CPR = ROWB / 16;              // 16-byte chunks per row

    constexpr int NBUF = (D == 64) ? 3 : 2;     // LDS stages (tiles in flight)
    constexpr int LPT = TILE / 1024 / kWaves;  // 1 KiB wave loads per wave per K (or V) tile
    static_assert(LPT * 1024 * kWaves == TILE, "tile split");
    __shared__ __attribute__((aligned(16))) unsigned char smem[NBUF][2][TILE];   // [stage][K,V]

    // ---- workgroup -> (head, query block) ---------------------------------
    const int w = blockIdx.x;
    const int per = num_wg / 8, rem = num_wg % 8;
    const int xcd = w % 8, idx = w / 8;
    const int L = xcd * per + min(xcd, rem) + idx;
    const int head = L / q_blocks;
    int qblk = L % q_blocks;
    if (CAUSAL) qblk = q_blocks - 1 - qblk;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // uniform per wave
    const int lane = tid % 64;
    const int g = lane / 16;    // lane row (0..3)
    const int li = lane % 16;   // lane column
    const int q0 = qblk * kBR;
    const int qw0 = q0 + wave * kQW;

    // Bounds-checked views of this head's Q, K, V (reads past the end give 0).
    const auto qrs = make_rsrc(q + (int64_t)head * N * D, (uint32_t)N * D * 2u);

    // ---- Q^T operands: lane holds Q[qw0 + qb*16 + li][ks*32 + 8g .. +7] ---
    vec8 qop[2][KS];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int row = qw0 + qb * 16 + li;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint32_t off = ((uint32_t)row * D + ks * 32 + 8 * g) * 2u;
            qop[qb][ks] = __builtin_bit_cast(vec8, buffer_load16(qrs, off));
        }
    }

    // ---- key range of this block ------------------------------------------
    int key_end = Nk;
    int full_end = Nk;   // keys below this are visible to every query of the block
    if (CAUSAL) {
        key_end = min(Nk, Nk - N + min(q0 + kBR, N));
        full_end = min(Nk, Nk - N + q0 + 1);
    }
    const int ntiles = key_end > 0 ? (key_end + kBC - 1) / kBC : 0;

    // K/V tiles go straight from memory to LDS (buffer_load ... lds): each
    // wave load writes 1 KiB of LDS, lane i's 16 bytes at offset 16 i, so the
    // swizzled layout is produced by choosing which global 16-byte piece each
    // lane fetches.  A tile index past the last one points the load outside
    // the buffers, which writes zeros and touches no memory.
    typedef __attribute__((address_space(3))) void lds_void;
    uint32_t koff[LPT], voff[LPT];   // per-lane global byte offsets within a tile
#pragma unroll
    for (int t = 0; t < LPT; ++t) {
        const int slot = (t * kWaves + wave) * 64 + lane;   // 16-byte slot in the tile
        const int row = slot / CPR, pc = slot % CPR;
        koff[t] = ((uint32_t)row * D + (pc ^ kswz<D>(row)) * 8) * 2u;
        voff[t] = ((uint32_t)row * D + (((2 * pc) ^ vswz<D>(row)) / 2) * 8) * 2u;
    }
    const u32x4 kw = rsrc_words(k + (int64_t)head * Nk * D, (uint32_t)Nk * D * 2u);
    const u32x4 vw = rsrc_words(v + (int64_t)head * Nk * D, (uint32_t)Nk * D * 2u);
    const uint32_t lds0 = (uint32_t)(size_t)(lds_void *)&smem[0][0][0];
    auto issue = [&](int j) {
        const int stage = j % NBUF;
        const uint32_t tile_off = j < ntiles ? (uint32_t)j * kBC * D * 2u : kOutOfRange;
#pragma unroll
        for (int t = 0; t < LPT; ++t) {
            const uint32_t dst = lds0 + stage * 2 * TILE + (t * kWaves + wave) * 1024;
            lds_dma16(kw, __builtin_amdgcn_readfirstlane(dst), tile_off + koff[t]);
            lds_dma16(vw, __builtin_amdgcn_readfirstlane(dst + TILE), tile_off + voff[t]);
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
    float l[2] = {0.f, 0.f};               // per-lane partial row sums
    f32x4 oacc[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One tile of the loop.  Masked tiles straddle the diagonal or the end of
    // the keys.
    auto tile = [&](const int buf, const int j0, const bool masked) {

        // ---- S^T = K Q^T ----------------------------------------------------
        const unsigned char *ks_base = smem[buf][0];
        f32x4 s[KB][2];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            s[kb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
            s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int row = kb * 16 + li;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int chunk = (ks * 4 + g) ^ kswz<D>(row);
                const vec8 a = *reinterpret_cast<const vec8 *>(ks_base + row * ROWB + chunk * 16);
                s[kb][0] = Mfma<T>::run(a, qop[0][ks], s[kb][0]);
                s[kb][1] = Mfma<T>::run(a, qop[1][ks], s[kb][1]);
            }
        }
        if (masked) {
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

        // ---- online softmax with lazy rescaling ------------------------------
        // The running max m only moves when a row's tile max exceeds it by
        // more than 8 (base 2); otherwise the stale m is kept, so the
        // probabilities stay <= 2^8 and the accumulator needs no rescale.
        // The result is unchanged: O and l share the same m.
        float mt[2];
        bool need[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float x = s[0][qb][0];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) x = __builtin_elementwise_maximum(x, s[kb][qb][r]);
            mt[qb] = rows_max(x) * c;
            need[qb] = mt[qb] > m[qb] + 8.f;
        }
        if (__builtin_amdgcn_ballot_w64(need[0] || need[1])) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const float m_new = need[qb] ? mt[qb] : m[qb];
                const float alpha = fast_exp2(m[qb] - m_new);   // 0 when m = -inf < m_new
                const float a = need[qb] ? alpha : 1.f;
                l[qb] *= a;
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db][qb] *= a;
                m[qb] = m_new;
            }
        }
        vec8 pb[PC][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float m_use = (m[qb] == -INFINITY) ? 0.f : m[qb];
#pragma unroll
            for (int pc = 0; pc < PC; ++pc) {
                f32x8 pf;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        pf[4 * h + r] = fast_exp2(fmaf(s[2 * pc + h][qb][r], c, -m_use));
                const vec8 t = __builtin_convertvector(pf, vec8);
                pb[pc][qb] = t;
                l[qb] = row_sum_pairs(t, l[qb]);
            }
        }

        // ---- O^T += V^T P^T ------------------------------------------------
        const unsigned char *vs_base = smem[buf][1];
#pragma unroll
        for (int pc = 0; pc < PC; ++pc) {
            {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int r_lo = pc * 32 + 4 * g + li / 4;
                    const int r_hi = r_lo + 16;
                    const int u = 4 * db + (li % 4);
                    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
                    lds_i16x4 *p_lo = (lds_i16x4 *)(vs_base + r_lo * ROWB + ((u ^ vswz<D>(r_lo)) * 8));
                    lds_i16x4 *p_hi = (lds_i16x4 *)(vs_base + r_hi * ROWB + ((u ^ vswz<D>(r_hi)) * 8));
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p_lo);
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p_hi);
                    const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    const vec8 a = __builtin_bit_cast(vec8, both);
                    oacc[db][0] = Mfma<T>::run(a, pb[pc][0], oacc[db][0]);
                    oacc[db][1] = Mfma<T>::run(a, pb[pc][1], oacc[db][1]);
                }
            }
        }
    };

    // Tile j is waited for (this wave's loads via vmcnt, everyone's via the
    // barrier, which also frees the stage tile j-1 used), then tile
    // j+NBUF-1 is issued into that freed stage, then tile j is consumed.
    // The explicit wait leaves the loads of the NBUF-2 later tiles in flight.
#pragma unroll
    for (int p = 0; p < NBUF - 1; ++p) issue(p);
    // Re-define the Q operands here so that the loop carries no dependence on
    // their loads (the loop would otherwise wait for every outstanding load).
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qop[qb][ks]));
    for (int j = 0; j < ntiles; ++j) {
        wait_vmcnt<2 * LPT * (NBUF - 2)>();
        __builtin_amdgcn_s_barrier();
        issue(j + NBUF - 1);
        const int j0 = j * kBC;
        tile(j % NBUF, j0, j0 + kBC > full_end);
    }

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----------------------
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float lt = rows_sum(l[qb]);
        const int qi = qw0 + qb * 16 + li;
        if (qi >= N) continue;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        T *orow = o + ((int64_t)head * N + qi) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            typedef T t4 __attribute__((ext_vector_type(4)));
            t4 out;
#pragma unroll
            for (int r = 0; r < 4; ++r) out[r] = static_cast<T>(oacc[db][qb][r] * inv);
            *reinterpret_cast<t4 *>(orow + db * 16 + 4 * g) = out;
        }
        if (g == 0) lse[(int64_t)head * N + qi] = lt > 0.f ? (m[qb] + fast_log2(lt)) * kLn2 : -INFINITY;
    }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch3(const FwdArgs &a) {
    const int q_blocks = (int)((a.N + kBR - 1) / kBR);
    const int64_t num_wg = a.B * a.H * q_blocks;
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, CAUSAL>), dim3((unsigned)num_wg), dim3(kThreads), 0,
                       a.stream, static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), static_cast<T *>(a.o), a.lse, (int)a.N,
                       (int)a.Nk, a.scale * kLog2e, q_blocks, (int)num_wg);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch2(const FwdArgs &a) {
    return a.causal ? launch3<T, D, true>(a) : launch3<T, D, false>(a);
}

template <typename T>
hipError_t launch1(const FwdArgs &a) {
    return a.d == 64 ? launch2<T, 64>(a) : launch2<T, 128>(a);
}

}  // namespace

bool fwd_mfma_supported(int dtype, int64_t d, int64_t dv, float scale) {
    return (dtype == kBF16 || dtype == kF16) && d == dv && (d == 64 || d == 128) && scale > 0.f;
}

hipError_t launch_fwd_mfma(const FwdArgs &a) {
    return a.dtype == kBF16 ? launch1<bf16_t>(a) : launch1<f16_t>(a);
}

}  // namespace fa
