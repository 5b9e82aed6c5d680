// fa_fwd_mfma_generic.hip -- exact attention forward on the matrix cores for
// every bf16/fp16 (d, dv) pair from {32, 64, 128, 256} and any scale: the
// shapes the tuned kernels of fa_fwd_mfma.hip and fa_fwd_mfma_wide.hip do
// not take (d or dv of 32 or 256, scale <= 0).
//
// Method: the FlashAttention-2 loop order of CS349E Lecture 11
// "flash_lab.py", section 3 (flash_fwd, order "fa2"): a workgroup owns 64
// query rows, streams the head's K/V tiles (32 keys) through LDS and keeps
// each row's running maximum, row sum and output accumulator on chip,
// updated with section 1's online-softmax rescaling (base 2, scale folded
// in); O is divided by the row sum once at the end and LSE = m + ln l is
// written beside it.  Causal tiles past the block's last visible key are not
// loaded.
//
// gfx950 mapping (4 waves, 16 query rows per wave as the MFMA columns; lane
// l, g = l / 16, i = l % 16):
//  * S^T = K Q^T on v_mfma_f32_16x16x32_{bf16,f16}: K (A operand) is read
//    row-major from LDS, Q^T (B operand, lane: row i, columns 32 ks + 8g ..)
//    stays in registers; the result gives lane (g, i) keys 4g + r (and
//    16 + 4g + r) of row i.
//  * Row maxima over the four lane groups with v_permlane16/32_swap; the
//    running maximum moves only when a tile exceeds it by more than 8 (base
//    2), so the accumulator is rarely rescaled; the row sum is kept per lane
//    and summed over the lane groups at the end.
//  * O^T += V^T P^T: P from the score registers is the B operand over the
//    key order {4g..4g+3, 16+4g..16+4g+3}; V^T comes from ds_read_b64_tr_b16.
//  * K and V tiles are staged through registers into XOR-swizzled LDS (the
//    forward kernels' conflict-free swizzles), two tiles ahead, one barrier
//    per tile.
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

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWG = kWaves * 16;
constexpr int kBC = 32;   // keys per tile

// K: 16-byte chunk c of key row r at chunk c ^ kswz(r) (rows i, chunks 4 ks + g
// are read); V: 8-byte quad u of row r at quad u ^ vswz(r) (rows 4g + i/4,
// quads 4 db + i%4 are read transposed).  Period 16 in the row.
template <int D> __device__ __forceinline__ int kswz(int r) {
    if constexpr (D == 64)
        return ((r >> 2) & 1) | ((__builtin_popcount(r & 15) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
    else if constexpr (D == 32) return r & 3;
    else return r & 15;
}
template <int DV> __device__ __forceinline__ int vswz(int r) {
    if constexpr (DV == 64) return 4 * ((r & 3) ^ ((r >> 2) & 1));
    else if constexpr (DV == 32) return 0;
    else return 4 * (r & 7);
}

__device__ __forceinline__ float rows4_max(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = __int_as_float(a[0]) + __int_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(b[0]) + __int_as_float(b[1]);
}

// This workgroup's (head, query block) in a 1-D grid; the blocks of a head
// share an XCD (ids congruent mod 8) when the head count allows it.
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

template <typename T, int D, int DV, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_mfma_generic_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    T *__restrict__ o, float *__restrict__ lse, int N, int Nk, float c, int heads) {
    typedef typename Mma<T>::vec vec8;
    constexpr int KS = D / 32;              // contraction steps of S^T over d
    constexpr int DB = DV / 16;             // 16-column blocks of O^T
    constexpr int ROWK = 2 * D, ROWV = 2 * DV;   // bytes per K / V row
    constexpr int CPRK = ROWK / 16, CPRV = ROWV / 16;
    constexpr int CHK = kBC * CPRK, CHV = kBC * CPRV;   // 16-byte chunks per tile
    constexpr int NL = (CHK + CHV + kThreads - 1) / kThreads;   // chunks per thread per tile
    static_assert(KS >= 1 && DB >= 2, "shape");

    __shared__ __attribute__((aligned(16))) unsigned char kbuf[2][kBC * ROWK];
    __shared__ __attribute__((aligned(16))) unsigned char vbuf[2][kBC * ROWV];

    int head, qblk;
    work_item((N + kRowsPerWG - 1) / kRowsPerWG, heads, head, qblk);
    const int i0 = qblk * kRowsPerWG;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;
    const int g = lane / 16;
    const int li = lane % 16;
    const int qw0 = i0 + wave * 16;
    const int row = qw0 + li;               // this lane's query row (MFMA column)

    const auto qrs = make_rsrc(q + (int64_t)head * N * D, (uint32_t)N * D * 2u);
    const auto krs = make_rsrc(k + (int64_t)head * Nk * D, (uint32_t)Nk * D * 2u);
    const auto vrs = make_rsrc(v + (int64_t)head * Nk * DV, (uint32_t)Nk * DV * 2u);

    vec8 qop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qop[ks] = __builtin_bit_cast(vec8, buffer_load16(qrs, ((uint32_t)row * D + ks * 32 + 8 * g) * 2u));

    const int off_c = Nk - N;
    const int key_end = CAUSAL ? min(Nk, off_c + min(i0 + kRowsPerWG, N)) : Nk;
    const int nsteps = key_end > 0 ? (key_end + kBC - 1) / kBC : 0;
    const int lim = row < N ? (CAUSAL ? min(Nk - 1, off_c + row) : Nk - 1) : -1;   // last visible key
    // Keys below `full` are visible to every row of the wave.
    const int full = CAUSAL ? min(Nk, off_c + qw0 + 1) : Nk;

    // Per-thread load slots: chunk t * kThreads + tid of [K chunks | V chunks].
    // CHK and CHK + CHV are multiples of 64, so a slot's use and tensor are
    // the same for the whole wave: derived from the wave index, the choice of
    // buffer resource stays scalar (a per-lane choice costs a loop per load).
    static_assert(CHK % 64 == 0 && (CHK + CHV) % 64 == 0, "wave-uniform chunk roles");
    uint32_t gofs[NL], wofs[NL];
    bool isv[NL], used[NL];
#pragma unroll
    for (int t = 0; t < NL; ++t) {
        const int cidx = t * kThreads + tid;
        const int cwave = t * kThreads + wave * 64;
        used[t] = cwave < CHK + CHV;
        isv[t] = cwave >= CHK;
        gofs[t] = 0;
        wofs[t] = 0;
        if (!used[t]) continue;
        if (!isv[t]) {
            const int r = cidx / CPRK, cc = cidx % CPRK;
            gofs[t] = ((uint32_t)r * D + cc * 8) * 2u;
            wofs[t] = r * ROWK + ((cc ^ kswz<D>(r)) * 16);
        } else {
            const int ch = cidx - CHK;
            const int r = ch / CPRV, cc = ch % CPRV;
            gofs[t] = ((uint32_t)r * DV + cc * 8) * 2u;
            wofs[t] = r * ROWV + (((2 * cc) ^ vswz<DV>(r)) * 8);
        }
    }
    uint32_t rK[KS], rV[DB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) rK[ks] = li * ROWK + (((ks * 4 + g) ^ kswz<D>(li)) * 16);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int r0 = 4 * g + li / 4;
        rV[db] = r0 * ROWV + (((4 * db + li % 4) ^ vswz<DV>(r0)) * 8);
    }

    u32x4 regs0[NL], regs1[NL];
    auto load_step = [&](u32x4 (&rg)[NL], int s) {
        const uint32_t kb0 = (uint32_t)(s * kBC) * D * 2u, vb0 = (uint32_t)(s * kBC) * DV * 2u;
        // One load per slot; an unused slot fetches a harmless chunk that is
        // never stored.
#pragma unroll
        for (int t = 0; t < NL; ++t)
            rg[t] = buffer_load16(isv[t] ? vrs : krs, (isv[t] ? vb0 : kb0) + gofs[t]);
    };
    auto store_step = [&](const u32x4 (&rg)[NL], int st) {
#pragma unroll
        for (int t = 0; t < NL; ++t) {
            if (!used[t]) continue;
            unsigned char *base = isv[t] ? vbuf[st] : kbuf[st];
            *reinterpret_cast<u32x4 *>(base + wofs[t]) = rg[t];
        }
    };

    float m = -INFINITY;   // running max of scaled scores (base 2), per row
    float l = 0.f;         // this lane's share of the row sum
    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int s, int st) {
        const int j0 = s * kBC;
        const bool active = qw0 < N && (!CAUSAL || j0 <= off_c + qw0 + 15);
        if (!active) return;
        const unsigned char *ka = kbuf[st], *va = vbuf[st];
        f32x4 S[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            S[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                S[kb] = Mma<T>::run(__builtin_bit_cast(vec8, *reinterpret_cast<const u32x4 *>(
                                                                 ka + kb * 16 * ROWK + rK[ks])),
                                    qop[ks], S[kb]);
        }
        // Scaled scores; keys past the row's last visible key are -inf (only
        // tiles reaching past the keys every row sees pay for the compare).
        const bool masked = j0 + kBC > full;
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = S[kb][r] * c;
                if (masked && j0 + kb * 16 + 4 * g + r > lim) x = -INFINITY;
                S[kb][r] = x;
                tmax = fmaxf(tmax, x);
            }
        tmax = rows4_max(tmax);
        // Lazy rescale: the running max moves only when the tile exceeds it
        // by more than 8, so probabilities stay below 2^8.
        const bool need = tmax > m + 8.f;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float m_new = need ? tmax : m;
            const float a = need ? fast_exp2(m - m_new) : 1.f;   // 0 when m = -inf
            l *= a;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= a;
            m = m_new;
        }
        const float m_use = m == -INFINITY ? 0.f : m;
        typename Mma<T>::vec pb;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = fast_exp2(S[kb][r] - m_use);   // -inf -> 0
                l += p;
                pb[4 * kb + r] = static_cast<T>(p);
            }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const unsigned char *p = va + rV[db];
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 16 * ROWV));
            const vec8 a = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[db] = Mma<T>::run(a, pb, oacc[db]);
        }
    };

    // Tiles are fetched two ahead, unconditionally: loads past the last tile
    // are bounds-checked and never stored, so every path issues the same
    // loads and each wait covers only what it needs.
    if (nsteps > 0) {
        load_step(regs0, 0);
        store_step(regs0, 0);
    }
    load_step(regs1, 1);
    // Re-define the Q operands (landed by now) so that the loop carries no
    // dependence on their loads, which would make it wait on the vector-memory
    // counter and so on its own prefetch.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qop[ks]));
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

    // Epilogue: O = acc / l, LSE = (m + log2 l) ln 2; a row with no visible
    // key gets O = 0 and LSE = -inf.
    // O leaves through LDS (the V stage buffers are idle after the loop's last
    // barrier and hold the workgroup's 64 rows) and is stored as whole rows.
    const float lt = rows4_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (row < N && g == 0) lse[(int64_t)head * N + row] = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
    static_assert(sizeof(vbuf) >= kWaves * 16 * ROWV, "output staging fits");
    store_rows<T, DV, ROWV>(&vbuf[0][0] + wave * 16 * ROWV, lane, oacc, inv,
                            make_rsrc(o + (int64_t)head * N * DV, (uint32_t)N * DV * 2u), qw0);
}

template <typename T, int D, int DV>
hipError_t launch3(const FwdArgs &a) {
    const int64_t heads = a.B * a.H;
    const int64_t nblk = (a.N + kRowsPerWG - 1) / kRowsPerWG;
    if (nblk * heads > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(nblk * heads));
    const float c = a.scale * kLog2e;
    if (a.causal)
        hipLaunchKernelGGL((fwd_mfma_generic_kernel<T, D, DV, true>), grid, dim3(kThreads), 0,
                           a.stream, static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                           static_cast<const T *>(a.v), static_cast<T *>(a.o), a.lse, (int)a.N,
                           (int)a.Nk, c, (int)heads);
    else
        hipLaunchKernelGGL((fwd_mfma_generic_kernel<T, D, DV, false>), grid, dim3(kThreads), 0,
                           a.stream, static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                           static_cast<const T *>(a.v), static_cast<T *>(a.o), a.lse, (int)a.N,
                           (int)a.Nk, c, (int)heads);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dv(const FwdArgs &a) {
    switch (a.dv) {
        case 32: return launch3<T, D, 32>(a);
        case 64: return launch3<T, D, 64>(a);
        case 128: return launch3<T, D, 128>(a);
        case 256: return launch3<T, D, 256>(a);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_d(const FwdArgs &a) {
    switch (a.d) {
        case 32: return launch_dv<T, 32>(a);
        case 64: return launch_dv<T, 64>(a);
        case 128: return launch_dv<T, 128>(a);
        case 256: return launch_dv<T, 256>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fwd_mfma_generic(const FwdArgs &a) {
    switch (a.dtype) {
        case kF16: return launch_d<f16_t>(a);
        case kBF16: return launch_d<bf16_t>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
