// fa_mfma32.h -- building blocks shared by the kernels built on the CDNA4
// 32x32x16 matrix-core instruction (v_mfma_f32_32x32x16_{bf16,f16}).
//
// Lane layouts of that instruction (lane l, n = l % 32, h = l / 32): the A
// operand holds A[n][8h + j], the B operand B[8h + j][n] (j = 0..7), and
// result register r holds D[8 (r/4) + 4h + r%4][n].
#pragma once

#include "fa_device.h"

namespace fa {
namespace mfma32 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
    typedef bf16x8 vec;
    static __device__ __forceinline__ f32x16 run(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<f16_t> {
    typedef f16x8 vec;
    static __device__ __forceinline__ f32x16 run(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// x combined with the value of lane ^ 32 (the other half of the same query).
__device__ __forceinline__ float halves_max(float x) {
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __builtin_elementwise_maximum(__int_as_float(b[0]), __int_as_float(b[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
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

// LDS swizzles (chosen so that the operand reads below are free of bank
// conflicts).  K: 16-byte chunk c of key row r is stored at chunk
// c ^ kswz(r).  V: 8-byte quad u of row r is stored at quad u ^ vswz(r), a
// multiple of 8 quads, so 16-byte chunks stay whole.  kswz depends only on
// r mod 32 and vswz on r mod 4, so shifting the row by a multiple of 32
// keeps both patterns.
template <int D> __device__ __forceinline__ int kswz(int r) {
    if constexpr (D == 64) return ((r >> 2) & 7) ^ ((r & 3) << 1);
    else return ((r >> 1) & 15) ^ ((r & 1) << 3);
}
template <int D> __device__ __forceinline__ int vswz(int r) {
    if constexpr (D == 64) return 8 * ((r >> 1) & 1);
    else return 8 * (r & 3);
}

// vmcnt wait that leaves at most `n` vector-memory operations outstanding;
// n is rounded down to a supported immediate (waiting longer is always safe).
__device__ __forceinline__ void wait_pending(int n) {
    if (n >= 32) wait_vmcnt<32>();
    else if (n >= 24) wait_vmcnt<24>();
    else if (n >= 16) wait_vmcnt<16>();
    else if (n >= 12) wait_vmcnt<12>();
    else if (n >= 8) wait_vmcnt<8>();
    else if (n >= 6) wait_vmcnt<6>();
    else if (n >= 4) wait_vmcnt<4>();
    else if (n >= 3) wait_vmcnt<3>();
    else if (n >= 2) wait_vmcnt<2>();
    else if (n >= 1) wait_vmcnt<1>();
    else wait_vmcnt<0>();
}

}  // namespace mfma32
}  // namespace fa
