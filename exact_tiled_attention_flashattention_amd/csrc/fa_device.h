// fa_device.h -- small device helpers shared by the gfx950 kernels:
// element types, conversions, 64-lane wavefront exchanges (DPP and
// v_permlane*_swap) and the softmax constants.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fa {

typedef __bf16 bf16_t;
typedef _Float16 f16_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f32(f16_t x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x) { return static_cast<T>(x); }

// 2^x on the hardware transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2 on the hardware unit (v_log_f32); only called with x > 0.
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---- DPP lane exchanges (within 16-lane rows) ---------------------------
// Control words: quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float xor1(float x) { return dpp<0xB1>(x); }
__device__ __forceinline__ float xor2(float x) { return dpp<0x4E>(x); }
__device__ __forceinline__ float half_mirror(float x) { return dpp<0x141>(x); }
__device__ __forceinline__ float row_mirror(float x) { return dpp<0x140>(x); }

// Sum over aligned groups of G consecutive lanes (G in {1,2,4,8,16,32,64});
// every lane of a group receives the group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (G >= 2) x += xor1(x);
    if constexpr (G >= 4) x += xor2(x);
    if constexpr (G >= 8) x += half_mirror(x);
    if constexpr (G >= 16) x += row_mirror(x);
    if constexpr (G >= 32) x += __shfl_xor(x, 16);
    if constexpr (G >= 64) x += __shfl_xor(x, 32);
    return x;
}

template <int G>
__device__ __forceinline__ float group_max(float x) {
    if constexpr (G >= 2) x = fmaxf(x, xor1(x));
    if constexpr (G >= 4) x = fmaxf(x, xor2(x));
    if constexpr (G >= 8) x = fmaxf(x, half_mirror(x));
    if constexpr (G >= 16) x = fmaxf(x, row_mirror(x));
    if constexpr (G >= 32) x = fmaxf(x, __shfl_xor(x, 16));
    if constexpr (G >= 64) x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

// ---- cross-row exchanges on gfx950 ---------------------------------------
// v_permlane32_swap(a, a): lanes l and l^32 exchange; returns the partner's value.
__device__ __forceinline__ float swap32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    // r[0]: lanes 0-31 keep x[0..31], lanes 32-63 receive x[0..31];
    // r[1]: lanes 0-31 receive x[32..63], lanes 32-63 keep x[32..63].
    int lane = __lane_id();
    return __int_as_float(lane < 32 ? r[1] : r[0]);
}

// 16-byte vector of raw bits.
struct alignas(16) u32x4 {
    uint32_t x, y, z, w;
};

}  // namespace fa
