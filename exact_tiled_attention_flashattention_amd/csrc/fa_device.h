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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---- buffer loads --------------------------------------------------------
// A raw buffer resource over `bytes` bytes at `base`: loads at byte offsets
// past the end return zeros instead of touching memory, so ragged tiles
// need no branch around the load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
}
// The same load with the non-temporal hint, for data that is read exactly
// once (the decode K/V stream): it measurably raises streaming bandwidth.
__device__ __forceinline__ u32x4 buffer_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 2);
}

// The same raw buffer resource as four scalar words (for inline assembly).
__device__ __forceinline__ u32x4 rsrc_words(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);   // stride 0
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000u;
    return r;
}

// Memory -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// lane i's bytes at buffer offset `voff` land at LDS address lds_addr + 16 i.
// Issued as inline assembly so that the compiler does not track it: the
// caller waits for it (s_waitcnt vmcnt) and publishes it (s_barrier) itself.
// Out-of-range offsets write zeros.  `lds_addr` must be wave-uniform.
// The LDS address travels in M0, declared clobbered so that the compiler
// saves it only where it holds a live value there; the sequence keeps the
// one wait state the ISA asks for between a scalar write of M0 and an
// LDS-copying load.
__device__ __forceinline__ void lds_dma16(u32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// The same copy with 4 bytes per lane (buffer_load_dword ... lds): lane i's
// word lands at lds_addr + 4 i.
__device__ __forceinline__ void lds_dma4(u32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// Stores a wave's 16 x W result tile (W = D or DV columns) as whole rows.
// acc[db] holds the transposed 16x16 block db: lane (li, g) has columns
// 16 db + 4g .. +3 of row li, which are multiplied by `mul` (per lane).  The lane's 8 bytes go to the wave's LDS slice
// `buf` (16 rows of ROWB = 2 W bytes, 16-byte chunks XOR-swizzled by the row
// so that the writes of one column spread over the banks); the wave then
// reads the tile back 16 bytes per lane in row order and stores each row
// chunk with a bounds-checked, non-temporal buffer store (rows at or past
// the buffer's end are dropped).  row0 is the tile's first row in `rs`.
// Every lane of the wave must call it; the caller makes sure that no other
// wave still reads `buf`.
template <typename T, int W, int ROWB, int NB, typename AccV>
__device__ __forceinline__ void store_rows(unsigned char *buf, int lane, const AccV (&acc)[NB],
                                           float mul,
                                           __amdgpu_buffer_rsrc_t rs, int row0) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
    constexpr int SW = CPR < 8 ? CPR : 8;        // swizzle period
    static_assert(NB == W / 16 && ROWB == 2 * W, "tile shape");
    // (the lane index is re-defined so that none of this address arithmetic
    // is hoisted into the caller's loops)
    int el = lane;
    asm volatile("" : "+v"(el));
    const int li = el % 16, g = el / 16;
#pragma unroll
    for (int db = 0; db < NB; ++db) {
        t4 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = static_cast<T>(acc[db][r] * mul);
        const int chunk = (2 * db + g / 2) ^ (li % SW);
        *reinterpret_cast<t4 *>(buf + li * ROWB + chunk * 16 + (g % 2) * 8) = a;
    }
    constexpr int RPI = 64 / CPR;                // rows per store instruction
    const int rr = el / CPR, cc = el % CPR;
#pragma unroll
    for (int t = 0; t < 16 / RPI; ++t) {
        const int r = t * RPI + rr;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(buf + r * ROWB + ((cc ^ (r % SW)) * 16));
        __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)((uint32_t)(row0 + r) * ROWB + cc * 16), 0, 2);
    }
}

}  // namespace fa
