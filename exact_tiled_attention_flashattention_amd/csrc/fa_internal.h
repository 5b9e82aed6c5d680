// fa_internal.h -- host-side interface between the C ABI (fa_api.cpp) and
// the kernel launchers (*.hip).  Arguments reaching a launcher have already
// been validated: non-null, sizes >= 1, supported (dtype, d, dv), aligned,
// and every per-head element count below 2^31.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace fa {

// Resident workgroups of one kernel on the current device: the CU count times
// the workgroups of `threads` threads a CU holds at once.  Cached per device
// in `cache` (one zero-initialised array per kernel); 0 if a query fails.
inline int resident_workgroups_of(const void *kernel, int threads, int (&cache)[64]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int val = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (val > 0) return val;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
        return 0;
    val = cus * (per_cu > 0 ? per_cu : 1);
    __atomic_store_n(&cache[dev], val, __ATOMIC_RELAXED);
    return val;
}

enum Dtype : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

struct FwdArgs {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *lse;
    int64_t B, H, N, Nk, d, dv;
    int causal;
    float scale;
    int dtype;
    hipStream_t stream;
};

struct DecodeArgs {
    FwdArgs a;            // a.H is the number of query heads
    int64_t Hkv;          // key/value heads; query head h reads key/value head h / (a.H / Hkv)
    int num_splits;
    int64_t seg_len;      // keys per segment (multiple of 64)
    float *ws_o;          // [B, H, num_splits, N, dv] (H query heads)
    float *ws_lse;        // [B, H, num_splits, N]
};

struct BwdArgs {
    FwdArgs a;            // q, k, v, o (forward output), lse (forward output), sizes
    const void *dout;     // [B, H, N, dv]
    void *dq;             // [B, H, N, d]   (written)
    void *dk;             // [B, H, Nk, d]  (written)
    void *dv;             // [B, H, Nk, dv] (written)
    float *Dsum;          // workspace [B, H, N, 2]: the matrix-core path keeps
                          // (LSE_i log2 e, D_i) per row (+inf for a row that
                          // sees no key), the VALU path D_i in the first B H N
                          // floats; D_i = sum_c dO_ic O_ic
};

// Row-parallel VALU forward: any dtype, d and dv in {32, 64, 128, 256}.
hipError_t launch_fwd_rowwise(const FwdArgs &a);

// MFMA forward for bf16/fp16 with d, dv in {64, 128} and scale > 0:
// d = dv = 128, d = 64 with dv = 128, and d = dv = 64 over short key ranges
// on the 32x32 kernel; the other cases on the 16x16 ping-pong kernel.
bool fwd_mfma_supported(int dtype, int64_t d, int64_t dv, float scale);
hipError_t launch_fwd_mfma16(const FwdArgs &a);      // fa_fwd_mfma.hip
// True where the 32x32 kernel of fa_fwd_mfma_wide.hip is the faster one:
// d = dv = 128, d = 64 with dv = 128, and d = dv = 64 with Nk <= 3072.
bool fwd_wide_preferred(int64_t d, int64_t dv, int64_t Nk);
hipError_t launch_fwd_mfma_wide(const FwdArgs &a);   // fa_fwd_mfma_wide.hip
// MFMA forward for every other bf16/fp16 case (any d, dv of 32..256, any
// scale), fa_fwd_mfma_generic.hip.
hipError_t launch_fwd_mfma_generic(const FwdArgs &a);

// Split-KV decode: segment kernel then merge kernel, same stream.
hipError_t launch_decode_splitkv(const DecodeArgs &a);
// The per-device static scratch that the allocation-free decode entry point
// uses as its workspace (fa_decode.hip): kDecodeScratchBytes bytes, 256-byte
// aligned.  *ptr receives the current device's address of it (looked up
// once per device with hipGetSymbolAddress, then cached).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch(void **ptr);
// Matrix-core segment kernel (bf16/fp16), fa_decode_mfma.hip; it serves
// kDecodeMfmaRows query rows per workgroup.
constexpr int kDecodeMfmaRows = 16;
hipError_t launch_decode_segment_mfma(const DecodeArgs &a);
// Segment-kernel workgroups per split for `rows` = (Hq / Hkv) x N query rows
// per key/value head (the same kernel choice as launch_decode_splitkv).
int64_t decode_workgroups_per_split(int dtype, int64_t d, int64_t dv, int64_t B, int64_t Hkv,
                                    int64_t rows);

// Backward (fa_bwd.hip): row dots, then dQ and (dK, dV); the matrix-core
// kernels (fa_bwd_mfma.hip) take bf16/fp16 with d, dv in {32, 64, 128, 256}.
hipError_t launch_bwd(const BwdArgs &b);
bool bwd_mfma_supported(int dtype, int64_t d, int64_t dv);
hipError_t launch_bwd_mfma(const BwdArgs &b);
// dK/dV kernel on the 32x32x16 instruction (fa_bwd_mfma32.hip): bf16/fp16,
// d = dv = 64; it reads the (LSE log2 e, D) pairs the dQ kernel of
// fa_bwd_mfma.hip writes.  _preferred: the shapes where it is the faster
// dK/dV kernel.
bool bwd_dkdv_mfma32_supported(int dtype, int64_t d, int64_t dv);
bool bwd_dkdv_mfma32_preferred(const BwdArgs &b);
hipError_t launch_bwd_dkdv_mfma32(const BwdArgs &b);
// dQ kernel on the 32x32x16 instruction (fa_bwd_dq_mfma32.hip): bf16/fp16,
// d = dv = 64; like the dQ kernel of fa_bwd_mfma.hip it also writes the
// (LSE log2 e, D) pairs.  _preferred: the shapes where it is the faster dQ
// kernel.
bool bwd_dq_mfma32_supported(int dtype, int64_t d, int64_t dv);
bool bwd_dq_mfma32_preferred(const BwdArgs &b);
hipError_t launch_bwd_dq_mfma32(const BwdArgs &b);

}  // namespace fa
