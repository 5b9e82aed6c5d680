// fa_api.cpp -- the C ABI of libfa.so (declared in include/fa.h).
//
// Every argument is checked before the first HIP call, so an invalid call
// returns a status and touches nothing.  Valid calls are dispatched on
// (dtype, d, dv) to a kernel launcher and enqueued on the caller's stream;
// nothing is allocated and nothing is synchronised.
#include "fa.h"

#include <cmath>
#include <cstdint>
#include <limits>

#include "fa_internal.h"

namespace {

constexpr int64_t kMaxI32 = std::numeric_limits<int32_t>::max();
constexpr int kMaxSplits = 65536;
constexpr int64_t kMaxHeadBytes = int64_t(1) << 31;

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > std::numeric_limits<int64_t>::max() / a) return false;
    *out = a * b;
    return true;
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool supported_dim(int64_t x) { return x == 32 || x == 64 || x == 128 || x == 256; }
bool supported_dims(int64_t d, int64_t dv) { return supported_dim(d) && supported_dim(dv); }

// Checks shared by both entry points.  Order: invalid arguments first, then
// the support matrix.
fa_status_t check_common(const void *q, const void *k, const void *v, const void *o,
                         const float *lse, int64_t B, int64_t H, int64_t N, int64_t Nk,
                         int64_t d, int64_t dv, float scale, fa_dtype_t dtype) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || N < 1 || Nk < 1 || d < 1 || dv < 1) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
        return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(lse, 4))
        return FA_ERR_INVALID_ARG;
    // Element counts must be representable; indices inside one head are
    // 32-bit in the kernels, and so are the workgroup counts.
    int64_t heads, t1, t2, t3, t4, t5;
    if (!mul_ok(B, H, &heads) || heads > kMaxI32) return FA_ERR_INVALID_ARG;
    if (!mul_ok(N, d, &t1) || !mul_ok(Nk, d, &t2) || !mul_ok(Nk, dv, &t3) || !mul_ok(N, dv, &t4))
        return FA_ERR_INVALID_ARG;
    if (t1 > kMaxI32 || t2 > kMaxI32 || t3 > kMaxI32 || t4 > kMaxI32) return FA_ERR_INVALID_ARG;
    if (!mul_ok(heads, N, &t5) || t5 > kMaxI32) return FA_ERR_INVALID_ARG;
    int64_t total;
    if (!mul_ok(heads, t2 > t3 ? t2 : t3, &total) || !mul_ok(heads, t1 > t4 ? t1 : t4, &total))
        return FA_ERR_INVALID_ARG;
    if (!supported_dims(d, dv)) return FA_ERR_UNSUPPORTED;
    // Kernels address one head's tensors with 32-bit byte offsets and treat
    // offsets of 3 GiB and more as "outside": each per-head tensor must stay
    // below 2 GiB.
    const int64_t esize = dtype == FA_DTYPE_F32 ? 4 : 2;
    const int64_t per_head_max = t1 > t2 ? (t1 > t3 ? (t1 > t4 ? t1 : t4) : (t3 > t4 ? t3 : t4))
                                         : (t2 > t3 ? (t2 > t4 ? t2 : t4) : (t3 > t4 ? t3 : t4));
    if (per_head_max * esize >= kMaxHeadBytes) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

fa::FwdArgs make_args(const void *q, const void *k, const void *v, void *o, float *lse,
                      int64_t B, int64_t H, int64_t N, int64_t Nk, int64_t d, int64_t dv,
                      int causal, float scale, fa_dtype_t dtype, void *stream) {
    fa::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.B = B;
    a.H = H;
    a.N = N;
    a.Nk = Nk;
    a.d = d;
    a.dv = dv;
    a.causal = causal ? 1 : 0;
    a.scale = scale;
    a.dtype = static_cast<int>(dtype);
    a.stream = static_cast<hipStream_t>(stream);
    return a;
}

// Automatic split count (num_splits = 0).  The smallest power of two S such
// that the segment kernel has at least kAutoWorkgroups workgroups (one full
// round of resident workgroups of the matrix-core kernel: 2 per CU x 256),
// halving the segments only while they keep at least kAutoMinKeys keys, and
// at most kAutoMaxSplits.  The constants were fitted to a sweep of measured
// decode times over split counts on MI355X (plain and grouped heads, 1 and 4
// queries, 1K to 256K keys): on each of the sweep's 66 shapes the rule's
// time is within 10% of the best split count's (1.5% on average).
constexpr int64_t kAutoWorkgroups = 512;
constexpr int64_t kAutoMinKeys = 256;
constexpr int kAutoMaxSplits = 256;

int auto_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t Nk, int64_t d, int64_t dv,
                int dtype) {
    const int64_t rows = (Hq / Hkv) * N;
    const int64_t units = fa::decode_workgroups_per_split(dtype, d, dv, B, Hkv, rows);
    int S = 1;
    while (S < kAutoMaxSplits && units * S < kAutoWorkgroups && Nk >= 2 * S * kAutoMinKeys) S *= 2;
    return S;
}

bool valid_dtype(fa_dtype_t dtype) {
    return dtype == FA_DTYPE_F32 || dtype == FA_DTYPE_F16 || dtype == FA_DTYPE_BF16;
}

// Keys per decode segment: ceil(Nk / S) rounded up to a multiple of 64.
int64_t segment_length(int64_t Nk, int num_splits) {
    int64_t per = (Nk + num_splits - 1) / num_splits;
    return ((per + 63) / 64) * 64;
}

}  // namespace

extern "C" {

fa_status_t fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                   int64_t B, int64_t H, int64_t N, int64_t Nk, int64_t d, int64_t dv,
                   int causal, float scale, fa_dtype_t dtype, void *stream) {
    fa_status_t st = check_common(q, k, v, o, lse, B, H, N, Nk, d, dv, scale, dtype);
    if (st != FA_OK) return st;
    fa::FwdArgs a = make_args(q, k, v, o, lse, B, H, N, Nk, d, dv, causal, scale, dtype, stream);
    (void)hipGetLastError();   // clear any stale error so it is not reported as ours
    // fp32: the VALU kernel (the 2e-5 bar needs fp32 operands); bf16/fp16:
    // the tuned matrix-core kernels where they apply, else the generic one.
    hipError_t e = dtype == FA_DTYPE_F32                         ? fa::launch_fwd_rowwise(a)
                   : !fa::fwd_mfma_supported(a.dtype, d, dv, scale) ? fa::launch_fwd_mfma_generic(a)
                   : fa::fwd_wide_preferred(d, dv, Nk)              ? fa::launch_fwd_mfma_wide(a)
                                                                   : fa::launch_fwd_mfma16(a);
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_decode_splitkv_workspace_size(int64_t B, int64_t H, int64_t N, int64_t dv,
                                        int num_splits) {
    if (B < 1 || H < 1 || N < 1 || dv < 1 || num_splits < 1) return 0;
    // rows = B H S N; bytes = rows (dv + 1) 4, formed without signed overflow
    int64_t rows, x;
    if (!mul_ok(B, H, &rows) || !mul_ok(rows, num_splits, &rows) || !mul_ok(rows, N, &rows) ||
        !mul_ok(rows, dv, &x) || x > std::numeric_limits<int64_t>::max() - rows)
        return 0;
    x += rows;
    if (!mul_ok(x, 4, &x)) return 0;
    if ((uint64_t)x > (uint64_t)std::numeric_limits<size_t>::max()) return 0;
    return static_cast<size_t>(x);
}

}  // extern "C"

namespace {

static_assert(fa::kDecodeScratchBytes == FA_DECODE_NOALLOC_MAX_WORKSPACE, "scratch size");

// use_scratch: the partials go to the device's static scratch (the
// allocation-free entry point) instead of `workspace`.
fa_status_t decode_impl(const void *q, const void *k, const void *v, void *o, float *lse,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t Nk, int64_t d,
                        int64_t dv, int causal, float scale, fa_dtype_t dtype, int num_splits,
                        void *workspace, size_t workspace_bytes, void *stream,
                        bool use_scratch = false) {
    if (num_splits < 0) return FA_ERR_INVALID_ARG;
    if (Hkv < 1 || Hq < 1 || Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
    fa_status_t st = check_common(q, k, v, o, lse, B, Hq, N, Nk, d, dv, scale, dtype);
    if (st != FA_OK) return st;
    if (num_splits == 0) num_splits = auto_splits(B, Hq, Hkv, N, Nk, d, dv, dtype);
    // Launch-shape limits of the segment kernel: (segment, key/value head,
    // row group of up to 8 of the (Hq / Hkv) x N rows).
    const int64_t rows = (Hq / Hkv) * N;
    if (B * Hkv > 65535 || (rows + 7) / 8 > 65535 || rows > kMaxI32 || num_splits > kMaxSplits)
        return FA_ERR_UNSUPPORTED;
    const size_t need = fa_decode_splitkv_workspace_size(B, Hq, N, dv, num_splits);
    if (need == 0) return FA_ERR_INVALID_ARG;
    if (use_scratch) {
        if (need > fa::kDecodeScratchBytes) return FA_ERR_WORKSPACE;
    } else if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) {
        return FA_ERR_WORKSPACE;
    }
    if (use_scratch && fa::decode_scratch(&workspace) != hipSuccess) return FA_ERR_LAUNCH;
    fa::DecodeArgs dargs;
    dargs.a = make_args(q, k, v, o, lse, B, Hq, N, Nk, d, dv, causal, scale, dtype, stream);
    dargs.Hkv = Hkv;
    dargs.num_splits = num_splits;
    dargs.seg_len = segment_length(Nk, num_splits);
    dargs.ws_o = static_cast<float *>(workspace);
    dargs.ws_lse = dargs.ws_o + B * Hq * (int64_t)num_splits * N * dv;
    (void)hipGetLastError();
    hipError_t e = fa::launch_decode_splitkv(dargs);
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

fa_status_t fa_decode_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                              int64_t B, int64_t H, int64_t N, int64_t Nk, int64_t d,
                              int64_t dv, int causal, float scale, fa_dtype_t dtype,
                              int num_splits, void *workspace, size_t workspace_bytes,
                              void *stream) {
    return decode_impl(q, k, v, o, lse, B, H, H, N, Nk, d, dv, causal, scale, dtype, num_splits,
                       workspace, workspace_bytes, stream);
}

fa_status_t fa_decode_splitkv_noalloc(const void *q, const void *k, const void *v, void *o,
                                      float *lse, int64_t B, int64_t H, int64_t N, int64_t Nk,
                                      int64_t d, int64_t dv, int causal, float scale,
                                      fa_dtype_t dtype, int num_splits, void *stream) {
    return decode_impl(q, k, v, o, lse, B, H, H, N, Nk, d, dv, causal, scale, dtype, num_splits,
                       nullptr, 0, stream, true);
}

fa_status_t fa_decode_splitkv_gqa(const void *q, const void *k, const void *v, void *o,
                                  float *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                                  int64_t Nk, int64_t d, int64_t dv, int causal, float scale,
                                  fa_dtype_t dtype, int num_splits, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    return decode_impl(q, k, v, o, lse, B, Hq, Hkv, N, Nk, d, dv, causal, scale, dtype,
                       num_splits, workspace, workspace_bytes, stream);
}

size_t fa_bwd_workspace_size(int64_t B, int64_t H, int64_t N) {
    if (B < 1 || H < 1 || N < 1) return 0;
    int64_t x;
    if (!mul_ok(B, H, &x) || !mul_ok(x, N, &x) || !mul_ok(x, 8, &x)) return 0;
    if ((uint64_t)x > (uint64_t)std::numeric_limits<size_t>::max()) return 0;
    return static_cast<size_t>(x);
}

fa_status_t fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dout, void *dq, void *dk, void *dv, int64_t B, int64_t H,
                   int64_t N, int64_t Nk, int64_t d, int64_t dv_dim, int causal, float scale,
                   fa_dtype_t dtype, void *workspace, size_t workspace_bytes, void *stream) {
    // o and lse are inputs here; check_common treats them like the forward's outputs.
    fa_status_t st = check_common(q, k, v, o, lse, B, H, N, Nk, d, dv_dim, scale, dtype);
    if (st != FA_OK) return st;
    if (!dout || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
    if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
        return FA_ERR_INVALID_ARG;
    if (B * H * ((N > Nk ? N : Nk) + 3) / 4 > kMaxI32) return FA_ERR_UNSUPPORTED;
    const size_t need = fa_bwd_workspace_size(B, H, N);
    if (need == 0) return FA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return FA_ERR_WORKSPACE;
    fa::BwdArgs b;
    b.a = make_args(q, k, v, const_cast<void *>(o), const_cast<float *>(lse), B, H, N, Nk, d,
                    dv_dim, causal, scale, dtype, stream);
    b.dout = dout;
    b.dq = dq;
    b.dk = dk;
    b.dv = dv;
    b.Dsum = static_cast<float *>(workspace);
    (void)hipGetLastError();
    hipError_t e = fa::launch_bwd(b);
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_decode_splitkv_auto_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t Nk,
                                  int64_t d, int64_t dv, fa_dtype_t dtype) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || N < 1 || Nk < 1 || d < 1 || dv < 1 ||
        !valid_dtype(dtype))
        return 0;
    int64_t t;
    if (!mul_ok(B, Hq, &t) || t > kMaxI32 || !mul_ok(Hq / Hkv, N, &t) || t > kMaxI32) return 0;
    return auto_splits(B, Hq, Hkv, N, Nk, d, dv, dtype);
}

const char *fa_status_string(fa_status_t status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
        case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH";
    }
    return "FA_UNKNOWN_STATUS";
}

}  // extern "C"
