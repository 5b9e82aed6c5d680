// fa_decode.hip -- split-KV flash-decoding: segment kernel + merge kernel.
//
// Method: CS349E Lecture 11 "flash_lab.py", section 4 (split_kv_decode):
// with only a few query rows per head there are too few query blocks to
// fill the GPU, so the keys are cut into segments instead; each segment is
// reduced independently to (o_s, lse_s) with o_s already normalised, and
// the segments are combined with lse = ln sum_s e^(lse_s) and
// o = sum_s e^(lse_s - lse) o_s -- section 1's merge_states written in
// log-sum-exp form.  The partials go through a workspace and a second,
// small kernel on the same stream merges them: no atomics, no inter-
// workgroup ordering (the partial-buffer pattern the lecture series uses
// to avoid racing writers).
//
// Grouped-query attention (several query heads sharing one key/value head,
// the packing the lecture recommends for decode): a workgroup serves rows
// of all G query heads of its key/value head, so K and V are read once per
// group instead of once per query head.
//
// Segment kernel mapping (one workgroup of 4 waves per (segment, key/value
// head, row group), rows counted over the G query heads x N queries): a key
// is served by LPK consecutive lanes, each holding one 16-byte piece of its
// K row and one of its V row (bf16/fp16 d = dv = 128: 16 lanes; with
// d != dv, LPK covers the longer row and the other row uses the first
// lanes), so one load instruction of a wave covers KPL = 64/LPK
// consecutive keys -- contiguous K or V rows.  Each "key slot" (group of
// LPK lanes) keeps its own online-softmax
// state (m, l, o) for every query row it serves, so the loop needs no
// cross-slot exchange; the dot product of a key is summed over its LPK
// lanes with DPP.  At the end the 4 waves x KPL slot states are merged
// through LDS with the same merge rule.  The loop issues U loads of K and
// U of V per lane before using them, to keep enough bytes in flight for
// HBM bandwidth.
#include <mutex>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kUnroll = 8;   // loads of K (and of V) in flight per lane per step
// A buffer offset beyond any head's K/V extent (at most 2^31 bytes).
constexpr uint32_t kOutOfRange = 0xC0000000u;

template <typename T, int D, int DV, int R>
__global__ __launch_bounds__(kThreads) void decode_segment_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    float *__restrict__ ws_o, float *__restrict__ ws_lse, int N, int Nk, int causal,
    float scale_log2, int num_splits, int seg_len, int G) {
    constexpr int EPL = 16 / (int)sizeof(T);   // elements per 16-byte piece
    constexpr int KP = D / EPL;                // pieces of a K row
    constexpr int VP = DV / EPL;               // pieces of a V row
    constexpr int LPK = KP > VP ? KP : VP;     // lanes per key
    constexpr int KPL = 64 / LPK;              // keys per wave load
    constexpr int KEYS_PER_STEP = KPL * kUnroll;
    static_assert(LPK >= 1 && LPK <= 64 && (64 % LPK) == 0, "bad key-row split");

    const int split = blockIdx.x;
    const int kvh = blockIdx.y;          // key/value head (over B x Hkv)
    const int row0 = blockIdx.z * R;     // first row of the group, over G x N
    const int tid = threadIdx.x;
    const int wave = tid / 64;
    const int lane = tid % 64;
    const int slot = lane / LPK;   // which key of a wave load this lane serves
    const int t = lane % LPK;      // which 16-byte piece of the K and V rows
    const bool has_k = t < KP, has_v = t < VP;   // (with d != dv some lanes hold one only)

    const T *kh = k + (int64_t)kvh * Nk * D;
    const T *vh = v + (int64_t)kvh * Nk * DV;

    // Query pieces of the R rows served by this workgroup.  Row x of the
    // group is query x % N of query head kvh * G + x / N; rows past G * N
    // are zero and see no key.
    float qr[R][EPL];
    int limit[R];   // last key index visible to each row
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int x = row0 + r;
        const bool ok = x < G * N;
        const int row = ok ? x % N : 0;
        const int64_t qhead = (int64_t)kvh * G + (ok ? x / N : 0);
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (ok && has_k) raw = *reinterpret_cast<const u32x4 *>(q + (qhead * N + row) * D + t * EPL);
        const T *e = reinterpret_cast<const T *>(&raw);
#pragma unroll
        for (int i = 0; i < EPL; ++i) qr[r][i] = to_f32(e[i]);
        limit[r] = !ok ? -1 : (causal ? Nk - N + row : Nk - 1);
    }

    const int seg_begin = split * seg_len;
    const int seg_end = min(Nk, seg_begin + seg_len);

    float m[R], l[R], acc[R][EPL];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) acc[r][i] = 0.f;
    }

    // Bounds-checked views of this head's K and V: keys past the segment
    // are pointed outside them and read as zeros, so the loads need no branch.
    const auto krs = make_rsrc(kh, (uint32_t)Nk * D * (uint32_t)sizeof(T));
    const auto vrs = make_rsrc(vh, (uint32_t)Nk * DV * (uint32_t)sizeof(T));

    // Waves take consecutive steps of KEYS_PER_STEP keys round-robin.
    for (int base = seg_begin + wave * KEYS_PER_STEP; base < seg_end;
         base += kWaves * KEYS_PER_STEP) {
        u32x4 kraw[kUnroll], vraw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int key = base + u * KPL + slot;
            const bool in = key < seg_end;
            const uint32_t koff = in && has_k ? ((uint32_t)key * D + t * EPL) * (uint32_t)sizeof(T)
                                              : kOutOfRange;
            const uint32_t voff = in && has_v ? ((uint32_t)key * DV + t * EPL) * (uint32_t)sizeof(T)
                                              : kOutOfRange;
            kraw[u] = buffer_load16_nt(krs, koff);
            vraw[u] = buffer_load16_nt(vrs, voff);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int key = base + u * KPL + slot;
            const T *ke = reinterpret_cast<const T *>(&kraw[u]);
            const T *ve = reinterpret_cast<const T *>(&vraw[u]);
            float kf[EPL], vf[EPL];
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                kf[i] = to_f32(ke[i]);
                vf[i] = to_f32(ve[i]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float part = 0.f;
#pragma unroll
                for (int i = 0; i < EPL; ++i) part = fmaf(qr[r][i], kf[i], part);
                const float dot = group_sum<LPK>(part);
                const bool vis = key < seg_end && key <= limit[r];
                const float s = vis ? dot * scale_log2 : -INFINITY;
                // Online update of this slot's state with one key.
                const float m_new = fmaxf(m[r], s);
                const float alpha = (m[r] == -INFINITY) ? 0.f : fast_exp2(m[r] - m_new);
                const float p = (s == -INFINITY) ? 0.f : fast_exp2(s - m_new);
                l[r] = l[r] * alpha + p;
#pragma unroll
                for (int i = 0; i < EPL; ++i) acc[r][i] = fmaf(acc[r][i], alpha, p * vf[i]);
                m[r] = m_new;
            }
        }
    }

    // Merge the kWaves * KPL slot states of every row through LDS.
    constexpr int STATES = kWaves * KPL;
    __shared__ float sm_m[R][STATES];
    __shared__ float sm_l[R][STATES];
    __shared__ float sm_o[R][STATES][DV];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int st = wave * KPL + slot;
        if (t == 0) {
            sm_m[r][st] = m[r];
            sm_l[r][st] = l[r];
        }
        if (has_v) {
#pragma unroll
            for (int i = 0; i < EPL; ++i) sm_o[r][st][t * EPL + i] = acc[r][i];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < R * DV; idx += kThreads) {
        const int r = idx / DV;
        const int c = idx % DV;
        const int x = row0 + r;
        if (x >= G * N) continue;
        const int row = x % N;
        const int64_t qhead = (int64_t)kvh * G + x / N;
        float mm = -INFINITY;
        for (int st = 0; st < STATES; ++st) mm = fmaxf(mm, sm_m[r][st]);
        float ll = 0.f, oo = 0.f;
        if (mm != -INFINITY) {
            for (int st = 0; st < STATES; ++st) {
                const float ms = sm_m[r][st];
                const float f = (ms == -INFINITY) ? 0.f : fast_exp2(ms - mm);
                ll = fmaf(sm_l[r][st], f, ll);
                oo = fmaf(sm_o[r][st][c], f, oo);
            }
        }
        // Workspace layout: o_s [B*Hq, S, N, DV], lse_s [B*Hq, S, N].
        const int64_t part = (qhead * num_splits + split) * N + row;
        ws_o[part * DV + c] = ll > 0.f ? oo / ll : 0.f;
        if (c == 0) ws_lse[part] = ll > 0.f ? (mm + fast_log2(ll)) * kLn2 : -INFINITY;
    }
}

// One workgroup of 4 waves per (head, row): merge num_splits partial states
// with lse = M + ln sum_s e^(lse_s - M) and o = sum_s e^(lse_s - lse) o_s.
// Each thread folds its share of the lse_s into a running (max, sum) pair;
// the pairs are combined over the wave with lane exchanges and over the 4
// waves through LDS.  The partial outputs are summed in chunks of 64
// segments, 16 per wave, each lane owning D / 64 columns; the loads of the
// first chunk are issued before the lse reduction, so the whole merge waits
// on memory about once.
constexpr int kMergeWaves = 4;
constexpr int kMergeSpw = 16;   // segments per wave per chunk

__device__ __forceinline__ void lse_fold(float &m, float &z, float x) {
    if (x == -INFINITY) return;
    if (x > m) {
        z = z * expf(m - x) + 1.f;   // m = -inf: z = 0 * 0 + 1
        m = x;
    } else {
        z += expf(x - m);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(kMergeWaves * 64) void decode_merge_kernel(
    const float *__restrict__ ws_o, const float *__restrict__ ws_lse, T *__restrict__ o,
    float *__restrict__ lse, int N, int num_splits) {
    constexpr int CPL = D >= 64 ? D / 64 : 1;      // columns per lane
    constexpr int CHUNK = kMergeWaves * kMergeSpw;
    const int64_t hr = blockIdx.x;                  // head * N + row
    const int64_t head = hr / N;
    const int row = (int)(hr % N);
    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int col0 = lane * CPL;
    const bool col_ok = col0 < D;
    const int64_t base = head * (int64_t)num_splits * N + row;   // segment s at base + s*N
    __shared__ float red[2][kMergeWaves];
    __shared__ float wts[CHUNK];
    __shared__ float part[kMergeWaves][D];

    float ov[kMergeSpw][CPL];
    auto load_chunk = [&](int s0) {
#pragma unroll
        for (int i = 0; i < kMergeSpw; ++i) {
            const int s = s0 + wave * kMergeSpw + i;
            const bool ok = col_ok && s < num_splits;
            const float *src = ws_o + (base + (int64_t)s * N) * D + col0;
#pragma unroll
            for (int c = 0; c < CPL; ++c) ov[i][c] = ok ? src[c] : 0.f;
        }
    };
    load_chunk(0);

    float mx = -INFINITY, z = 0.f, x0 = -INFINITY;
    for (int s = tid; s < num_splits; s += kMergeWaves * 64) {
        const float x = ws_lse[base + (int64_t)s * N];
        if (s == tid) x0 = x;
        lse_fold(mx, z, x);
    }
    {   // combine (max, sum) over the wave, then over the waves
        const float wm = group_max<64>(mx);
        float zz = (mx == -INFINITY) ? 0.f : z * expf(mx - wm);
        zz = group_sum<64>(zz);
        if (lane == 0) {
            red[0][wave] = wm;
            red[1][wave] = zz;
        }
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) M = fmaxf(M, red[0][w]);
    T *orow = o + hr * D;
    if (M == -INFINITY) {   // no visible key in any segment
        for (int c = tid; c < D; c += kMergeWaves * 64) orow[c] = from_f32<T>(0.f);
        if (tid == 0) lse[hr] = -INFINITY;
        return;
    }
    float Z = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w)
        Z += red[0][w] == -INFINITY ? 0.f : red[1][w] * expf(red[0][w] - M);
    const float total = M + logf(Z);

    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    for (int s0 = 0; s0 < num_splits; s0 += CHUNK) {
        if (s0 > 0) {
            load_chunk(s0);
            __syncthreads();   // previous chunk's weights consumed
        }
        if (tid < CHUNK && s0 + tid < num_splits) {
            const float x = s0 == 0 ? x0 : ws_lse[base + (int64_t)(s0 + tid) * N];
            wts[tid] = expf(x - total);   // 0 for an empty segment
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kMergeSpw; ++i) {
            const int j = wave * kMergeSpw + i;
            const float w = s0 + j < num_splits ? wts[j] : 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c] = fmaf(w, ov[i][c], acc[c]);
        }
    }
    if (col_ok) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) part[wave][col0 + c] = acc[c];
    }
    __syncthreads();
    for (int c = tid; c < D; c += kMergeWaves * 64)
        orow[c] = from_f32<T>((part[0][c] + part[1][c]) + (part[2][c] + part[3][c]));
    if (tid == 0) lse[hr] = total;
}

template <typename T, int D, int DV, int R>
hipError_t launch_segment(const DecodeArgs &d) {
    const FwdArgs &a = d.a;
    const int G = (int)(a.H / d.Hkv);
    const int64_t groups = ((int64_t)G * a.N + R - 1) / R;
    dim3 grid((unsigned)d.num_splits, (unsigned)(a.B * d.Hkv), (unsigned)groups);
    hipLaunchKernelGGL((decode_segment_kernel<T, D, DV, R>), grid, dim3(kThreads), 0, a.stream,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), d.ws_o, d.ws_lse, (int)a.N, (int)a.Nk,
                       a.causal, a.scale * kLog2e, d.num_splits, (int)d.seg_len, G);
    return hipGetLastError();
}

// Segment kernel choice.  bf16/fp16 with d, dv <= 128 or d = dv = 256, and
// at least kMfmaMinRows rows per key/value head (grouped heads, several
// queries) run on the matrix cores (fa_decode_mfma.hip): there the per-key
// work grows with the rows and the VALU kernel below would stop being bound
// by memory.
// Otherwise the VALU kernel runs with the smallest of 1, 2, 4, 8 rows per
// workgroup that covers the rows (8 at most; more rows take more workgroups).
constexpr int64_t kMfmaMinRows = 2;

bool use_mfma(int dtype, int64_t d, int64_t dv, int64_t rows) {
    return dtype != kF32 && ((d <= 128 && dv <= 128) || (d == 256 && dv == 256)) &&
           rows >= kMfmaMinRows;
}
int64_t valu_rows(int64_t rows) { return rows == 1 ? 1 : rows == 2 ? 2 : rows <= 4 ? 4 : 8; }

template <typename T, int D, int DV>
hipError_t launch_dims(const DecodeArgs &d) {
    const FwdArgs &a = d.a;
    const int64_t rows = (a.H / d.Hkv) * a.N;
    hipError_t e;
    if (use_mfma(a.dtype, a.d, a.dv, rows)) e = launch_decode_segment_mfma(d);
    else if (valu_rows(rows) == 1) e = launch_segment<T, D, DV, 1>(d);
    else if (valu_rows(rows) == 2) e = launch_segment<T, D, DV, 2>(d);
    else if (valu_rows(rows) == 4) e = launch_segment<T, D, DV, 4>(d);
    else e = launch_segment<T, D, DV, 8>(d);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_kernel<T, DV>), dim3((unsigned)(a.B * a.H * a.N)),
                       dim3(kMergeWaves * 64), 0, a.stream, d.ws_o, d.ws_lse,
                       static_cast<T *>(a.o), a.lse, (int)a.N, d.num_splits);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dv(const DecodeArgs &d) {
    switch (d.a.dv) {
        case 32: return launch_dims<T, D, 32>(d);
        case 64: return launch_dims<T, D, 64>(d);
        case 128: return launch_dims<T, D, 128>(d);
        case 256: return launch_dims<T, D, 256>(d);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_typed(const DecodeArgs &d) {
    switch (d.a.d) {
        case 32: return launch_dv<T, 32>(d);
        case 64: return launch_dv<T, 64>(d);
        case 128: return launch_dv<T, 128>(d);
        case 256: return launch_dv<T, 256>(d);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int64_t decode_workgroups_per_split(int dtype, int64_t d, int64_t dv, int64_t B, int64_t Hkv,
                                    int64_t rows) {
    const int64_t per = use_mfma(dtype, d, dv, rows) ? kDecodeMfmaRows : valu_rows(rows);
    return B * Hkv * ((rows + per - 1) / per);
}

hipError_t launch_decode_splitkv(const DecodeArgs &d) {
    switch (d.a.dtype) {
        case kF32: return launch_typed<float>(d);
        case kF16: return launch_typed<f16_t>(d);
        case kBF16: return launch_typed<bf16_t>(d);
        default: return hipErrorInvalidValue;
    }
}

// ---- scratch of the allocation-free entry point ----------------------------
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops), the segment partials go to this fixed array instead
// of a caller's workspace.  Each device holds its own copy from module load
// until the process ends.  In host code the name `scratch` is only a host
// stand-in, so its device address is looked up once per device, with that
// device current, and only that address is ever passed to a kernel.  Every
// call on a device shares the array: calls that overlap on one device race.
// No part of it needs clearing: the segment kernels write every partial the
// merge kernel reads (empty segments as lse = -inf, o = 0).
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace fa
