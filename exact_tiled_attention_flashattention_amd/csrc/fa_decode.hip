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
// head, row group), rows counted over the G query heads x N queries): a key row of D elements is read as 16-byte pieces by LPK
// consecutive lanes (bf16/fp16 d=128: 16 lanes), so one load instruction of
// a wave covers KPL = 64/LPK consecutive keys -- a contiguous 1 KiB of K or
// V.  Each "key slot" (group of LPK lanes) keeps its own online-softmax
// state (m, l, o) for every query row it serves, so the loop needs no
// cross-slot exchange; the dot product of a key is summed over its LPK
// lanes with DPP.  At the end the 4 waves x KPL slot states are merged
// through LDS with the same merge rule.  The loop issues U loads of K and
// U of V per lane before using them, to keep enough bytes in flight for
// HBM bandwidth.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kUnroll = 8;   // loads of K (and of V) in flight per lane per step
// A buffer offset beyond any head's K/V extent (at most 2^31 bytes).
constexpr uint32_t kOutOfRange = 0xC0000000u;

template <typename T, int D, int R>
__global__ __launch_bounds__(kThreads) void decode_segment_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    float *__restrict__ ws_o, float *__restrict__ ws_lse, int N, int Nk, int causal,
    float scale_log2, int num_splits, int seg_len, int G) {
    constexpr int EPL = 16 / (int)sizeof(T);   // elements per 16-byte piece
    constexpr int LPK = D / EPL;               // lanes per key row
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
    const int t = lane % LPK;      // which 16-byte piece of the row

    const T *kh = k + (int64_t)kvh * Nk * D;
    const T *vh = v + (int64_t)kvh * Nk * D;

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
        if (ok) raw = *reinterpret_cast<const u32x4 *>(q + (qhead * N + row) * D + t * EPL);
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
    const auto vrs = make_rsrc(vh, (uint32_t)Nk * D * (uint32_t)sizeof(T));

    // Waves take consecutive steps of KEYS_PER_STEP keys round-robin.
    for (int base = seg_begin + wave * KEYS_PER_STEP; base < seg_end;
         base += kWaves * KEYS_PER_STEP) {
        u32x4 kraw[kUnroll], vraw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int key = base + u * KPL + slot;
            const uint32_t off = key < seg_end
                                     ? ((uint32_t)key * D + t * EPL) * (uint32_t)sizeof(T)
                                     : kOutOfRange;
            kraw[u] = buffer_load16(krs, off);
            vraw[u] = buffer_load16(vrs, off);
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
    __shared__ float sm_o[R][STATES][D];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int st = wave * KPL + slot;
        if (t == 0) {
            sm_m[r][st] = m[r];
            sm_l[r][st] = l[r];
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) sm_o[r][st][t * EPL + i] = acc[r][i];
    }
    __syncthreads();
    for (int idx = tid; idx < R * D; idx += kThreads) {
        const int r = idx / D;
        const int c = idx % D;
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
        // Workspace layout: o_s [B*Hq, S, N, D], lse_s [B*Hq, S, N].
        const int64_t part = (qhead * num_splits + split) * N + row;
        ws_o[part * D + c] = ll > 0.f ? oo / ll : 0.f;
        if (c == 0) ws_lse[part] = ll > 0.f ? (mm + fast_log2(ll)) * kLn2 : -INFINITY;
    }
}

// One workgroup of 4 waves per (head, row): merge num_splits partial states.
// Every lane first takes some segments' lse_s to find M = max lse_s and
// Z = sum exp(lse_s - M) (wave reductions, then across the 4 waves through
// LDS); then the weights w_s = exp(lse_s - lse) of a chunk of 64 segments
// are computed once, one per lane, and staged in LDS, and each wave
// accumulates w_s * o_s over its share of the chunk's segments with the
// row's columns spread over its lanes; the 4 partial sums meet in LDS.
constexpr int kMergeWaves = 4;

template <typename T, int D>
__global__ __launch_bounds__(kMergeWaves * 64) void decode_merge_kernel(
    const float *__restrict__ ws_o, const float *__restrict__ ws_lse, T *__restrict__ o,
    float *__restrict__ lse, int N, int num_splits) {
    constexpr int CPL = D >= 64 ? D / 64 : 1;      // columns per lane
    const int64_t hr = blockIdx.x;                  // head * N + row
    const int64_t head = hr / N;
    const int row = (int)(hr % N);
    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int64_t base = head * (int64_t)num_splits * N + row;   // segment s at base + s*N
    __shared__ float red[2][kMergeWaves];
    __shared__ float wts[64];
    __shared__ float part[kMergeWaves][D];

    float mx = -INFINITY;
    for (int s = tid; s < num_splits; s += kMergeWaves * 64) mx = fmaxf(mx, ws_lse[base + (int64_t)s * N]);
    mx = group_max<64>(mx);
    if (lane == 0) red[0][wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    T *orow = o + hr * D;
    if (mx == -INFINITY) {   // no visible key in any segment
        for (int c = tid; c < D; c += kMergeWaves * 64) orow[c] = from_f32<T>(0.f);
        if (tid == 0) lse[hr] = -INFINITY;
        return;
    }
    float z = 0.f;
    for (int s = tid; s < num_splits; s += kMergeWaves * 64) z += expf(ws_lse[base + (int64_t)s * N] - mx);
    z = group_sum<64>(z);
    if (lane == 0) red[1][wave] = z;
    __syncthreads();
    z = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    const float total = mx + logf(z);

    float acc[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
    const int col0 = lane * CPL;
    for (int s0 = 0; s0 < num_splits; s0 += 64) {
        const int cnt = min(64, num_splits - s0);
        __syncthreads();   // previous chunk's weights consumed
        if (tid < cnt) wts[tid] = expf(ws_lse[base + (int64_t)(s0 + tid) * N] - total);   // 0 if empty
        __syncthreads();
        if (col0 < D) {
#pragma unroll 4
            for (int i = wave; i < cnt; i += kMergeWaves) {
                const float w = wts[i];
                const float *src = ws_o + (base + (int64_t)(s0 + i) * N) * D + col0;
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[c] = fmaf(w, src[c], acc[c]);
            }
        }
    }
    if (col0 < D) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) part[wave][col0 + c] = acc[c];
    }
    __syncthreads();
    for (int c = tid; c < D; c += kMergeWaves * 64)
        orow[c] = from_f32<T>((part[0][c] + part[1][c]) + (part[2][c] + part[3][c]));
    if (tid == 0) lse[hr] = total;
}

template <typename T, int D, int R>
hipError_t launch_rows(const DecodeArgs &d) {
    const FwdArgs &a = d.a;
    const int G = (int)(a.H / d.Hkv);
    const int64_t groups = ((int64_t)G * a.N + R - 1) / R;
    dim3 grid((unsigned)d.num_splits, (unsigned)(a.B * d.Hkv), (unsigned)groups);
    hipLaunchKernelGGL((decode_segment_kernel<T, D, R>), grid, dim3(kThreads), 0, a.stream,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), d.ws_o, d.ws_lse, (int)a.N, (int)a.Nk,
                       a.causal, a.scale * kLog2e, d.num_splits, (int)d.seg_len, G);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)(a.B * a.H * a.N)),
                       dim3(kMergeWaves * 64),
                       0, a.stream, d.ws_o, d.ws_lse, static_cast<T *>(a.o), a.lse, (int)a.N,
                       d.num_splits);
    return hipGetLastError();
}

// Rows per workgroup: the smallest of 1, 2, 4, 8 that covers the G x N rows
// of a key/value head (8 at most; more rows take more workgroups).
template <typename T, int D>
hipError_t launch_dim(const DecodeArgs &d) {
    const int64_t rows = (d.a.H / d.Hkv) * d.a.N;
    if (rows == 1) return launch_rows<T, D, 1>(d);
    if (rows == 2) return launch_rows<T, D, 2>(d);
    if (rows <= 4) return launch_rows<T, D, 4>(d);
    return launch_rows<T, D, 8>(d);
}

template <typename T>
hipError_t launch_typed(const DecodeArgs &d) {
    switch (d.a.d) {
        case 32: return launch_dim<T, 32>(d);
        case 64: return launch_dim<T, 64>(d);
        case 128: return launch_dim<T, 128>(d);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_splitkv(const DecodeArgs &d) {
    switch (d.a.dtype) {
        case kF32: return launch_typed<float>(d);
        case kF16: return launch_typed<f16_t>(d);
        case kBF16: return launch_typed<bf16_t>(d);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
