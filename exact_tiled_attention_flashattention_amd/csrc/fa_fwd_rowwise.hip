// fa_fwd_rowwise.hip -- row-parallel exact attention forward on the VALU.
//
// The general path of fa_fwd: every dtype, d and dv in {32, 64, 128, 256}
// (dv may differ from d).  It is the path for fp32 inputs, which the
// bf16/fp16 matrix cores cannot take without losing the fp32 accuracy, and
// for every (d, dv) the matrix-core kernels do not take.
//
// Method: the FlashAttention-2 loop order of CS349E Lecture 11
// "flash_lab.py", section 3 (flash_fwd, order "fa2"): a workgroup owns a
// block of query rows, keeps their softmax state (m, l) and output
// accumulator on chip, and streams the head's K/V tiles through LDS; each
// tile updates the state with the online-softmax rescaling of section 1
// (softmax_online).  The division by l happens once at the end and
// LSE = m + ln l is written next to O.  Causal tiles beyond the block's last
// visible key are never loaded.
//
// Mapping: 4 lanes per query row (lane s of the quad owns head dims
// c*4 + s), 64 rows per 256-thread workgroup; K/V tiles of 32 keys are
// widened to fp32 in LDS, where the quad's four lanes read four consecutive
// words (distinct banks) and all rows share them (broadcast).  Scores live
// in the base-2 domain: s' = (q.k) * scale * log2(e), so that p = 2^(s'-m').
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 4;
constexpr int kRowsPerBlock = kThreads / kLanesPerRow;   // 64
constexpr int kTileKeys = 32;

template <typename T, int D, int DV>
__global__ __launch_bounds__(kThreads) void fwd_rowwise_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    T *__restrict__ o, float *__restrict__ lse, int N, int Nk, int causal,
    float scale_log2, int q_blocks) {
    constexpr int DS = D / kLanesPerRow;    // dims of q/k owned by one lane
    constexpr int DVS = DV / kLanesPerRow;  // dims of v/o owned by one lane
    __shared__ float ks[kTileKeys * D];
    __shared__ float vs[kTileKeys * DV];

    const int tid = threadIdx.x;
    const int sub = tid % kLanesPerRow;
    const int head = blockIdx.x / q_blocks;
    const int qblk = blockIdx.x % q_blocks;
    const int row0 = qblk * kRowsPerBlock;
    const int row = row0 + tid / kLanesPerRow;
    const bool row_ok = row < N;

    const T *qh = q + (int64_t)head * N * D;
    const T *kh = k + (int64_t)head * Nk * D;
    const T *vh = v + (int64_t)head * Nk * DV;

    float qr[DS];
#pragma unroll
    for (int c = 0; c < DS; ++c)
        qr[c] = row_ok ? to_f32(qh[(int64_t)row * D + c * kLanesPerRow + sub]) : 0.f;

    // Keys this block may see: all, or up to the position of its last row.
    const int last_row = min(row0 + kRowsPerBlock, N) - 1;
    int key_end = Nk;
    if (causal) key_end = min(Nk, Nk - N + last_row + 1);   // may be <= 0
    // Position of this row; keys beyond it are masked.
    const int row_limit = causal ? (Nk - N + row) : (Nk - 1);

    float m = -INFINITY;   // running max of s' (base-2 domain)
    float l = 0.f;         // running sum of 2^(s' - m)
    float acc[DVS];
#pragma unroll
    for (int c = 0; c < DVS; ++c) acc[c] = 0.f;

    for (int j0 = 0; j0 < key_end; j0 += kTileKeys) {
        const int nkeys = min(kTileKeys, key_end - j0);
        __syncthreads();   // previous tile fully consumed
        for (int e = tid; e < kTileKeys * D; e += kThreads) {
            int j = e / D;
            ks[e] = j < nkeys ? to_f32(kh[(int64_t)(j0 + j) * D + e % D]) : 0.f;
        }
        for (int e = tid; e < kTileKeys * DV; e += kThreads) {
            int j = e / DV;
            vs[e] = j < nkeys ? to_f32(vh[(int64_t)(j0 + j) * DV + e % DV]) : 0.f;
        }
        __syncthreads();

        float s[kTileKeys];
        float tile_max = -INFINITY;
#pragma unroll
        for (int j = 0; j < kTileKeys; ++j) {
            float part = 0.f;
#pragma unroll
            for (int c = 0; c < DS; ++c) part = fmaf(qr[c], ks[j * D + c * kLanesPerRow + sub], part);
            float dot = group_sum<kLanesPerRow>(part);
            bool vis = (j < nkeys) && (j0 + j <= row_limit);
            s[j] = vis ? dot * scale_log2 : -INFINITY;
            tile_max = fmaxf(tile_max, s[j]);
        }
        const float m_new = fmaxf(m, tile_max);
        // Guards of the online update: nothing seen yet -> carry factor 0;
        // everything masked so far -> subtract 0 instead of -inf.
        const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - m_new);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        l *= alpha;
#pragma unroll
        for (int c = 0; c < DVS; ++c) acc[c] *= alpha;
#pragma unroll
        for (int j = 0; j < kTileKeys; ++j) {
            float p = fast_exp2(s[j] - m_use);
            l += p;
#pragma unroll
            for (int c = 0; c < DVS; ++c) acc[c] = fmaf(p, vs[j * DV + c * kLanesPerRow + sub], acc[c]);
        }
        m = m_new;
    }

    if (!row_ok) return;
    T *orow = o + ((int64_t)head * N + row) * DV;
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int c = 0; c < DVS; ++c) orow[c * kLanesPerRow + sub] = from_f32<T>(acc[c] * inv_l);
    if (sub == 0)
        lse[(int64_t)head * N + row] = l > 0.f ? (m + fast_log2(l)) * kLn2 : -INFINITY;
}

template <typename T, int D, int DV>
hipError_t launch_typed(const FwdArgs &a) {
    const int q_blocks = (int)((a.N + kRowsPerBlock - 1) / kRowsPerBlock);
    const int64_t grid = a.B * a.H * q_blocks;
    hipLaunchKernelGGL((fwd_rowwise_kernel<T, D, DV>), dim3((unsigned)grid), dim3(kThreads), 0,
                       a.stream, static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), static_cast<T *>(a.o), a.lse, (int)a.N,
                       (int)a.Nk, a.causal, a.scale * kLog2e, q_blocks);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dv(const FwdArgs &a) {
    switch (a.dv) {
        case 32: return launch_typed<T, D, 32>(a);
        case 64: return launch_typed<T, D, 64>(a);
        case 128: return launch_typed<T, D, 128>(a);
        case 256: return launch_typed<T, D, 256>(a);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_dim(const FwdArgs &a) {
    switch (a.d) {
        case 32: return launch_dv<T, 32>(a);
        case 64: return launch_dv<T, 64>(a);
        case 128: return launch_dv<T, 128>(a);
        case 256: return launch_dv<T, 256>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fwd_rowwise(const FwdArgs &a) {
    switch (a.dtype) {
        case kF32: return launch_dim<float>(a);
        case kF16: return launch_dim<f16_t>(a);
        case kBF16: return launch_dim<bf16_t>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
