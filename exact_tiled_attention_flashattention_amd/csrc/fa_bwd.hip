// fa_bwd.hip -- attention backward: the row-dot kernel and the VALU
// (any dtype) gradient kernels, plus the launcher that picks them or the
// matrix-core kernels of fa_bwd_mfma.hip.
//
// Method: CS349E Lecture 11 "flash_lab.py", section 3 (flash_bwd, the
// FlashAttention-2 backward): the N x Nk probabilities are not stored by the
// forward; they are recomputed on chip from Q, K and the forward's LSE as
// P_ij = exp(S_ij - LSE_i).  With D_i = sum_c dO_ic O_ic (one number per
// row, computed first):
//     dV_j += P_ij dO_i,   dP_ij = dO_i . V_j,   dS_ij = P_ij (dP_ij - D_i),
//     dQ_i += scale dS_ij K_j,   dK_j += scale dS_ij Q_i.
// The pages accumulate dQ into device memory inside the loop over key
// blocks; here dQ and (dK, dV) are produced by two separate kernels, one
// looping over keys for a query row and one over query rows for a key, so no
// location is written by more than one workgroup and the result is
// deterministic.  The price is that S, P and dP are recomputed in both.
//
// The VALU kernels here serve fp32, whose 2e-5 bar needs fp32 operands (the
// matrix-core kernels take every bf16/fp16 (d, dv)): one wave per query row
// (dQ) or per key (dK, dV), the head dimension spread over the lanes, dot
// products summed over the wave.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

// D_i = sum_c dO_ic O_ic in fp32.  A row is read as 16-byte pieces by
// LPR = DV * sizeof(T) / 16 consecutive lanes; 256 / LPR rows per workgroup.
template <typename T, int DV>
__global__ __launch_bounds__(256) void bwd_dot_kernel(const T *__restrict__ o,
                                                      const T *__restrict__ dout,
                                                      float *__restrict__ D, int64_t rows) {
    constexpr int EPL = 16 / (int)sizeof(T);
    constexpr int LPR = DV / EPL;
    static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "row split");
    const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
    const int t = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(o + row * DV + t * EPL);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(dout + row * DV + t * EPL);
        const T *ea = reinterpret_cast<const T *>(&a);
        const T *eb = reinterpret_cast<const T *>(&b);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(to_f32(ea[e]), to_f32(eb[e]), acc);
    }
    acc = group_sum<LPR>(acc);
    if (row < rows && t == 0) D[row] = acc;
}

// dQ: one wave per query row.
template <typename T, int D, int DV>
__global__ __launch_bounds__(256) void bwd_dq_rowwise_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ lse, const T *__restrict__ dout, const float *__restrict__ Dsum,
    T *__restrict__ dq, int64_t heads, int N, int Nk, int causal, float scale) {
    constexpr int E = (D + 63) / 64, EV = (DV + 63) / 64;
    const int64_t gw = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 64;   // head * N + row
    const int lane = threadIdx.x % 64;
    if (gw >= heads * N) return;   // whole waves exit together
    const int64_t head = gw / N;
    const int i = (int)(gw % N);
    const T *qi = q + gw * D;
    const T *di = dout + gw * DV;
    const T *kh = k + head * Nk * D;
    const T *vh = v + head * Nk * DV;
    float qr[E], dr[EV], acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int c = lane + 64 * e;
        qr[e] = c < D ? to_f32(qi[c]) : 0.f;
        acc[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < EV; ++e) {
        const int c = lane + 64 * e;
        dr[e] = c < DV ? to_f32(di[c]) : 0.f;
    }
    const float L = lse[gw];
    const float Di = Dsum[gw];
    const int last = causal ? min(Nk - 1, Nk - N + i) : Nk - 1;
    if (L != -INFINITY) {
        for (int j = 0; j <= last; ++j) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int c = lane + 64 * e;
                if (c < D) s = fmaf(qr[e], to_f32(kh[(int64_t)j * D + c]), s);
            }
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                const int c = lane + 64 * e;
                if (c < DV) dp = fmaf(dr[e], to_f32(vh[(int64_t)j * DV + c]), dp);
            }
            s = group_sum<64>(s);
            dp = group_sum<64>(dp);
            const float p = expf(s * scale - L);
            const float ds = p * (dp - Di) * scale;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int c = lane + 64 * e;
                if (c < D) acc[e] = fmaf(ds, to_f32(kh[(int64_t)j * D + c]), acc[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int c = lane + 64 * e;
        if (c < D) dq[gw * D + c] = from_f32<T>(acc[e]);
    }
}

// dK, dV: one wave per key.
template <typename T, int D, int DV>
__global__ __launch_bounds__(256) void bwd_dkdv_rowwise_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ lse, const T *__restrict__ dout, const float *__restrict__ Dsum,
    T *__restrict__ dk, T *__restrict__ dvo, int64_t heads, int N, int Nk, int causal,
    float scale) {
    constexpr int E = (D + 63) / 64, EV = (DV + 63) / 64;
    const int64_t gw = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 64;   // head * Nk + key
    const int lane = threadIdx.x % 64;
    if (gw >= heads * Nk) return;
    const int64_t head = gw / Nk;
    const int j = (int)(gw % Nk);
    const T *qh = q + head * N * D;
    const T *dh = dout + head * N * DV;
    const float *Lh = lse + head * N;
    const float *Dh = Dsum + head * N;
    float kr[E], vr[EV], gk[E], gv[EV];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int c = lane + 64 * e;
        kr[e] = c < D ? to_f32(k[gw * D + c]) : 0.f;
        gk[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < EV; ++e) {
        const int c = lane + 64 * e;
        vr[e] = c < DV ? to_f32(v[gw * DV + c]) : 0.f;
        gv[e] = 0.f;
    }
    // Rows that see key j: all, or (causal) those with Nk - N + i >= j.
    const int first = causal ? max(0, j - (Nk - N)) : 0;
    for (int i = first; i < N; ++i) {
        const float L = Lh[i];
        if (L == -INFINITY) continue;   // uniform over the wave
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int c = lane + 64 * e;
            if (c < D) s = fmaf(kr[e], to_f32(qh[(int64_t)i * D + c]), s);
        }
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            const int c = lane + 64 * e;
            if (c < DV) dp = fmaf(vr[e], to_f32(dh[(int64_t)i * DV + c]), dp);
        }
        s = group_sum<64>(s);
        dp = group_sum<64>(dp);
        const float p = expf(s * scale - L);
        const float ds = p * (dp - Dh[i]) * scale;
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            const int c = lane + 64 * e;
            if (c < DV) gv[e] = fmaf(p, to_f32(dh[(int64_t)i * DV + c]), gv[e]);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int c = lane + 64 * e;
            if (c < D) gk[e] = fmaf(ds, to_f32(qh[(int64_t)i * D + c]), gk[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int c = lane + 64 * e;
        if (c < D) dk[gw * D + c] = from_f32<T>(gk[e]);
    }
#pragma unroll
    for (int e = 0; e < EV; ++e) {
        const int c = lane + 64 * e;
        if (c < DV) dvo[gw * DV + c] = from_f32<T>(gv[e]);
    }
}

template <typename T, int D, int DV>
hipError_t launch_rowwise(const BwdArgs &b) {
    const FwdArgs &a = b.a;
    const int64_t heads = a.B * a.H;
    const unsigned gq = (unsigned)((heads * a.N + 3) / 4);
    hipLaunchKernelGGL((bwd_dq_rowwise_kernel<T, D, DV>), dim3(gq), dim3(256), 0, a.stream,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), a.lse, static_cast<const T *>(b.dout),
                       b.Dsum, static_cast<T *>(b.dq), heads, (int)a.N, (int)a.Nk, a.causal,
                       a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned gk = (unsigned)((heads * a.Nk + 3) / 4);
    hipLaunchKernelGGL((bwd_dkdv_rowwise_kernel<T, D, DV>), dim3(gk), dim3(256), 0, a.stream,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), a.lse, static_cast<const T *>(b.dout),
                       b.Dsum, static_cast<T *>(b.dk), static_cast<T *>(b.dv), heads,
                       (int)a.N, (int)a.Nk, a.causal, a.scale);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_rowwise_dv(const BwdArgs &b) {
    switch (b.a.dv) {
        case 32: return launch_rowwise<T, D, 32>(b);
        case 64: return launch_rowwise<T, D, 64>(b);
        case 128: return launch_rowwise<T, D, 128>(b);
        case 256: return launch_rowwise<T, D, 256>(b);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, int DV>
hipError_t launch_dot(const BwdArgs &b) {
    const FwdArgs &a = b.a;
    const int64_t rows = a.B * a.H * a.N;
    constexpr int rpb = 256 / (DV * (int)sizeof(T) / 16);   // rows per workgroup
    hipLaunchKernelGGL((bwd_dot_kernel<T, DV>), dim3((unsigned)((rows + rpb - 1) / rpb)),
                       dim3(256), 0, a.stream, static_cast<const T *>(a.o),
                       static_cast<const T *>(b.dout), b.Dsum, rows);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const BwdArgs &b) {
    const FwdArgs &a = b.a;
    // The matrix-core dQ kernel computes the row dots itself.
    if (bwd_mfma_supported(a.dtype, a.d, a.dv)) return launch_bwd_mfma(b);
    hipError_t e = a.dv == 32    ? launch_dot<T, 32>(b)
                   : a.dv == 64  ? launch_dot<T, 64>(b)
                   : a.dv == 128 ? launch_dot<T, 128>(b)
                                 : launch_dot<T, 256>(b);
    if (e != hipSuccess) return e;
    switch (a.d) {
        case 32: return launch_rowwise_dv<T, 32>(b);
        case 64: return launch_rowwise_dv<T, 64>(b);
        case 128: return launch_rowwise_dv<T, 128>(b);
        case 256: return launch_rowwise_dv<T, 256>(b);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &b) {
    switch (b.a.dtype) {
        case kF32: return launch_typed<float>(b);
        case kF16: return launch_typed<f16_t>(b);
        case kBF16: return launch_typed<bf16_t>(b);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
