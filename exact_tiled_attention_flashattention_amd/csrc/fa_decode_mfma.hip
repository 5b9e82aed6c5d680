// fa_decode_mfma.hip -- split-KV decode segment kernel on the matrix cores
// (bf16/fp16 inputs, d and dv in {32, 64, 128}, and d = dv = 256; fp32
// accumulation).
//
// Method: CS349E Lecture 11 "flash_lab.py", section 4 (split_kv_decode):
// each (segment, key/value head) is reduced to a normalised partial output
// o_s and its lse_s; the merge kernel in fa_decode.hip combines them.  With
// grouped-query attention all (Hq / Hkv) x N query rows of a key/value head
// share one pass over the segment's K and V (the packing the lecture
// recommends for decode), which turns the per-key work into small matrix
// products: this kernel runs them on v_mfma_f32_16x16x32_{bf16,f16}.
//
// Mapping (a persistent grid of workgroups of 4 waves, each walking units of
// (segment, key/value head, 16-row tile); rows are counted over query heads
// x queries of the group):
//  * The waves take 32-key blocks of the segment round-robin; each keeps its
//    own online-softmax state per row (section 1's rescaling rule, in base
//    2 with the scale folded in).  A block of K and of V is fetched with
//    16-byte loads of whole consecutive rows (1 KiB per wave instruction,
//    non-temporal: each byte is read once) into registers, one block ahead
//    of the block being computed, and is then written row-major to the
//    wave's own LDS buffers.
//  * Scores are formed transposed, S^T = K Q^T: the 16 query rows are the
//    MFMA columns (lane & 15), 16 keys the MFMA rows; the A operand (K) is
//    read from LDS with ds_read_b128, the B operand (Q^T) is loaded once.
//  * O^T += V^T P^T: P comes straight from the score registers as the B
//    operand, reading the contraction index as the key order
//    {4g..4g+3, 16+4g..16+4g+3}; V^T is read from LDS with
//    ds_read_b64_tr_b16.  Rows are XOR-swizzled in 16-byte (K) and 8-byte
//    (V) units so that both kinds of read are free of bank conflicts.
//  * At the end of a unit the 4 wave states of each row are merged through
//    LDS with the same rule and written to the workspace as (o_s, lse_s).
//    The next unit's first block and Q rows are already being fetched then,
//    so a workgroup streams from one unit into the next without a gap.
//  * d = dv = 256: a block is 32 KiB of K and V per wave, so one register
//    set holds the block in flight (the next block's loads are issued right
//    after the current block has moved to LDS), and one workgroup of 4
//    waves per CU has the 128 KiB of LDS and one wave per SIMD the
//    registers; the 4 waves' independent streams keep 128 KiB per CU in
//    flight.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
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
constexpr int kRows = kDecodeMfmaRows;    // query rows per workgroup (16)
constexpr int kBlk = 32;                  // keys per wave step
constexpr uint32_t kOutOfRange = 0xC0000000u;   // past any head's K/V (< 2^31 bytes)

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).
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

// LDS swizzles.  K: 16-byte chunk c of key row r is stored at chunk
// c ^ kswz(r), so the A-operand reads (rows i, chunks 4 ks + g) hit distinct
// banks.  V: 8-byte quad u of row r is stored at quad u ^ vswz(r) (a
// multiple of 4, so 16-byte chunks stay whole), for the transposing reads
// of rows 4g + i/4, quads 4 db + i%4.
template <int D> __device__ __forceinline__ int kswz(int r) {
    if constexpr (D >= 128) return r & 15;
    else if constexpr (D == 64)
        return ((r >> 2) & 1) | ((__builtin_popcount(r & 15) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
    else return r & 3;
}
template <int D> __device__ __forceinline__ int vswz(int r) {
    if constexpr (D >= 128) return 4 * (r & 7);
    else if constexpr (D == 64) return 4 * ((r & 3) ^ ((r >> 2) & 1));
    else return 0;
}

template <int VLK, int VLV>
__device__ __forceinline__ void load_block(u32x4 (&kr)[VLK], u32x4 (&vr)[VLV],
                                           __amdgpu_buffer_rsrc_t krs,
                                           __amdgpu_buffer_rsrc_t vrs, bool ok, uint32_t kbase,
                                           uint32_t vbase, uint32_t lane16) {
    // `kbase`, `vbase` are the block's first bytes in K and V; piece t of a
    // block is its bytes 1024 t + 16 lane .. +15 (whole consecutive rows).
    // Blocks past the wave's share read nothing (offsets outside the buffer
    // return zeros without a memory access).
#pragma unroll
    for (int t = 0; t < VLK; ++t)
        kr[t] = buffer_load16_nt(krs, ok ? kbase + 1024u * t + lane16 : kOutOfRange);
#pragma unroll
    for (int t = 0; t < VLV; ++t)
        vr[t] = buffer_load16_nt(vrs, ok ? vbase + 1024u * t + lane16 : kOutOfRange);
}

// One register set for the block in flight where a block is too large for
// two (d = dv = 256), and then one workgroup per CU.
template <int D, int DV> constexpr bool single_set() { return D + DV > 256; }

template <typename T, int D, int DV>
__global__ __launch_bounds__(kThreads, (single_set<D, DV>() ? 1 : 2)) void decode_segment_mfma_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    float *__restrict__ ws_o, float *__restrict__ ws_lse, int N, int Nk, int causal, float c,
    int num_splits, int seg_len, int G, int heads_kv, int tiles) {
    typedef typename Mma<T>::vec vec8;
    constexpr int KS = D / 32;              // contraction steps of S^T over d
    constexpr int DB = DV / 16;             // 16-column blocks of O^T
    constexpr int ROWB = 2 * D;             // bytes per key row
    constexpr int ROWBV = 2 * DV;           // bytes per value row
    constexpr int CPR = ROWB / 16;          // 16-byte chunks per key row
    constexpr int CPRV = ROWBV / 16;        // ... per value row
    constexpr int VL = kBlk * CPR / 64;     // 16-byte loads of K per lane per block
    constexpr int VLV = kBlk * CPRV / 64;   // ... of V
    constexpr int WBYTES = kBlk * ROWB;     // one K block
    constexpr int WBYTESV = kBlk * ROWBV;   // one V block; later the wave's O^T partials
    static_assert(kRows == 16 && KS >= 1 && VL >= 1 && VLV >= 1 && kRows * DV * 4 == WBYTESV,
                  "shape");

    __shared__ __attribute__((aligned(16))) unsigned char kbuf[kWaves][WBYTES];
    __shared__ __attribute__((aligned(16))) unsigned char vbuf[kWaves][WBYTESV];
    __shared__ float sm_m[kWaves][kRows];
    __shared__ float sm_l[kWaves][kRows];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;
    const int g = lane / 16;
    const int li = lane % 16;
    const int units = num_splits * heads_kv * tiles;

    // Unit u (one segment of one key/value head for one 16-row tile) ->
    // (split, key/value head, first row), and this wave's share of it.
    auto unit_of = [&](int u, int &split, int &kvh, int &row0, int &seg_begin, int &seg_end,
                       int &mine) {
        split = u % num_splits;
        const int rest = u / num_splits;
        row0 = (rest % tiles) * kRows;
        kvh = rest / tiles;
        seg_begin = split * seg_len;
        seg_end = min(Nk, seg_begin + seg_len);
        const int nblk = seg_end > seg_begin ? (seg_end - seg_begin + kBlk - 1) / kBlk : 0;
        mine = nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0;   // blocks wave, wave+4, ...
    };
    // This lane's query row of a unit: query x % N of query head kvh * G + x / N.
    auto load_q = [&](int kvh, int row0, vec8 (&qop)[KS], int &limit) {
        const int x = row0 + li;
        const bool row_ok = x < G * N;
        const int qrow = row_ok ? x % N : 0;
        const int64_t qhead = (int64_t)kvh * G + (row_ok ? x / N : 0);
        limit = !row_ok ? -1 : (causal ? Nk - N + qrow : Nk - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (row_ok)
                raw = *reinterpret_cast<const u32x4 *>(q + (qhead * N + qrow) * D + (ks * 4 + g) * 8);
            qop[ks] = __builtin_bit_cast(vec8, raw);
        }
    };
    // (The head index is uniform; readfirstlane says so to the compiler, which
    // otherwise may hold the resource in vector registers and wrap every load
    // in a loop over its distinct values.)
    auto k_rsrc = [&](int kvh) {
        const int h = __builtin_amdgcn_readfirstlane(kvh);
        return make_rsrc(k + (int64_t)h * Nk * D, (uint32_t)Nk * D * (uint32_t)sizeof(T));
    };
    auto v_rsrc = [&](int kvh) {
        const int h = __builtin_amdgcn_readfirstlane(kvh);
        return make_rsrc(v + (int64_t)h * Nk * DV, (uint32_t)Nk * DV * (uint32_t)sizeof(T));
    };

    // Per-lane byte offsets: LDS stores of K and V (16-byte piece t * 64 +
    // lane of the block, row-major), and the LDS reads of the K rows li,
    // 16 + li (the swizzle is the same for both) and of V^T.  The swizzles
    // repeat every 16 rows (K) and 8 rows (V), and touch only the low 16
    // chunks (K) and 32 quads (V) of a row, so only one period of each is
    // held in registers and the rest is an immediate offset from it.
    constexpr int RPT = 64 / CPR, RPTV = 64 / CPRV;            // rows per piece index
    constexpr int PK = RPT >= 16 ? 1 : 16 / RPT, PV = RPTV >= 8 ? 1 : 8 / RPTV;
    constexpr int PKS = KS < 4 ? KS : 4, PDB = DB < 8 ? DB : 8;
    static_assert(VL % PK == 0 && VLV % PV == 0, "swizzle periods");
    uint32_t kwp[PK], vwp[PV], krdp[PKS], vrdp[PDB];
#pragma unroll
    for (int t = 0; t < PK; ++t) {
        const int slot = t * 64 + lane, row = slot / CPR, ch = slot % CPR;
        kwp[t] = row * ROWB + ((ch ^ kswz<D>(row)) * 16);
    }
#pragma unroll
    for (int t = 0; t < PV; ++t) {
        const int slot = t * 64 + lane, row = slot / CPRV, ch = slot % CPRV;
        vwp[t] = row * ROWBV + (((2 * ch) ^ vswz<DV>(row)) * 8);
    }
#pragma unroll
    for (int ks = 0; ks < PKS; ++ks) krdp[ks] = li * ROWB + (((ks * 4 + g) ^ kswz<D>(li)) * 16);
#pragma unroll
    for (int db = 0; db < PDB; ++db) {
        const int r0 = 4 * g + li / 4;
        vrdp[db] = r0 * ROWBV + (((4 * db + li % 4) ^ vswz<DV>(r0)) * 8);
    }
    auto kw = [&](int t) { return kwp[t % PK] + (t / PK) * (PK * RPT) * ROWB; };
    auto vw = [&](int t) { return vwp[t % PV] + (t / PV) * (PV * RPTV) * ROWBV; };
    auto krd = [&](int ks) { return krdp[ks % 4 % PKS] + (ks / 4) * 256; };
    auto vrd = [&](int db) { return vrdp[db % 8 % PDB] + (db / 8) * 256; };
    const uint32_t lane16 = 16u * lane;
    unsigned char *kwb = kbuf[wave];
    unsigned char *wbuf = vbuf[wave];

    // The current unit.  The grid has at most `units` workgroups, so every
    // workgroup has a first unit.
    int u = blockIdx.x;
    int split, kvh, row0, seg_begin, seg_end, mine, limit;
    unit_of(u, split, kvh, row0, seg_begin, seg_end, mine);
    vec8 qop[KS];
    load_q(kvh, row0, qop, limit);
    auto krs = k_rsrc(kvh), vrs = v_rsrc(kvh);

    float m, l;
    f32x4 oacc[DB];

    // First byte of the wave's i-th block in K (row width W = D) or V (DV).
    auto block_base = [&](int sb, int i, int W) -> uint32_t {
        return ((uint32_t)(sb + (wave + kWaves * i) * kBlk) * W) * 2u;
    };

    // One 32-key block of the current unit: its K and V rows to the wave's
    // LDS buffers, then scores, mask, online softmax, O^T += V^T P^T.
    auto stage = [&](const u32x4 (&kr)[VL], const u32x4 (&vr)[VLV]) {
#pragma unroll
        for (int t = 0; t < VL; ++t) *reinterpret_cast<u32x4 *>(kwb + kw(t)) = kr[t];
#pragma unroll
        for (int t = 0; t < VLV; ++t) *reinterpret_cast<u32x4 *>(wbuf + vw(t)) = vr[t];
    };
    auto compute = [&](int i) {
        f32x4 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(kwb + kb * 16 * ROWB + krd(ks));
                s[kb] = Mma<T>::run(__builtin_bit_cast(vec8, a), qop[ks], s[kb]);
            }
        }
        const int key0 = seg_begin + (wave + kWaves * i) * kBlk + 4 * g;
        float bmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = key0 + 16 * kb + r;
                const bool vis = key < seg_end && key <= limit;
                s[kb][r] = vis ? s[kb][r] * c : -INFINITY;
                bmax = fmaxf(bmax, s[kb][r]);
            }
        bmax = rows4_max(bmax);
        const float m_new = fmaxf(m, bmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_use);   // 0 while nothing was visible
        float psum = 0.f;
        vec8 pb;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = fast_exp2(s[kb][r] - m_use);   // masked: exp2(-inf) = 0
                psum += p;
                pb[4 * kb + r] = static_cast<T>(p);
            }
        l = l * alpha + psum;
        m = m_new;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            oacc[db] *= alpha;
            const unsigned char *p = wbuf + vrd(db);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 16 * ROWBV));
            const vec8 a = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[db] = Mma<T>::run(a, pb, oacc[db]);
        }
    };
    auto step = [&](const u32x4 (&kr)[VL], const u32x4 (&vr)[VLV], int i) {
        stage(kr, vr);
        compute(i);
    };

    // Persistent loop over units.  Within a unit the loop is double-buffered
    // (block i + 1's loads are in flight while block i is computed); the last
    // block's partner load fetches the next unit's first block and its Q is
    // loaded before the current unit's epilogue, so consecutive units stream
    // without a gap.
    constexpr bool kSingle = single_set<D, DV>();
    u32x4 kA[VL], vA[VLV], kB[kSingle ? 1 : VL], vB[kSingle ? 1 : VLV];
    auto load = [&](u32x4 (&kr)[VL], u32x4 (&vr)[VLV], __amdgpu_buffer_rsrc_t ks,
                    __amdgpu_buffer_rsrc_t vs, bool ok, int sb, int i) {
        load_block<VL, VLV>(kr, vr, ks, vs, ok, block_base(sb, i, D), block_base(sb, i, DV), lane16);
    };
    load(kA, vA, krs, vrs, 0 < mine, seg_begin, 0);
    for (;;) {
        const int un = u + (int)gridDim.x;
        const bool has_next = un < units;
        int nsplit = 0, nkvh = kvh, nrow0 = 0, nbegin = 0, nend = 0, nmine = 0;
        if (has_next) unit_of(un, nsplit, nkvh, nrow0, nbegin, nend, nmine);
        const auto nkrs = k_rsrc(nkvh), nvrs = v_rsrc(nkvh);
        const bool nfirst = has_next && nmine > 0;   // this wave has a first block of the next unit

        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (kSingle) {
            for (int i = 0; i < mine; ++i) {
                stage(kA, vA);
                if (i + 1 < mine)
                    load(kA, vA, krs, vrs, true, seg_begin, i + 1);
                else
                    load(kA, vA, nkrs, nvrs, nfirst, nbegin, 0);
                compute(i);
            }
        } else {
            for (int i = 0; i < mine; i += 2) {
                load(kB, vB, krs, vrs, i + 1 < mine, seg_begin, i + 1);
                step(kA, vA, i);
                if (i + 2 < mine)
                    load(kA, vA, krs, vrs, true, seg_begin, i + 2);
                else
                    load(kA, vA, nkrs, nvrs, nfirst, nbegin, 0);
                if (i + 1 < mine) step(kB, vB, i + 1);
            }
        }
        if (mine == 0) load(kA, vA, nkrs, nvrs, nfirst, nbegin, 0);
        vec8 qnext[KS];
        int nlimit = -1;
        if (has_next) load_q(nkvh, nrow0, qnext, nlimit);

        // ---- merge the 4 wave states of each row through LDS ----------------
        const float lt = rows4_sum(l);
        float *ow = reinterpret_cast<float *>(wbuf);   // [16 rows][DV], this wave's O^T
#pragma unroll
        for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4 *>(ow + li * DV + 16 * db + 4 * g) = oacc[db];
        if (g == 0) {
            sm_m[wave][li] = m;
            sm_l[wave][li] = lt;
        }
        __syncthreads();
        for (int idx = tid; idx < kRows * DV; idx += kThreads) {
            const int r = idx / DV, col = idx % DV;
            const int xr = row0 + r;
            if (xr >= G * N) continue;
            float mm = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, sm_m[w][r]);
            float ll = 0.f, oo = 0.f;
            if (mm != -INFINITY) {
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    const float f = fast_exp2(sm_m[w][r] - mm);   // exp2(-inf) = 0
                    ll = fmaf(sm_l[w][r], f, ll);
                    oo = fmaf(reinterpret_cast<const float *>(vbuf[w])[r * DV + col], f, oo);
                }
            }
            // Workspace layout: o_s [B*Hq, S, N, DV], lse_s [B*Hq, S, N].
            const int64_t head = (int64_t)kvh * G + xr / N;
            const int64_t part = (head * num_splits + split) * N + xr % N;
            ws_o[part * DV + col] = ll > 0.f ? oo / ll : 0.f;
            if (col == 0) ws_lse[part] = ll > 0.f ? (mm + fast_log2(ll)) * kLn2 : -INFINITY;
        }
        __syncthreads();   // the partials in LDS are read before the next unit overwrites them
        if (!has_next) break;
        u = un;
        split = nsplit;
        kvh = nkvh;
        row0 = nrow0;
        seg_begin = nbegin;
        seg_end = nend;
        mine = nmine;
        limit = nlimit;
        krs = nkrs;
        vrs = nvrs;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[ks] = qnext[ks];
    }
}

// Resident workgroups of one instantiation on the current device (cached).
template <typename T, int D, int DV>
int resident_workgroups() {
    static int cache[64];
    return resident_workgroups_of(reinterpret_cast<const void *>(&decode_segment_mfma_kernel<T, D, DV>),
                                  kThreads, cache);
}

template <typename T, int D, int DV>
hipError_t launch_typed(const DecodeArgs &d) {
    const FwdArgs &a = d.a;
    const int G = (int)(a.H / d.Hkv);
    const int64_t tiles = ((int64_t)G * a.N + kRows - 1) / kRows;
    const int64_t units = (int64_t)d.num_splits * a.B * d.Hkv * tiles;
    if (units > 0x7fffffff) return hipErrorInvalidValue;
    const int resident = resident_workgroups<T, D, DV>();
    if (resident <= 0) return hipErrorInvalidDevice;
    const int64_t grid = units < resident ? units : resident;
    hipLaunchKernelGGL((decode_segment_mfma_kernel<T, D, DV>), dim3((unsigned)grid), dim3(kThreads),
                       0, a.stream, static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), d.ws_o, d.ws_lse, (int)a.N, (int)a.Nk,
                       a.causal, a.scale * kLog2e, d.num_splits, (int)d.seg_len, G,
                       (int)(a.B * d.Hkv), (int)tiles);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dv(const DecodeArgs &d) {
    if constexpr (D == 256) {
        return d.a.dv == 256 ? launch_typed<T, 256, 256>(d) : hipErrorInvalidValue;
    } else {
        switch (d.a.dv) {
            case 32: return launch_typed<T, D, 32>(d);
            case 64: return launch_typed<T, D, 64>(d);
            case 128: return launch_typed<T, D, 128>(d);
            default: return hipErrorInvalidValue;
        }
    }
}

template <typename T>
hipError_t launch_dim(const DecodeArgs &d) {
    switch (d.a.d) {
        case 32: return launch_dv<T, 32>(d);
        case 64: return launch_dv<T, 64>(d);
        case 128: return launch_dv<T, 128>(d);
        case 256: return launch_dv<T, 256>(d);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_segment_mfma(const DecodeArgs &d) {
    switch (d.a.dtype) {
        case kF16: return launch_dim<f16_t>(d);
        case kBF16: return launch_dim<bf16_t>(d);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
