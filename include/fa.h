/*
 * fa.h -- C ABI of the exact tiled attention library (libfa.so) for AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed.  For every (batch b, head h) pair, exact softmax
 * attention of the head's queries over its keys:
 *
 *     S = scale * Q K^T                      (Q: [N, d], K: [Nk, d])
 *     P = softmax(S) row by row              (masked scores are -inf)
 *     O = P V                                (V: [Nk, dv], O: [N, dv])
 *     LSE_i = ln sum_j exp(S_ij)             (over visible keys only)
 *
 * as defined by standard attention in the CS349E Lecture 11 shared module
 * "flash_lab.py" (section 2, standard_attention), which the tiled forward of
 * section 3 (flash_fwd, FlashAttention-2 loop order) and the split-KV decode
 * of section 4 (split_kv_decode) reach exactly up to rounding order.  The
 * N x Nk score matrix never reaches device memory.
 *
 * Causal mask (same page, section 2, _causal_mask; and "02_flash_forward.py"
 * demo 1): query row i sits at sequence position Nk - N + i and sees key j
 * iff j <= Nk - N + i ("bottom-right" alignment; with N < Nk the first
 * Nk - N keys are a cached prefix).  A query row that sees no key at all
 * (causal with N > Nk, rows i < N - Nk) gets O = 0 and LSE = -inf, the
 * identity state (m = -inf, l = 0) of merge_states in section 1.
 *
 * Memory layout (all tensors dense, row-major, no strides):
 *     q   [B, H, N,  d ]   element type `dtype`
 *     k   [B, H, Nk, d ]   element type `dtype`
 *     v   [B, H, Nk, dv]   element type `dtype`
 *     o   [B, H, N,  dv]   element type `dtype` (written, round-to-nearest-even)
 *     lse [B, H, N     ]   float32 (written; natural log)
 * Arithmetic: products of `dtype` operands accumulated in float32; softmax
 * state and LSE in float32.  For bf16/fp16 the probabilities are rounded to
 * `dtype` before the P V product.
 *
 * Ownership and execution.  Every pointer is DEVICE memory owned by the
 * caller; the library allocates nothing, keeps no pointer after returning,
 * and holds no state, so calls are reentrant.  Work is enqueued on `stream`
 * (a hipStream_t passed as void*; NULL means the default stream) and the
 * call returns without synchronising: outputs are valid once the stream has
 * executed the work.  Inputs must not be modified until then.
 *
 * Errors.  All argument checks happen before any HIP call, so an invalid
 * call has no side effect.  A failed kernel launch is reported as
 * FA_ERR_LAUNCH.  NaN or Inf inside the inputs are not trapped; they
 * propagate into the outputs.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. */
typedef enum {
    FA_DTYPE_F32 = 0,   /* IEEE float32 */
    FA_DTYPE_F16 = 1,   /* IEEE float16 */
    FA_DTYPE_BF16 = 2   /* bfloat16 */
} fa_dtype_t;

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,  /* null pointer, size < 1, misalignment, bad scale/dtype, overflow */
    FA_ERR_UNSUPPORTED = 2,  /* valid request outside the supported (dtype, d, dv) set */
    FA_ERR_WORKSPACE = 3,    /* decode workspace missing, misaligned or too small */
    FA_ERR_LAUNCH = 4        /* the HIP runtime rejected a kernel launch */
} fa_status_t;

/*
 * fa_fwd -- exact attention forward (FlashAttention-2 loop order: one block
 * of query rows per workgroup, K/V tiles streamed through LDS, online
 * softmax with the division by the row sum deferred to the end, causal tiles
 * that are fully masked skipped).  flash_lab.py section 3, flash_fwd.
 *
 *   q, k, v  inputs, layout above; 16-byte aligned.
 *   o, lse   outputs, layout above; o 16-byte aligned, lse 4-byte aligned.
 *   B, H     batch and head counts (>= 1).
 *   N, Nk    query rows and keys per head (>= 1).
 *   d, dv    head dims of q/k and of v/o.  Supported: d and dv each in
 *            {32, 64, 128, 256}; dv may differ from d (the pages' convention
 *            has V [Nk, dv]).  bf16/fp16 run on the matrix cores (tuned
 *            kernels for d, dv in {64, 128} with scale > 0, a generic one
 *            otherwise); fp32 runs on the vector ALUs.
 *            Each per-head slice (N*d, Nk*d, Nk*dv, N*dv elements) must be
 *            smaller than 2 GiB, else FA_ERR_UNSUPPORTED.
 *   causal   0: no mask; non-zero: bottom-right causal mask (see above).
 *   scale    multiplies Q K^T before the softmax; any finite value (0 gives
 *            uniform weights over the visible keys).  The usual value 1/sqrt(d)
 *            is the caller's choice.
 *   dtype    element type of q, k, v, o.
 *   stream   hipStream_t (as void*), NULL for the default stream.
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or FA_ERR_LAUNCH.
 */
fa_status_t fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                   int64_t B, int64_t H, int64_t N, int64_t Nk, int64_t d, int64_t dv,
                   int causal, float scale, fa_dtype_t dtype, void *stream);

/*
 * fa_decode_splitkv_workspace_size -- bytes of device workspace that
 * fa_decode_splitkv needs: the per-segment partial outputs o_s
 * [B, H, num_splits, N, dv] followed by the per-segment log-sum-exps
 * lse_s [B, H, num_splits, N], both float32:
 *     B * H * num_splits * N * (dv + 1) * 4.
 * Returns 0 if an argument is < 1 or the size overflows.
 */
size_t fa_decode_splitkv_workspace_size(int64_t B, int64_t H, int64_t N, int64_t dv,
                                        int num_splits);

/*
 * fa_decode_splitkv -- the same result as fa_fwd, computed the flash-decoding
 * way (flash_lab.py section 4, split_kv_decode, with section 1's
 * merge_states): the Nk keys of every head are cut into `num_splits`
 * segments of ceil(ceil(Nk / num_splits) / 64) * 64 keys each (the last ones
 * may be short or empty); one workgroup per (b, h, segment) streams that
 * segment once and writes (o_s, lse_s) -- o_s already divided by the
 * segment's row sum -- into the workspace; a second kernel on the same
 * stream merges the segments of each row:
 *     lse = ln sum_s exp(lse_s),  o = sum_s exp(lse_s - lse) * o_s.
 * An empty segment has lse_s = -inf and weight 0.  Meant for few query rows
 * (decode: N = 1) and long Nk; any N >= 1 gives the fa_fwd result.
 *
 *   q .. stream       as for fa_fwd (causal uses the same bottom-right mask).
 *   num_splits        segments per head, 1 .. 65536 (larger: FA_ERR_UNSUPPORTED;
 *                     negative: FA_ERR_INVALID_ARG); it may exceed the key
 *                     count, surplus segments are then empty.  0 selects
 *                     fa_decode_splitkv_auto_splits(B, H, H, N, Nk, d,
 *                     dv, dtype) segments.  Also FA_ERR_UNSUPPORTED: B*H > 65535.
 *   workspace         device scratch of at least
 *                     fa_decode_splitkv_workspace_size(B, H, N, dv, num_splits)
 *                     bytes, 16-byte aligned, owned by the caller; its
 *                     contents on entry are ignored and on exit undefined.
 *   workspace_bytes   size of `workspace` in bytes.
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE or
 * FA_ERR_LAUNCH.
 */
fa_status_t fa_decode_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                              int64_t B, int64_t H, int64_t N, int64_t Nk, int64_t d,
                              int64_t dv, int causal, float scale, fa_dtype_t dtype,
                              int num_splits, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * fa_decode_splitkv_noalloc -- fa_decode_splitkv without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * The per-segment partials go to a static device array of
 * FA_DECODE_NOALLOC_MAX_WORKSPACE bytes inside the library (one per GPU,
 * held from library load until the process ends); the call allocates
 * nothing.  Same kernels and result as fa_decode_splitkv with a workspace.
 *
 *   all arguments   as for fa_decode_splitkv (num_splits = 0 selects the
 *                   automatic count).
 * The workspace this shape would need,
 * fa_decode_splitkv_workspace_size(B, H, N, dv, num_splits), must not
 * exceed FA_DECODE_NOALLOC_MAX_WORKSPACE, else FA_ERR_WORKSPACE (nothing is
 * launched).  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (on different streams, or from several threads) race
 * and give undefined results; calls serialised on one stream are safe.  The
 * array needs no clearing between calls: every partial the merge reads is
 * written by the same call.  The first call on a device looks up the array's
 * address on that device (the device must be current); failure there is
 * FA_ERR_LAUNCH.
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE or
 * FA_ERR_LAUNCH.
 */
#define FA_DECODE_NOALLOC_MAX_WORKSPACE ((size_t)16 << 20)
fa_status_t fa_decode_splitkv_noalloc(const void *q, const void *k, const void *v, void *o,
                                      float *lse, int64_t B, int64_t H, int64_t N, int64_t Nk,
                                      int64_t d, int64_t dv, int causal, float scale,
                                      fa_dtype_t dtype, int num_splits, void *stream);

/*
 * fa_decode_splitkv_gqa -- fa_decode_splitkv for grouped-query attention: Hq
 * query heads share Hkv key/value heads (Hq a multiple of Hkv), query head h
 * attending with key/value head h / (Hq / Hkv).  The result is that of
 * fa_fwd on K and V with each key/value head repeated Hq / Hkv times.  Each
 * workgroup serves the rows of all query heads of one key/value head, so K
 * and V are read once per group -- the packing flash_lab.py section 4 names
 * for grouped heads in decode.  fa_decode_splitkv is this call with
 * Hkv == Hq.
 *
 *   q, o      [B, Hq, N, d] and [B, Hq, N, dv]; lse [B, Hq, N].
 *   k, v      [B, Hkv, Nk, d] and [B, Hkv, Nk, dv].
 *   Hq, Hkv   query and key/value heads (>= 1, Hq % Hkv == 0, else
 *             FA_ERR_INVALID_ARG; B * Hkv > 65535: FA_ERR_UNSUPPORTED).
 *   workspace at least fa_decode_splitkv_workspace_size(B, Hq, N, dv,
 *             num_splits) bytes (partials are kept per query head).
 *   num_splits  as for fa_decode_splitkv; 0 selects
 *             fa_decode_splitkv_auto_splits(B, Hq, Hkv, N, Nk, d, dv,
 *             dtype).
 *   all else  as for fa_decode_splitkv.
 */
fa_status_t fa_decode_splitkv_gqa(const void *q, const void *k, const void *v, void *o,
                                  float *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                                  int64_t Nk, int64_t d, int64_t dv, int causal, float scale,
                                  fa_dtype_t dtype, int num_splits, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * fa_decode_splitkv_auto_splits -- the split count that num_splits = 0
 * selects in the decode entry points for this shape (flash_lab.py section
 * 4 chooses it with a time model; this library uses a rule measured on
 * MI355X): the smallest power of two S for which the segment kernel has at
 * least 512 workgroups, doubling S only while Nk >= 2 S * 256 (so that a
 * segment keeps at least 256 keys), and S <= 256.  The workgroup count
 * per split is B * Hkv * ceil(rows / r) with rows = (Hq / Hkv) * N and r the
 * query rows per workgroup of the kernel the shape runs on (16 for bf16 and
 * fp16 with d == dv <= 128 and rows >= 2; else the smallest of 1, 2, 4, 8
 * covering rows).  Pure host logic: no HIP call.
 *
 *   B, Hq, Hkv, N, Nk, d, dv, dtype   as for fa_decode_splitkv_gqa.
 * Returns the split count (1 .. 256), or 0 if an argument is out of range
 * (a size < 1, Hq % Hkv != 0, an unknown dtype, B * Hq or
 * (Hq / Hkv) * N above 2^31 - 1).
 */
int fa_decode_splitkv_auto_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t Nk,
                                  int64_t d, int64_t dv, fa_dtype_t dtype);

/*
 * fa_bwd_workspace_size -- bytes of device workspace fa_bwd needs: two
 * float32 per query row, B * H * N * 8.  Returns 0 if an argument is < 1 or
 * the size overflows.
 */
size_t fa_bwd_workspace_size(int64_t B, int64_t H, int64_t N);

/*
 * fa_bwd -- gradients of exact attention (the FlashAttention-2 backward of
 * flash_lab.py section 3, flash_bwd): given the forward's inputs, its outputs
 * o and lse (as fa_fwd writes them) and the output gradient dout, writes
 *     dq = dL/dq, dk = dL/dk, dv = dL/dv   for L = sum(dout * O),
 * i.e. with P = exp(S - LSE) recomputed from q, k and lse (never stored),
 *     D_i = sum_c dout_ic o_ic,  dv = P^T dout,  dP = dout v^T,
 *     dS = P * (dP - D),  dq = scale dS k,  dk = scale dS^T q,
 * the gradients section 2's standard_attention_bwd defines.  Rows that see
 * no key (lse = -inf) contribute nothing; keys no row sees get dk = dv = 0.
 *
 *   q, k, v, causal, scale, dtype, sizes   as for fa_fwd (the same call).
 *   o, lse     fa_fwd's outputs for these inputs (read; same layout).
 *   dout       [B, H, N, dv] element type `dtype`, 16-byte aligned (read).
 *   dq, dk, dv [B, H, N, d], [B, H, Nk, d], [B, H, Nk, dv], element type
 *              `dtype`, 16-byte aligned (written, round-to-nearest-even).
 *   workspace  device scratch of at least fa_bwd_workspace_size(B, H, N)
 *              bytes, 16-byte aligned, owned by the caller (per query row
 *              the row dot D and the LSE in base 2);
 *              contents on entry ignored, on exit undefined.
 * Arithmetic: products accumulated in float32; for bf16/fp16 the
 * probabilities and dS are rounded to `dtype` before the products that use
 * them (matrix cores); fp32 stays in float32 throughout.  Deterministic: every output element is written by
 * one workgroup.  Returns FA_OK, FA_ERR_INVALID_ARG (as fa_fwd, plus null or
 * misaligned dout/dq/dk/dv), FA_ERR_UNSUPPORTED (as fa_fwd), FA_ERR_WORKSPACE
 * or FA_ERR_LAUNCH.
 */
fa_status_t fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dout, void *dq, void *dk, void *dv, int64_t B, int64_t H,
                   int64_t N, int64_t Nk, int64_t d, int64_t dv_dim, int causal, float scale,
                   fa_dtype_t dtype, void *workspace, size_t workspace_bytes, void *stream);

/* fa_status_string -- a static, human-readable name of a status code. */
const char *fa_status_string(fa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
