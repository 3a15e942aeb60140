/*
 * fa.h — fused forward pass of exact dense softmax attention on AMD MI355X (gfx950).
 *
 * Operation (lihaoran.work, "The intermediate matrix comes first": O = softmax(QK^T/sqrt(d)) V,
 * with N the sequence length and d the head dimension; here the score scale is a parameter):
 *
 *   for every batch b, head h and query row i (0 <= i < N):
 *     s_ij      = scale * sum_c q[b,h,i,c] * k[b,h,j,c]      for j in J_i
 *     J_i       = {0 .. N-1}, or {0 .. i} when causal = 1 (key j kept only when j <= i)
 *     o[b,h,i,:] = sum_{j in J_i} exp(s_ij - lse_i) * v[b,h,j,:]
 *     lse[b,h,i] = ln sum_{j in J_i} exp(s_ij)                (natural log, fp32)
 *
 * The library computes this in one fused, tiled pass. Each query row carries the running
 * maximum m, the running denominator l and the unnormalised numerator u across key/value
 * tiles, and rescales l and u together by e^(m - m') whenever the maximum rises
 * (liminalml.com, "FlashAttention", online update equations; interactiveml.org,
 * "FlashAttention saves the matrix, not the quadratic work", merge of three sufficient
 * statistics). No N x N score or probability matrix is ever written to device memory
 * (sadullah.online, "FlashAttention's trick: fused, tiled computation").
 *
 * Results equal the definition up to floating-point rounding, not bit for bit: the
 * summation order differs from a materialised implementation (lihaoran.work, "Exact
 * attention does not mean bitwise equality").
 *
 * Layout: q, k, v, o are contiguous row-major [B][H][N][d] arrays (d fastest); lse is a
 * contiguous [B][H][N] fp32 array. All pointers are device pointers owned by the caller;
 * q, k, v, o (and the backward's dout, dq, dk, dv) must be 16-byte aligned and lse (and
 * delta) 4-byte aligned, since rows are moved in 16-byte pieces.
 * The library allocates no device memory, keeps no state between calls and may be called
 * from several host threads at once.
 *
 * Execution: work is enqueued on `stream` (NULL = the default stream) and the call returns
 * without waiting for it. Outputs must not overlap inputs.
 *
 * Errors: every argument check runs on the host before any HIP call, and a rejected call
 * writes nothing. Bad device pointers are not detected (C convention). A failed kernel
 * launch returns FA_ERR_HIP; asynchronous faults surface on the caller's next
 * synchronisation.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null q/k/v/o, B/H/N/d < 1, non-finite or non-positive-size problem,
                              causal not 0/1, element count above 2^62, misaligned or
                              overlapping buffers */
  FA_ERR_UNSUPPORTED = -2, /* d > 256 (the largest head width compiled), or a grid too large */
  FA_ERR_HIP = -3,         /* the HIP runtime rejected the launch */
  FA_ERR_WORKSPACE = -4,   /* split-KV call: workspace missing or smaller than required */
  FA_ERR_SCRATCH = -5      /* fa_fwd_splitkv_noalloc: the partial states would not fit its
                              fixed buffer of FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

/* Element type selector of the split-KV entry points (the single-pass entry points carry the
 * type in their names instead). */
typedef enum { FA_BF16 = 0, FA_F32 = 1 } fa_dtype;

/* bf16 inputs and output (the hot path).
 *   q, k, v : device, bf16 (IEEE binary32 upper halves), [B][H][N][d], read only
 *   o       : device, bf16 [B][H][N][d], written (round to nearest even from fp32)
 *   lse     : device, fp32 [B][H][N], written; may be NULL to skip it
 *   scale   : multiplies q.k before the softmax; must be finite (callers pass 1/sqrt(d))
 *   causal  : 0 = all keys, 1 = keys j <= i
 * Arithmetic: fp32 accumulation of both products; the probabilities are rounded to bf16
 * before the product with V; statistics and the normalisation are fp32.
 * Supported: 1 <= d <= 256 (d = 64 and d = 128 are the tuned widths; other widths run on the
 * kernel for the next width up of 64, 128 or 256), any N >= 1. */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* fp32 inputs and output; same parameters and semantics as fa_fwd. Both products use
 * fp32 matrix instructions with fp32 accumulation; the probabilities stay fp32. */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* Backward pass, bf16 (recomputes the probabilities from q, k and lse instead of storing
 * them: lihaoran.work, "The intermediate matrix comes first"; the gradients are those of the
 * definition O = softmax(scale q k^T [masked]) v).
 *   q, k, v : the forward's inputs, device bf16 [B][H][N][d], read only
 *   o, lse  : the forward's outputs for the same q, k, v, scale, causal: o bf16 [B][H][N][d],
 *             lse fp32 [B][H][N] (natural-log normaliser, as fa_fwd writes it), read only
 *   dout    : gradient of the loss with respect to o, device bf16 [B][H][N][d], read only
 *   dq, dk, dv : gradients with respect to q, k, v, device bf16 [B][H][N][d], written
 *   delta   : device fp32 workspace of B*H*N floats, written (row sums of dout * o); owned by
 *             the caller, no allocation happens inside
 * Arithmetic: fp32 accumulation; the probabilities and their gradients are rounded to bf16
 * before the matrix products. No output may overlap an input or another output.
 * Supported: d = 64 or 128, any N >= 1; other widths return FA_ERR_UNSUPPORTED. Asynchronous
 * on `stream` like fa_fwd; the same error rules apply. */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, float* delta,
           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* Forward pass with the key range split over several workgroups (split-KV), for grids that
 * the single-pass kernels leave small: few heads, few query tiles, long key ranges.
 *
 * Every query tile is paired with each of S consecutive key ranges ("split columns"); each
 * pair runs as its own workgroup and leaves the partial online-softmax state of its rows in
 * the workspace: the reference maximum m_s, the denominator l_s and the unnormalised numerator
 * u_s. A second kernel merges the S states of every row with the rule for combining two blocks
 * (interactiveml.org, "FlashAttention saves the matrix, not the quadratic work", merge of the
 * three sufficient statistics): m* = max m_s, l = sum e^(m_s - m*) l_s, u = sum e^(m_s - m*) u_s,
 * o = u / l, lse = m* + ln l. The result is the function fa_fwd / fa_fwd_f32 computes (same
 * arguments, same layouts and outputs), up to rounding.
 *   dtype      : FA_BF16 (q, k, v, o bf16, as fa_fwd) or FA_F32 (fp32, as fa_fwd_f32)
 *   num_splits : 0 = the library's choice (one column when the single pass already has 256
 *                workgroups or more; else about 256 workgroups in all, 2048 under the causal
 *                mask, in columns of at least 1024 keys), else 1..64 requested columns; the
 *                call uses at most one column per key tile of the kernel and drops columns
 *                that would hold no key (fa_fwd_splitkv_plan reports the count)
 *   workspace  : device memory owned by the caller, 256-byte aligned, at least the size
 *                fa_fwd_splitkv_plan reports for the same (B, H, N, d, dtype, causal,
 *                num_splits); its contents on entry are ignored and on return unspecified.
 *                It must not overlap q, k, v, o or lse. When the plan has one column
 *                (workspace size 0) the call is the single-pass fa_fwd / fa_fwd_f32 and the
 *                workspace may be NULL.
 * The library allocates nothing. Two kernels are enqueued on `stream` (partial pass, merge);
 * calls that share a workspace must be ordered (same stream or synchronised). Errors as for
 * fa_fwd, plus FA_ERR_WORKSPACE (missing or too small workspace) and FA_ERR_INVALID_ARG for
 * dtype not in {FA_BF16, FA_F32}, num_splits outside 0..64 or a misaligned or overlapping
 * workspace. */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal, int dtype, int num_splits,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Host-only planning of a fa_fwd_splitkv call (no HIP call): writes the number of split
 * columns the call will use and the workspace bytes it needs (0 when one column remains) to
 * the non-NULL output pointers. Returns FA_OK or the status fa_fwd_splitkv would return for
 * these sizes (FA_ERR_INVALID_ARG / FA_ERR_UNSUPPORTED). */
int fa_fwd_splitkv_plan(int B, int H, int N, int d, int dtype, int causal, int num_splits,
                        int* nsplit_out, size_t* workspace_bytes_out);

/* Size of the device buffer fa_fwd_splitkv_noalloc keeps its partial states in (64 MiB per GPU,
 * held from the library's first use on that GPU until the process ends). */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* fa_fwd_splitkv without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * partial states go to a fixed buffer the library owns, one per GPU (the GPU of `stream`, or
 * the current GPU for the NULL stream). The call itself allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine. Arguments, result and errors as for fa_fwd_splitkv;
 * a plan whose workspace (fa_fwd_splitkv_plan) exceeds FA_NOALLOC_SCRATCH_BYTES is rejected
 * with FA_ERR_SCRATCH before any launch.
 * All calls on one GPU share the buffer: calls that overlap on one GPU (different streams, or
 * host threads without ordering) race and must be serialised by the caller. */
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, float scale, int causal, int dtype, int num_splits,
                           hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
