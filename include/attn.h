/*
 * attn.h - C ABI of the fused tiled self-attention library for AMD Instinct
 * MI355X (CDNA4, gfx950): libattn.so.
 *
 * The operation. Article "Selbstaufmerksamkeit, CUDA-Kernel und FlashAttention"
 * (German edition of the self-attention / Triton / FlashAttention article,
 * itimpress.au, 2026-11-15):
 *   - §1, "Scores" and "Attention" formulas: for every (batch b, head h)
 *       O = softmax(scale * Q K^T) V,  softmax taken row by row (each row of
 *       probabilities sums to 1); the formula's scale is 1/sqrt(d_k).
 *   - §1, last paragraph: heads are independent copies of this computation.
 *   - §3, tiling bullet: Q, K, V are processed in on-chip tiles and only the
 *       final output goes back to device memory; the N x N score matrix is
 *       never stored.
 *   - §3, online-softmax bullet: a running row maximum and normaliser rescale
 *       the partial outputs tile by tile.
 *   - §3, recompute bullet: the forward pass keeps only small per-row
 *       normalisation statistics; the backward pass rebuilds the attention
 *       tiles from them.
 *
 * Conventions shared by every entry point.
 *   Layout.   Q, K, V, O, dO, dQ, dK, dV are [B, H, N, d_k] contiguous,
 *             row-major (one head is an N x d_k block, rows d_k elements
 *             apart). lse is [B, H, N] contiguous float32.
 *   Statistic. lse[b,h,i] = log(sum_j exp(scale * <q_i, k_j>)), natural log:
 *             the one per-row statistic the forward keeps for the backward.
 *   Memory.   Every pointer is a device pointer owned by the caller and must
 *             be 16-byte aligned. The library allocates no device memory and
 *             keeps no pointer after a call returns.
 *   Streams.  `stream` is a hipStream_t (NULL = the default stream). Work is
 *             enqueued asynchronously; outputs are valid once the caller has
 *             synchronised the stream, and inputs must stay unchanged until
 *             then. Faults inside a kernel surface at that synchronisation,
 *             not in the return code.
 *   Errors.   Arguments are validated before anything is launched; on any
 *             error nothing is launched and nothing is written. Return codes
 *             are attn_status_t values.
 *   Threads.  The library holds no state: calls from several host threads
 *             are safe (ordering between them is the streams' business).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, B/H/N < 1, non-finite scale, aliasing,
                                 causal not 0 or 1 */
  ATTN_ERR_UNSUPPORTED = -2,  /* d_k not in {32, 64, 96, 128}, dtype unknown, or sizes beyond the int32
                                 index range */
  ATTN_ERR_WORKSPACE = -3,    /* workspace missing or smaller than attn_bwd_workspace_bytes() */
  ATTN_ERR_HIP = -4           /* the HIP runtime rejected a launch */
} attn_status_t;

/*
 * Forward, bfloat16 storage with float32 accumulation (the §3 fused method).
 *   q, k, v  in : bf16 [B,H,N,d_k]
 *   o        out: bf16 [B,H,N,d_k], O = softmax(scale Q K^T) V, rounded to
 *                 nearest-even
 *   lse      out: float32 [B,H,N] natural-log row logsumexp of scale Q K^T
 *   d_k      32, 64, 96 or 128 (the article's ViT heads have 64); scale any
 *            finite float (1/sqrt(d_k) in the formula).
 * o and lse must not overlap each other or any input.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d_k, float scale, void* stream);

/*
 * Forward, float32 storage and float32 arithmetic throughout; same contract
 * as attn_fwd otherwise.
 */
int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                 int B, int H, int N, int d_k, float scale, void* stream);

/*
 * Bytes of device workspace attn_bwd needs for this shape: lse * log2(e) and
 * -delta_i = -<dO_i, O_i>, float32 [B,H,N] each (each rounded up to 256 bytes).
 * Returns 0 for arguments attn_bwd would reject.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int N, int d_k);

/*
 * Backward, bfloat16 storage with float32 accumulation (the §3 recompute
 * bullet): rebuilds each probability tile P = exp(scale Q K^T - lse) from the
 * saved lse, and returns the gradients of a scalar loss L given dO = dL/dO:
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
 *   dQ = scale dS K,  dK = scale dS^T Q.
 *   q, k, v, o, dO in : bf16 [B,H,N,d_k]  (o as returned by attn_fwd)
 *   lse            in : float32 [B,H,N]    (as returned by attn_fwd)
 *   dq, dk, dv     out: bf16 [B,H,N,d_k]
 *   workspace          device scratch of at least attn_bwd_workspace_bytes()
 *                      bytes, owned by the caller; its contents on entry are
 *                      ignored and on return are unspecified.
 * dq, dk, dv and the workspace must be distinct and overlap no input.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dO, void* dq, void* dk, void* dv,
             int B, int H, int N, int d_k, float scale,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward, float32 storage and float32 arithmetic throughout (vector ALU):
 * the gradients of attn_fwd_f32's output, same formulas, stages and
 * workspace contract as attn_bwd (attn_bwd_workspace_bytes gives the size),
 * with float32 [B,H,N,d_k] tensors in place of bf16 ones.
 */
int attn_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* lse,
                 const float* dO, float* dq, float* dk, float* dv,
                 int B, int H, int N, int d_k, float scale,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Extended entry points: element type, memory layout and masks.
 *
 * The article defines unmasked attention (§1 "Attention" formula). §3 opens
 * with long text sequences as the case where the N x N score matrix becomes
 * the limit; for text, two masks are standard, and these entry points take
 * them (the article prints neither, so the definition below is a reading):
 *   key padding  kv_len: device pointer to B int32 (4-byte aligned), or NULL
 *                for "all N keys". Keys j >= kv_len[b] are hidden from every
 *                query of batch entry b. Values outside [0, N] are clamped to
 *                it on the device (no error can be reported from there).
 *   causal       0 or 1. With 1, query i sees keys j <= i only (positions in
 *                the same sequence, counted from 0).
 * A hidden pair has score -inf, i.e. probability 0; each row's softmax runs
 * over its visible keys. A row with no visible key (kv_len[b] = 0) gets
 * O = 0 and lse = -inf, and passes no gradient: its dQ row is 0, and keys no
 * query sees get dK = dV = 0.
 *
 * dtype is an attn_dtype_t, the storage type of Q, K, V, O, dO, dQ, dK, dV
 * (lse and the workspace stay float32): ATTN_DTYPE_BF16 (bfloat16) or
 * ATTN_DTYPE_F16 (IEEE binary16). Both use the matrix cores in that type with
 * float32 accumulation; probabilities and dS are rounded to it (nearest even)
 * before their products, and outputs are rounded to it.
 * attn_fwd_ex(ATTN_DTYPE_BF16, ATTN_LAYOUT_BHND, ..., 0, NULL, stream) is
 * attn_fwd. Any other dtype returns ATTN_ERR_UNSUPPORTED.
 */
typedef enum { ATTN_DTYPE_BF16 = 0, ATTN_DTYPE_F16 = 1 } attn_dtype_t;

/*
 * layout is an attn_layout_t: where the rows of head (b, h) sit. In every
 * layout the d_k elements of a row are contiguous and lse stays [B, H, N].
 *   ATTN_LAYOUT_BHND        every tensor [B, H, N, d_k] contiguous (as for
 *                           attn_fwd / attn_bwd).
 *   ATTN_LAYOUT_BNHD        every tensor [B, N, H, d_k] contiguous: the
 *                           token-major layout a row-wise projection X W
 *                           produces, read and written with no transpose.
 *   ATTN_LAYOUT_QKV_PACKED  q, k, v point into one [B, N, 3, H, d_k] buffer
 *                           (the output of one fused Q/K/V projection):
 *                           k = q + H d_k and v = q + 2 H d_k elements;
 *                           dq, dk, dv likewise into one gradient buffer of
 *                           that shape; o and dO are [B, N, H, d_k].
 *                           Otherwise ATTN_ERR_INVALID_ARG.
 * An unknown layout returns ATTN_ERR_UNSUPPORTED.
 */
typedef enum { ATTN_LAYOUT_BHND = 0, ATTN_LAYOUT_BNHD = 1, ATTN_LAYOUT_QKV_PACKED = 2 } attn_layout_t;

int attn_fwd_ex(int dtype, int layout, const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int N, int d_k, float scale, int causal, const int* kv_len, void* stream);

/*
 * Backward with masks: the gradients of attn_fwd_ex's output for the same
 * dtype, layout, causal and kv_len (which must be the values the forward
 * used); dq, dk, dv come back in that layout. The workspace contract is
 * attn_bwd's; kv_len must not overlap an output.
 */
int attn_bwd_ex(int dtype, int layout, const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, void* dq, void* dk, void* dv,
                int B, int H, int N, int d_k, float scale, int causal, const int* kv_len,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * One stage of attn_bwd_ex, same arguments plus `stage`; stages 0, 1, 2 in
 * order on `stream` compute exactly what attn_bwd_ex computes, bit for bit
 * (attn_bwd_ex itself runs stages 0 and 3). For callers that schedule or time
 * the stages separately:
 *   stage 0  prep:  workspace <- lse * log2(e) and -delta_i = -<dO_i, O_i>
 *                   (float32); reads o, dO, lse.
 *   stage 1  dK/dV: rebuilds P from q, k, lse and writes dk, dv; needs the
 *                   workspace of stage 0.
 *   stage 2  dQ:    rebuilds P from q, k, lse and writes dq; needs the
 *                   workspace of stage 0 (stages 1 and 2 are independent).
 *   stage 3  stages 1 and 2 as attn_bwd_ex runs them: one launch of both
 *            kernels' work where attn_bwd_fused() says so, otherwise stage 1
 *            then stage 2.
 * All stages are deterministic: no atomics, bitwise-repeatable results.
 * Every check of attn_bwd_ex applies to every stage (all pointers are
 * required). Returns ATTN_ERR_INVALID_ARG for a stage outside 0..3.
 */
int attn_bwd_stage(int stage, int dtype, int layout, const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d_k, float scale, int causal, const int* kv_len,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_ex without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). The workspace is a 16 MiB array inside the library
 * (one per GPU, reserved when the library's code is loaded on that GPU and
 * held until the process ends); the call itself allocates nothing. Same
 * arguments, checks, kernels and results (bit for bit) as attn_bwd_ex.
 * Limit: attn_bwd_workspace_bytes(B, H, N, d_k) <= 16 MiB (8 bytes per row
 * of B H N, so about 2 million rows), else ATTN_ERR_WORKSPACE. Every call on
 * one GPU shares that GPU's array: calls that may overlap in time on one GPU
 * (concurrent streams, several host threads) race and must be serialised by
 * the caller. Returns ATTN_ERR_HIP if the array's device address cannot be
 * obtained.
 */
int attn_bwd_ex_noalloc(int dtype, int layout, const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dO, void* dq, void* dk, void* dv,
                        int B, int H, int N, int d_k, float scale, int causal, const int* kv_len, void* stream);

/*
 * 1 when attn_bwd / attn_bwd_ex run the dK/dV and dQ work of this shape as
 * one launch (stage 3), 0 when they launch it as stages 1 and 2 (or the shape
 * is rejected). Depends on the shape only: d_k <= 64 and a small dK/dV grid
 * (a multiple of 8 and at most 1024 workgroups of 128 keys), where the tail
 * of a separate dK/dV launch would leave CUs idle. Results are the same
 * either way, bit for bit.
 */
int attn_bwd_fused(int B, int H, int N, int d_k);

/*
 * Query/key/value projection (article §1, first bullet: Q = X W_Q,
 * K = X W_K, V = X W_V, with D x d_k weight matrices, one set per head):
 *   qkv[b, n, t, h, :] = sum_c x[b, n, c] * w[c, t, h, :],  t = 0 (Q), 1 (K), 2 (V).
 *   x    [B, N, D]        token matrix, row-major;
 *   w    [D, 3, H, d_k]   the W_Q, W_K, W_V of every head side by side
 *                         (row c holds the weights of input feature c);
 *   qkv  [B, N, 3, H, d_k] output: the packed layout that attn_fwd_ex /
 *                         attn_bwd_ex read with ATTN_LAYOUT_QKV_PACKED
 *                         (q = qkv, k = qkv + H d_k, v = qkv + 2 H d_k).
 * Storage type `dtype` (ATTN_DTYPE_BF16 or ATTN_DTYPE_F16) for all three;
 * products accumulate in float32 and are rounded once (to nearest even).
 * No bias (the formula has none). Shapes: B, N, D, H, d_k >= 1; D and H d_k
 * multiples of 8 (16-byte rows); B N below 2^30; otherwise
 * ATTN_ERR_UNSUPPORTED (ATTN_ERR_INVALID_ARG for non-positive sizes). qkv
 * must not overlap x or w. The library allocates nothing.
 */
int attn_qkv_proj(int dtype, const void* x, const void* w, void* qkv, int B, int N, int D, int H, int d_k,
                  void* stream);

/*
 * Backward of attn_qkv_proj for a loss whose gradient with respect to qkv is
 * dqkv [B, N, 3, H, d_k] (the packed gradient attn_bwd_ex writes for
 * ATTN_LAYOUT_QKV_PACKED):
 *   dx[b, n, c]     = sum_{t,h,j} dqkv[b, n, t, h, j] * w[c, t, h, j]   (dqkv W^T),
 *   dw[c, t, h, j]  = sum_{b,n}   x[b, n, c] * dqkv[b, n, t, h, j]     (X^T dqkv,
 *                     summed over every token of the batch).
 * Same storage type, shapes and rules as attn_qkv_proj; dx and dw are written
 * in full (not accumulated into) and must overlap neither each other nor an
 * input. `workspace` (device, 256-byte aligned, caller-owned, contents need
 * not be initialised) must hold attn_qkv_proj_bwd_workspace_bytes(B, N, D, H,
 * d_k) bytes, else ATTN_ERR_WORKSPACE; it may be NULL when that size is 0.
 * It holds float32 partial sums of products whose contraction is split over
 * several workgroups; a second kernel adds them in a fixed order, so results
 * are deterministic (bitwise repeatable). It must not overlap any other
 * argument.
 */
int attn_qkv_proj_bwd(int dtype, const void* x, const void* w, const void* dqkv, void* dx, void* dw,
                      int B, int N, int D, int H, int d_k, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes attn_qkv_proj_bwd needs for this shape (0 for shapes it rejects or that need none). */
size_t attn_qkv_proj_bwd_workspace_bytes(int B, int N, int D, int H, int d_k);

/* Static, human-readable text for a status code (never NULL). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
