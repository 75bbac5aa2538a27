/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library, libfa.so.
 *
 * What is computed.  Exact attention as defined by the everydayai.blog
 * flash-attention article (opening standard_attention snippet; "The Math Behind
 * Flash Attention", formula 1) and by the FlashAttention abstract on Tri Dao's
 * scite.ai author page (IO-aware *exact* attention, tiled so that the N x N
 * score matrix never reaches HBM; a block-sparse extension).  Per batch b and
 * head h, with s_ij = scale * <q_i, k_j>:
 *
 *     visible(i,j) = (!causal || j <= i) && (no mask || mask[i/128][j/128] != 0)
 *     O_i   = sum_j softmax_j(s_ij over visible j) v_j
 *     lse_i = ln sum_{visible j} exp(s_ij)            (natural log, fp32)
 *
 * A row with no visible key gets O_i = 0 and lse_i = -inf.
 *
 * Conventions shared by every entry point.
 *   Layout    q, k, v, o, dO, dq, dk, dv: contiguous row-major [B, H, N, d]
 *             (d innermost); lse and the backward's D: contiguous [B, H, N] fp32.
 *             Any N >= 1 (ragged tails are masked inside the kernels) up to
 *             N * d * 4 <= 2^31 - 1.  d must be 64 or 128.
 *   dtype     FA_BF16 or FA_F32; it applies to q, k, v, o and dO.  bf16 inputs
 *             are computed with bf16 MFMA and fp32 accumulation; fp32 inputs with
 *             fp32 arithmetic throughout.
 *   Memory    Every pointer is a device pointer owned by the caller and must be
 *             16-byte aligned.  Outputs must not overlap inputs.  The library
 *             keeps no state and allocates nothing; the backward takes a
 *             caller-provided workspace sized by fa_bwd_workspace_size().
 *   Streams   `stream` is a hipStream_t passed as void* (NULL = default stream).
 *             Each call validates its arguments on the host, then only enqueues
 *             kernels on `stream` and returns; buffers must stay valid until the
 *             stream reaches that point.  Calls are re-entrant and may run
 *             concurrently on different streams.
 *   Errors    Every int-returning entry point returns FA_OK (0) or a negative
 *             code.  Argument validation happens before any HIP call, so an
 *             invalid call has no effect on the device.  FA_ERR_HIP reports a
 *             launch error; faults during execution surface at the caller's next
 *             synchronisation, as with any HIP kernel.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 5
#define FA_MASK_BLOCK 128 /* rows and keys covered by one block-sparse mask entry */
#define FA_FP8_BLOCK 128  /* rows of one head that share one fp8 scale */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20) /* static workspace of fa_bwd_noalloc, per GPU */

enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null required pointer, B/H/N < 1, non-finite scale, bad
                              enum, misaligned pointer, output overlapping an input,
                              H_kv not a divisor of H, or a size whose grid would not fit */
  FA_ERR_UNSUPPORTED = -2, /* d not in {64, 128}; N * d * 4 > 2^31 - 1 (one head's slice is
                              addressed with 32-bit byte offsets); fp32 with block-sparse;
                              a block-sparse N whose tile list does not fit in LDS
                              (N above about 2.09M); bf16 gradients for
                              fp32 inputs */
  FA_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than fa_bwd_workspace_size() */
  FA_ERR_HIP = -4,         /* a HIP launch reported an error */
  FA_ERR_SCRATCH = -5      /* fa_bwd_noalloc: the call needs more than FA_NOALLOC_SCRATCH_BYTES */
};

enum fa_dtype { FA_F32 = 0, FA_BF16 = 1 };

/*
 * Forward.  o <- attention(q, k, v) as defined above; lse <- the row
 * log-sum-exp (may be NULL when the caller does not need it, e.g. inference).
 * scale is any finite float (typically 1/sqrt(d)); causal is 0 or 1.
 * Extents: q, o hold B*H*N*d elements and so do k and v -- this call reads
 * B*H*N*d elements of each of k and v (one K/V head per query head).  K/V with
 * fewer heads must go to fa_fwd_gqa, which reads B*H_kv*N*d of each; handing
 * such buffers to fa_fwd reads past their end.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, int dtype, void* stream);

/*
 * Grouped-query / multi-query forward (everydayai.blog flash-attention article,
 * "FlashAttention-2", point 3, lists both variants).  q, o: [B, H, N, d] and lse
 * [B, H, N] as for fa_fwd; k, v: [B, H_kv, N, d] with H_kv dividing H.  Query
 * head h attends with key/value head h / (H / H_kv): each run of H / H_kv
 * consecutive query heads shares one K/V head (H_kv = 1: multi-query; H_kv = H:
 * identical to fa_fwd).  Same dtypes, limits and errors as fa_fwd, plus
 * FA_ERR_INVALID_ARG for an H_kv outside [1, H] or not dividing H.
 */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int H_kv, int N, int d, float scale, int causal, int dtype, void* stream);

/*
 * Block-sparse forward (FlashAttention abstract: extension to block-sparse
 * attention).  block_mask is a device uint8 array [nb, nb], nb = ceil(N/128),
 * row-major, shared by every (b, h); key j is visible to query i iff
 * block_mask[(i/128)*nb + j/128] != 0 and (!causal || j <= i).  Masked
 * 128x128 tiles cost neither HBM traffic nor MFMA work.  bf16 only.
 */
int fa_fwd_blocksparse(const void* q, const void* k, const void* v, const unsigned char* block_mask,
                       void* o, float* lse, int B, int H, int N, int d, float scale, int causal,
                       int dtype, void* stream);

/*
 * Bytes of workspace fa_bwd needs: 8 per row of [B, H, N] (the row's lse * log2 e
 * and -D with D = rowsum(dO * O), two fp32 values).  Returns 0 for arguments
 * fa_bwd would reject.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d, int grad_dtype);

/*
 * Backward.  Gradients of L = sum(dO * O) with respect to q, k and v, for the
 * same (scale, causal) as the forward that produced o and lse.  The score tiles
 * are recomputed from lse (everydayai.blog flash-attention article, "Enter Flash
 * Attention", point 2: recomputation in the backward pass); nothing N x N is
 * stored.  dq, dk, dv are written in grad_dtype (FA_F32 or FA_BF16; FA_BF16
 * requires dtype FA_BF16).  The workspace must hold fa_bwd_workspace_size()
 * bytes; its contents on entry do not matter.  Every gradient element is
 * reduced by one thread in a fixed order: results are deterministic.
 * Extents: as fa_fwd, this call reads B*H*N*d elements of each of k and v and
 * writes B*H*N*d of each of dk and dv; grouped-query K/V go to fa_bwd_gqa.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
           void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
           int dtype, int grad_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace fa_bwd_gqa needs: as fa_bwd_workspace_size(B, H, N, d) when
 * H_kv == H; otherwise that figure rounded up to 256 bytes plus 8 * B*H*N*d (fp32
 * dK and dV of every query head before the group sums).  0 for arguments
 * fa_bwd_gqa would reject.
 */
size_t fa_bwd_gqa_workspace_size(int B, int H, int H_kv, int N, int d, int grad_dtype);

/*
 * Grouped-query / multi-query backward: gradients of L = sum(dO * O) for the
 * attention of fa_fwd_gqa (same H_kv, scale and causal; o and lse from that
 * call).  dq: [B, H, N, d]; dk, dv: [B, H_kv, N, d], each the sum over the
 * group's query heads of that head's gradient (the chain rule through the
 * shared K/V head).  The per-head fp32 dK/dV are written to the workspace and
 * summed in head order by a final kernel, so results stay deterministic.
 * Arguments, dtypes and errors as fa_bwd, the workspace sized by
 * fa_bwd_gqa_workspace_size().
 */
int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
               void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d, float scale, int causal,
               int dtype, int grad_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-sparse backward.  Gradients of L = sum(dO * O) for the block-sparse
 * attention of fa_fwd_blocksparse (same block_mask, scale and causal; o and lse
 * from that call).  Masked 128x128 tiles cost neither HBM traffic nor MFMA
 * work: the dK/dV pass visits, per 128-key block, the query tiles of the mask
 * rows that keep its column, the dQ pass the key tiles of each query row's
 * kept columns.  bf16 inputs only; arguments, workspace and errors as fa_bwd.
 * Block-sparse training is part of the FlashAttention abstract's block-sparse
 * extension (scite.ai page of Tri Dao).
 */
int fa_bwd_blocksparse(const void* q, const void* k, const void* v, const unsigned char* block_mask,
                       const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                       int B, int H, int N, int d, float scale, int causal, int dtype, int grad_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-sparse attention with grouped-query / multi-query K/V heads: the mask
 * of fa_fwd_blocksparse and the head sharing of fa_fwd_gqa together (q, o, lse
 * [B, H, ...]; k, v [B, H_kv, N, d]; one block_mask shared by every (b, h)).
 * Arguments, limits and errors as fa_fwd_blocksparse, plus those of H_kv as in
 * fa_fwd_gqa; H_kv == H is identical to fa_fwd_blocksparse.
 */
int fa_fwd_blocksparse_gqa(const void* q, const void* k, const void* v, const unsigned char* block_mask,
                           void* o, float* lse, int B, int H, int H_kv, int N, int d, float scale,
                           int causal, int dtype, void* stream);

/*
 * Backward of fa_fwd_blocksparse_gqa (same block_mask, H_kv, scale and causal;
 * o and lse from that call): dq [B, H, N, d]; dk, dv [B, H_kv, N, d] summed
 * over each group's query heads in head order, as in fa_bwd_gqa.  The
 * workspace is sized by fa_bwd_gqa_workspace_size(); arguments and errors as
 * fa_bwd_blocksparse and fa_bwd_gqa.
 */
int fa_bwd_blocksparse_gqa(const void* q, const void* k, const void* v, const unsigned char* block_mask,
                           const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                           int B, int H, int H_kv, int N, int d, float scale, int causal, int dtype,
                           int grad_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8 quantisation with incoherent processing (everydayai.blog flash-attention
 * article, "FlashAttention-3": FP8 support, and incoherent processing to reduce
 * quantisation error).  x: [B, H, N, d] in dtype (FA_BF16 or FA_F32), finite.
 * codes: uint8 [B, H, N, d], OCP E4M3 (bias 7, largest finite 448, no
 * infinities); scales: fp32 [B, H, ceil(N/128)], one per block of FA_FP8_BLOCK
 * consecutive rows of a head.  Per block, with y the block's rows: the exponent
 * e is the smallest integer with max|y| * 2^-e <= 448 (0 for an all-zero block),
 * codes = round-to-nearest-even of y * 2^-e, scale = 2^e (times fl32(1/sqrt(d))
 * when rotating), so that code * scale approximates the row.
 * signs: NULL, or a device array of d int8 values (negative = -1, else +1): the
 * rows are then rotated first, y = x diag(signs) H_d with the Sylvester Hadamard
 * matrix H_d, by the fast Walsh-Hadamard transform in fp32 (stages of pair
 * distance 1, 2, 4, ..., d/2 in that order; this fixes every rounding).  Rotate
 * Q and K with the same signs and V not at all: (Q M)(K M)^T = Q K^T for the
 * orthogonal M = diag(signs) H_d / sqrt(d), so fa_fwd_fp8 then computes the
 * attention of the unrotated inputs.  Pointers 16-byte aligned (scales 4-byte);
 * outputs must not overlap inputs.
 */
int fa_quantize_fp8(const void* x, const signed char* signs, unsigned char* codes, float* scales,
                    int B, int H, int N, int d, int dtype, void* stream);

/*
 * FP8 forward: o (bf16 [B, H, N, d]) and lse (fp32 [B, H, N], may be NULL) of
 * exact attention of the dequantised inputs code * scale, computed with the
 * e4m3 matrix cores.  q, q_scale as written by fa_quantize_fp8 for [B, H, N, d];
 * k, v, k_scale, v_scale for [B, H_kv, N, d] (H_kv divides H; grouped-query as in
 * fa_fwd_gqa).  Scales must be positive and finite.  Two roundings go beyond
 * the dequantised inputs.  (1) The matrix cores sum each group of 64 fp8
 * products of S = Q K^T with an error of up to about 2^-11 of the group's
 * largest product (then accumulate in fp32).  (2) P = exp(S - m), with m
 * within one binade below the running row maximum, is rounded to e4m3 for the
 * P V product (the row sums use the unrounded P): |dO| <= (2^-4 sum_{P >= 2^-6} P |v| + 2^-10 sum_{P < 2^-6} |v|)
 * / sum P per element.  O is rounded to bf16.
 * Arguments and errors as fa_fwd_gqa.
 */
/*
 * General forward: every variant above in one call, plus an optional second
 * output for training.  block_mask: NULL (dense) or a mask as for
 * fa_fwd_blocksparse; k, v: [B, H_kv, N, d] as for fa_fwd_gqa (H_kv == H: one
 * K/V head per query head).  o_lo: NULL, or (bf16 only) a [B, H, N, d] bf16
 * buffer that receives the low-order part of the output, o_lo = bf16(O - o)
 * where O is the fp32 result before its rounding to o; o + o_lo then carries O
 * to about 16 significant bits (relative error <= 2^-17).  Passing it on to
 * fa_bwd_ex lets the backward form D = rowsum(dO * O) from that O instead of
 * from the bf16 o (D's rounding error then no longer dominates the gradients
 * at long N).  It costs one more write of B*H*N*d bf16.  Errors as
 * fa_fwd_blocksparse_gqa (without a mask: fa_fwd_gqa), plus FA_ERR_INVALID_ARG
 * for an o_lo that is misaligned, overlaps another argument, or is given with
 * dtype FA_F32.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, const unsigned char* block_mask, void* o, void* o_lo,
              float* lse, int B, int H, int H_kv, int N, int d, float scale, int causal, int dtype, void* stream);

/*
 * General backward: the gradients of the forward of fa_fwd_ex with the same
 * block_mask (NULL: dense), H_kv, scale and causal; o, o_lo and lse from that
 * call.  o_lo may be NULL: D is then formed from the bf16 o alone, exactly as
 * fa_bwd does.  dq [B, H, N, d]; dk, dv [B, H_kv, N, d] (grouped heads summed in
 * head order).  The workspace is sized by fa_bwd_gqa_workspace_size(); o_lo is
 * read-only and must not overlap an output.  Arguments and errors otherwise as
 * fa_bwd_blocksparse_gqa (without a mask: fa_bwd_gqa).
 */
int fa_bwd_ex(const void* q, const void* k, const void* v, const unsigned char* block_mask, const void* o,
              const void* o_lo, const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H,
              int H_kv, int N, int d, float scale, int causal, int dtype, int grad_dtype, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * Backward that allocates nothing and takes no workspace: fa_bwd_ex with the
 * workspace replaced by a static device array of FA_NOALLOC_SCRATCH_BYTES
 * (32 MiB) inside the library, one per GPU, held from the first call on that
 * GPU until the process ends.  For callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the call makes no hipMalloc or hipFree and no allocating library
 * call; the caller still passes every input and output.  The calls that fit are
 * those whose fa_bwd_gqa_workspace_size() is at most FA_NOALLOC_SCRATCH_BYTES
 * (without grouped heads: B*H*N <= 4194304 rows); larger ones return
 * FA_ERR_SCRATCH before any GPU work.  The array belongs to the GPU that is
 * current at the call (the stream and the buffers must be on it); its address
 * is looked up on the first call on each GPU.  Every call on one GPU uses the
 * same array and leaves its contents there (nothing in it needs clearing: each
 * call writes every workspace entry it reads before reading it), so calls
 * that overlap on one GPU -- on two streams, or from two threads without
 * ordering -- race on it and must not be made.  Arguments, results and other
 * errors as fa_bwd_ex; results are bitwise those of fa_bwd_ex.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const unsigned char* block_mask, const void* o,
                   const void* o_lo, const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H,
                   int H_kv, int N, int d, float scale, int causal, int dtype, int grad_dtype, void* stream);

int fa_fwd_fp8(const unsigned char* q, const unsigned char* k, const unsigned char* v,
               const float* q_scale, const float* k_scale, const float* v_scale, void* o, float* lse,
               int B, int H, int H_kv, int N, int d, float scale, int causal, void* stream);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char* fa_status_string(int status);

/* FA_ABI_VERSION of the loaded library. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
