/*
 * fa.h - C ABI of libfa, exact blockwise scaled-dot-product attention for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  For every (batch b, head h) slice, with Q of shape
 * [Lq, d], K and V of shape [Lk, d]:
 *     S   = scale * Q K^T                       (Lq x Lk scores)
 *     S_ij = -inf where causal and j > i        (mask; rows and keys are
 *                                                aligned at index 0)
 *     lse_i = log sum_j exp(S_ij)               (natural log)
 *     O   = exp(S - lse) V
 * This is the score matrix / softmax / value product of the "standard
 * attention" that the blockwise method reproduces exactly ("How Flash
 * Attention Improves Transformer Memory Efficiency ...", sections "Full
 * Matrix Construction" and "Intermediate Tensor Storage"), computed instead
 * tile by tile with an online softmax: a running max m, a running sum l and
 * an unnormalised accumulator rescaled whenever the max grows, divided by l
 * at the end (same page, section "The Three Running Statistics";
 * "What Is FlashAttention?", section "What FlashAttention does instead").
 * S and P are never written to device memory.
 *
 * The backward (loss <dO, O>) recomputes the probabilities from the saved
 * lse and uses the row statistic D_i = sum_c dO_ic O_ic (annotated-code
 * page, section "Backward Pass Efficiency"; glossary page "Flash
 * Attention", section "How it works", on recomputing intermediates):
 *     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
 *     dQ = scale * dS K,  dK = scale * dS^T Q.
 *
 * Conventions shared by every entry point:
 *   Layout     Q, K, V, O, dO, dQ, dK, dV are dense row-major [B, H, L, d]
 *              (d fastest, then L, then H, then B); lse and the D statistic
 *              are dense [B, H, Lq] float.  Base pointers must be 16-byte
 *              aligned.
 *   Dtypes     FA_BF16 inputs compute on bf16 matrix cores with fp32
 *              accumulation and fp32 softmax statistics; FA_F32 inputs
 *              compute in fp32 throughout.
 *   Ownership  Every pointer is a device pointer owned by the caller.  The
 *              library never allocates or frees device memory and keeps no
 *              state between calls; calls on different streams are
 *              independent.
 *   Execution  Work is enqueued on `stream` (NULL = the default stream) and
 *              returns before it completes; there is no hidden synchronise.
 *   Errors     Arguments are validated before any HIP call; an invalid call
 *              returns a status and enqueues nothing.  A launch failure
 *              reported by the HIP runtime returns FA_ERR_HIP.  No entry
 *              point aborts or throws.
 *   Empty      B, H or Lq equal to 0 is valid and does no work (the backward
 *              with Lq = 0 still writes zero dK and dV).  Lk = 0 with Lq > 0
 *              is FA_ERR_SHAPE: a softmax over no keys is undefined.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_API __attribute__((visibility("default")))

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  FA_ERR_SHAPE = 2,       /* negative size, Lk = 0 with Lq > 0, or a size too
                             large for 32-bit per-slice offsets or for a
                             launch's 32-bit work-item count (B*H times the
                             longer length, times d/8 at bf16 or 32 at fp32,
                             over 2^32)                                         */
  FA_ERR_UNSUPPORTED = 3, /* valid request the kernels do not implement (head
                             dimension, dtype combination)                     */
  FA_ERR_ALIGN = 4,       /* a base pointer is not 16-byte aligned             */
  FA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required           */
  FA_ERR_HIP = 6,         /* the HIP runtime reported an error at launch       */
  FA_ERR_ARG = 7          /* non-finite scale, an unknown enum value, or a
                             split count outside [1, 4096]                     */
} fa_status;

typedef enum fa_dtype {
  FA_F32 = 0,
  FA_BF16 = 1
} fa_dtype;

/*
 * Forward: O and lse from Q, K, V.
 *   in_dtype   dtype of Q, K, V.
 *   out_dtype  dtype of O: equal to in_dtype, or FA_F32 with bf16 inputs
 *              (the fp32 accumulator divided by l, not rounded to bf16).
 *   B, H       batch and heads.  Lq, Lk: query and key lengths.  d: head
 *              dimension; supported: 64 and 128.
 *   Q          [B,H,Lq,d] in_dtype.   K, V: [B,H,Lk,d] in_dtype.
 *   scale      score multiplier (callers usually pass 1/sqrt(d)); finite.
 *   causal     nonzero: key j is hidden from query row i when j > i.
 *   O          [B,H,Lq,d] out_dtype, written.
 *   lse        [B,H,Lq] float, written: natural-log log-sum-exp of each
 *              row's scaled, masked scores (saved for the backward).
 * Per (b, h) slice, Lq*d and Lk*d times the element size must each stay
 * below 2^31 bytes.
 */
FA_API fa_status fa_fwd(fa_dtype in_dtype, fa_dtype out_dtype,
                 int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 const void* Q, const void* K, const void* V,
                 float scale, int causal,
                 void* O, float* lse, hipStream_t stream);

/*
 * Block-sparse forward: fa_fwd with whole 128 x 128 (query, key) blocks
 * removed from the attention pattern by a block mask, a generalisation of
 * the causal tile skip (glossary page "Flash Attention", FAQ on block-sparse
 * extensions: such a pattern is a different attention, kept apart from the
 * dense exact core; it is still computed exactly over what it keeps).
 *   block_mask   uint8 [mask_slices, ceil(Lq/128), ceil(Lk/128)] device
 *                memory (any alignment): entry [s][qb][kb] nonzero means
 *                queries 128 qb .. 128 qb + 127 of slice s may see keys
 *                128 kb .. 128 kb + 127.
 *   mask_slices  1 (one mask for every slice) or B*H (one per slice, in
 *                slice order b*H + h); other values are FA_ERR_ARG.
 * Element (i, j) of a slice is visible iff its block entry is nonzero and,
 * with `causal`, j <= i.  Softmax, O and lse are over the visible keys only;
 * a row that sees no key gets O = 0 and lse = -inf.  Other arguments,
 * layouts and status codes as for fa_fwd.  Supported: in_dtype FA_BF16, d in
 * {64, 128}, ceil(Lk/128) <= 4096 (else FA_ERR_UNSUPPORTED).  Work and time
 * scale with the visible blocks.
 */
FA_API fa_status fa_fwd_blocksparse(fa_dtype in_dtype, fa_dtype out_dtype,
                 int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 const void* Q, const void* K, const void* V,
                 float scale, int causal,
                 const uint8_t* block_mask, int64_t mask_slices,
                 void* O, float* lse, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes: the D statistic
 * (bf16 path: stored negated)
 * and lse in base 2 ([B,H,Lq] float each, each padded to a multiple of 256
 * bytes).  Linear in Lq; independent of the number of scores.  Returns 0
 * for sizes fa_bwd would reject.
 */
FA_API size_t fa_bwd_workspace_bytes(fa_dtype in_dtype, int64_t B, int64_t H,
                              int64_t Lq, int64_t Lk, int64_t d);

/*
 * Backward: dQ, dK, dV from Q, K, V, the forward's O and lse, and dO.
 * Probabilities are recomputed tile by tile from lse rather than read from
 * memory, with the row statistic D_i = sum_c dO_ic O_ic ("How Flash
 * Attention Improves Transformer Memory Efficiency ...", section "Backward
 * Pass Efficiency"; glossary page "Flash Attention", section "How it
 * works"); the gradients are the chain rule through the forward:
 * dV = P^T dO, dS = P * (dO V^T - D), dK = scale dS^T Q, dQ = scale dS K.
 * Equivalent to fa_bwd_prepare, then fa_bwd_dkdv and fa_bwd_dq on the same
 * stream, and to fa_bwd_prepare_dq then fa_bwd_dkdv (bit for bit, either
 * way).  No atomics: every gradient row is summed in a fixed order by one
 * workgroup, so results are bitwise reproducible.
 *   in_dtype   dtype of Q, K, V, dO, dQ, dK, dV.
 *   o_dtype    dtype of O, as the forward wrote it: equal to in_dtype, or
 *              FA_F32 with bf16 inputs (fa_fwd's fp32-output variant).  O
 *              enters only D = rowsum(dO * O), which is formed in fp32 from
 *              whichever O is given.  dO stays in in_dtype: it is an operand
 *              of the matrix products.  FA_F32 inputs with bf16 O return
 *              FA_ERR_UNSUPPORTED; a value that is not an fa_dtype returns
 *              FA_ERR_ARG.
 *   lse        the forward's [B,H,Lq] output.
 *   scale, causal  the values the forward was called with.
 *   dQ         [B,H,Lq,d], dK, dV: [B,H,Lk,d], written.
 *   workspace  device memory of at least fa_bwd_workspace_bytes(...) bytes,
 *              16-byte aligned; its contents on entry do not matter and are
 *              scratch afterwards.  Concurrent calls need separate
 *              workspaces.
 */
FA_API fa_status fa_bwd(fa_dtype in_dtype, fa_dtype o_dtype,
                 int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 const void* Q, const void* K, const void* V,
                 const void* O, const void* dO, const float* lse,
                 float scale, int causal,
                 void* dQ, void* dK, void* dV,
                 void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/*
 * The backward in three stages, for callers that run dK/dV and dQ on
 * different streams or time them apart.  Arguments mean what they mean for
 * fa_bwd, with the same shapes, layouts, alignment and status codes; each
 * stage validates only the pointers it uses.
 *
 * fa_bwd_prepare writes the per-row statistics (D and lse in base 2) into
 * `workspace`; it reads O in o_dtype (as for fa_bwd).  It must complete
 * before fa_bwd_dkdv or fa_bwd_dq starts reading that workspace (same
 * stream, or an event).
 */
FA_API fa_status fa_bwd_prepare(fa_dtype in_dtype, fa_dtype o_dtype,
                 int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 const void* O, const void* dO, const float* lse,
                 void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/*
 * fa_bwd_dkdv writes dK and dV ([B,H,Lk,d]); it reads the prepared
 * workspace and does not modify it.  Key-stationary: each workgroup owns a
 * block of keys and sums over every query tile that can see them.
 */
FA_API fa_status fa_bwd_dkdv(fa_dtype in_dtype,
                 int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 const void* Q, const void* K, const void* V, const void* dO,
                 float scale, int causal,
                 void* dK, void* dV,
                 const void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/*
 * fa_bwd_dq writes dQ ([B,H,Lq,d]); it reads the prepared workspace and
 * does not modify it.  Query-stationary: each workgroup owns a block of
 * queries and sums over every key tile they can see.  It may run
 * concurrently with fa_bwd_dkdv.
 */
FA_API fa_status fa_bwd_dq(fa_dtype in_dtype,
                 int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 const void* Q, const void* K, const void* V, const void* dO,
                 float scale, int causal,
                 void* dQ,
                 const void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/*
 * fa_bwd_prepare_dq is fa_bwd_prepare and fa_bwd_dq in one call: it writes
 * the per-row statistics into `workspace` and dQ.  With bf16 O both run in
 * one kernel (the dQ kernel forms D and lse in base 2 from the O, dO and
 * lse rows it reads anyway, with the prepare stage's arithmetic in the
 * same order, so the workspace and dQ get the same bits as the two stages
 * give); with fp32 O, or fp32 inputs, the two stages run one after the
 * other.  fa_bwd_dkdv can follow it on the same stream (this is what
 * fa_bwd does).  Arguments as for fa_bwd.
 */
FA_API fa_status fa_bwd_prepare_dq(fa_dtype in_dtype, fa_dtype o_dtype,
                 int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 const void* Q, const void* K, const void* V,
                 const void* O, const void* dO, const float* lse,
                 float scale, int causal,
                 void* dQ,
                 void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/*
 * Key-split forward, for a few query rows against a long key sequence (the
 * decode shape: generating one token attends its query to every cached key,
 * a single pass over K and V that memory traffic bounds -- blog page "What
 * Is FlashAttention? ...", section "What it changes for you"; explainer
 * page "Flash attention explained", section "Why this pattern keeps
 * recurring").  Same operation, arguments, layouts, masks and outputs as
 * fa_fwd; the keys are cut into `nsplit` ranges processed in parallel, and
 * the per-range results are merged exactly through their softmax
 * normalisers (annotated-code page, section "The Three Running
 * Statistics"):  lse = log sum_s exp(lse_s),  O = sum_s exp(lse_s - lse) O_s.
 *
 * Ranges.  chunk = 64 * ceil(ceil(Lk / nsplit) / 64); range s covers keys
 * [s*chunk, min((s+1)*chunk, Lk)).  Ranges past the end of the keys are
 * empty.  Causal masks keep their top-left meaning (absolute key and row
 * indices).
 *
 * Workspace layout (fp32, written by the partial stage, read by the merge):
 *   Opart   [nsplit, B, H, Lq, d] at byte 0: range s's output normalised by
 *           its own softmax sum (0 for a row that sees no key of the range);
 *   LSEpart [nsplit, B, H, Lq] at byte round_up(nsplit*B*H*Lq*d*4, 256):
 *           range s's natural-log lse (-inf for such a row).
 *
 * Supported: in_dtype FA_BF16, d in {64, 128}; out_dtype FA_BF16 or FA_F32.
 * FA_F32 inputs return FA_ERR_UNSUPPORTED (use fa_fwd).  1 <= nsplit <= 4096,
 * else FA_ERR_ARG.  Any Lq is accepted (query rows go in blocks of 16);
 * long query blocks are faster through fa_fwd.
 */

/* A split count that fills the current device (its compute-unit count)
 * for these sizes: at least two workgroups per compute unit where the keys
 * allow, with ranges of at least 256 keys.  Returns 1 for empty or invalid
 * sizes.  Makes one HIP query of the current device. */
FA_API int64_t fa_fwd_splitkv_default_splits(int64_t B, int64_t H, int64_t Lq,
                 int64_t Lk, int64_t d);

/* Bytes of workspace for nsplit ranges (layout above); 0 for sizes or
 * nsplit the call would reject. */
FA_API size_t fa_fwd_splitkv_workspace_bytes(fa_dtype in_dtype,
                 int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 int64_t nsplit);

/* Partial stage then merge, on `stream`.  Arguments as for fa_fwd, plus
 * nsplit and a 16-byte-aligned workspace of at least
 * fa_fwd_splitkv_workspace_bytes(...) bytes (contents on entry do not
 * matter; scratch afterwards; concurrent calls need separate workspaces). */
FA_API fa_status fa_fwd_splitkv(fa_dtype in_dtype, fa_dtype out_dtype,
                 int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 const void* Q, const void* K, const void* V,
                 float scale, int causal, int64_t nsplit,
                 void* O, float* lse,
                 void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* Partial stage alone: writes Opart and LSEpart into the workspace. */
FA_API fa_status fa_fwd_splitkv_partial(fa_dtype in_dtype,
                 int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 const void* Q, const void* K, const void* V,
                 float scale, int causal, int64_t nsplit,
                 void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* Merge stage alone: reads Opart and LSEpart (for these B, H, Lq, d and
 * nsplit) from the workspace and writes O ([B,H,Lq,d], out_dtype) and lse
 * ([B,H,Lq] float).  Every row must have at least one finite LSEpart entry
 * (true for anything the partial stage wrote). */
FA_API fa_status fa_fwd_splitkv_merge(fa_dtype out_dtype,
                 int64_t B, int64_t H, int64_t Lq, int64_t d, int64_t nsplit,
                 const void* workspace, size_t workspace_bytes,
                 void* O, float* lse, hipStream_t stream);

/*
 * Block-sparse backward: fa_bwd for the attention fa_fwd_blocksparse
 * computes, with the same block_mask and mask_slices.  The gradients are the
 * chain rule through the masked definition (P is zero outside the kept
 * pairs; a row that sees no key contributes nothing).  lse and O must be
 * fa_fwd_blocksparse's outputs (rows that see no key: O = 0, lse = -inf).
 * o_dtype, workspace, layouts and status codes as for fa_bwd; supported: in_dtype
 * FA_BF16, d in {64, 128}, ceil(Lq/128) and ceil(Lk/128) <= 4096 (else
 * FA_ERR_UNSUPPORTED).  The key-side kernel visits only the query blocks
 * that see its key block; the query side only the key blocks its 128-row
 * block (one row block of the mask) sees.
 */
FA_API fa_status fa_bwd_blocksparse(fa_dtype in_dtype, fa_dtype o_dtype,
                 int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 const void* Q, const void* K, const void* V,
                 const void* O, const void* dO, const float* lse,
                 float scale, int causal,
                 const uint8_t* block_mask, int64_t mask_slices,
                 void* dQ, void* dK, void* dV,
                 void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): fa_bwd
 * with no workspace argument.  The per-row statistics (D and base-2 lse)
 * go to a fixed array inside the library, one per GPU, of
 * fa_bwd_noalloc_max_scratch_bytes() bytes (16 MiB: up to 2^21 query rows,
 * B*H*Lq); each GPU holds its copy until the process ends.  Sizes whose
 * statistics need more return FA_ERR_WORKSPACE before any HIP call.  The
 * call allocates and frees nothing.
 *
 * Every call on one GPU uses that GPU's array: calls that overlap in time
 * on one GPU (different streams, or different threads) race and must be
 * ordered by the caller.  The array keeps the previous call's contents;
 * nothing in it needs to start at zero.  The first call on a device looks
 * up the array's device address (with that device current), which needs no
 * allocation.  Other arguments, checks, outputs and status codes as for
 * fa_bwd; the results are bitwise those of fa_bwd.
 */
FA_API size_t fa_bwd_noalloc_max_scratch_bytes(void);
FA_API fa_status fa_bwd_noalloc(fa_dtype in_dtype, fa_dtype o_dtype,
                 int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 const void* Q, const void* K, const void* V,
                 const void* O, const void* dO, const float* lse,
                 float scale, int causal,
                 void* dQ, void* dK, void* dV, hipStream_t stream);

/* Static description of a status code; never NULL. */
FA_API const char* fa_status_str(fa_status s);

/* Library version and target, e.g. "libfa 0.1.0 gfx950". */
FA_API const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
