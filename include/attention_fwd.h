/*
 * attention_fwd.h -- C ABI of the attention forward pass in the MI355X
 * (gfx950) GEMM library (libgemm_tn.so).
 *
 *     S = scale * Q K^T,   P = softmax of each row of S,   O = P V
 *     lse = log(sum_j exp(S[i][j]))  (natural log, one value per query)
 *
 * for `batch` independent heads.  The score product is the TN product of
 * page "为什么 cutlass_cute_tutorial_zh.md 中要用 retile_D"
 * (blog.qingsen.net): score = Q @ K.T with Q as the A operand and K as the
 * B operand, fp16 operands accumulated in fp32 (sections 1 and 2), head
 * dimension 64 (section 3), taken from a FlashAttention-style tutorial;
 * the softmax and the P V product complete that forward pass.
 *
 * Precision: Q, K, V are IEEE binary16.  Scores are accumulated in fp32;
 * the softmax runs in fp32 with a per-row shift by a running maximum; the
 * probabilities are rounded to fp16 for the P V product, which accumulates
 * in fp32; each row is divided by its fp32 sum at the end and rounded once
 * (round to nearest even) to the output type.
 *
 * Layout (packed, row-major, per head h):
 *   Q at Q + h*Lq*d, element (i, x) at i*d + x       (Lq x d)
 *   K at K + h*Lk*d, element (j, x) at j*d + x       (Lk x d)
 *   V at V + h*Lk*d, element (j, x) at j*d + x       (Lk x d)
 *   O at O + h*Lq*d, element (i, x) at i*d + x       (Lq x d), o_dtype
 *   lse at lse + h*Lq + i (fp32), written only when lse != NULL.
 * Q, K, V and O must be 16-byte aligned, lse 4-byte aligned.
 *
 * Ownership, asynchrony, threading: device pointers owned by the caller;
 * work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 * and the call returns without waiting.  No memory is allocated.
 *
 * Errors (checked before any HIP call; nothing is enqueued on error):
 *   GEMM_TN_ERR_INVALID_ARG : negative sizes; Lk == 0 with work to do (a
 *       softmax over no keys is undefined); a non-finite scale; o_dtype
 *       not GEMM_TN_F16 / GEMM_TN_F32; NULL Q, K, V or O with work to do;
 *       size overflow; O or lse overlapping an input or each other;
 *   GEMM_TN_ERR_UNSUPPORTED : d != 64; Lk > 2^23; misaligned pointers;
 *       more than 2^31 - 1 workgroups;
 *   GEMM_TN_ERR_LAUNCH : the HIP runtime rejected the launch.
 * batch == 0 or Lq == 0 is a no-op.
 */
#ifndef ATTENTION_FWD_H
#define ATTENTION_FWD_H

#include <stdint.h>

#include "gemm_tn.h"

#ifdef __cplusplus
extern "C" {
#endif

int attention_fwd(int64_t batch, int64_t Lq, int64_t Lk, int64_t d,
                  float scale, const void *Q, const void *K, const void *V,
                  void *O, int o_dtype, void *lse, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTENTION_FWD_H */
