/*
 * gemm_f16acc.h -- C ABI of the fp16-accumulating TN GEMM in the MI355X
 * (gfx950) GEMM library (libgemm_tn.so).
 *
 *     D[b] = A[b] * B[b]^T,  A: M x K, B: N x K, D: M x N, all binary16,
 *     with the running sum rounded to binary16 after every 16-deep step:
 *         acc_0 = 0,
 *         acc_{s+1} = rn16(acc_s + sum_{k=16s}^{16s+15} a(i,k) b(j,k)),
 *         d(i,j) = acc_{ceil(K/16)}
 *     (rn16: round to nearest even, overflow to +-inf).
 *
 * This is the arithmetic of the MMA atom of page "cute(8) smem_gemm"
 * (yuyanqi.com, kernel listing and section 2.3): fp16 A, B, C and D, 16 deep
 * in K, so the accumulator is an fp16 value after every step; the page's
 * kernel has no alpha, beta or C.  The 16-term sum of a step is formed in
 * fp32 before the rounding (exact for integer-valued inputs; otherwise it
 * can move a rounding decision by one fp16 spacing).  gemm_tn() is the
 * fp32-accumulating GEMM and is the one to use for accuracy.
 *
 * Layout: packed row-major, K-contiguous A and B (lda = ldb = K), D with
 * ldd = N; batch entry b at A + b*strideA, B + b*strideB, D + b*strideD
 * (elements).  strideA or strideB 0 broadcasts that operand; batches of D
 * must not overlap.  16-byte loads are used when K is a multiple of 8 and A
 * and B are 16-byte aligned (strides multiples of 8); any other shape or
 * alignment takes an element-wise loader with the same results.
 *
 * Ownership, asynchrony, threading: as for gemm_tn (see gemm_tn.h).  No
 * memory is allocated.
 *
 * Errors: GEMM_TN_ERR_INVALID_ARG for negative sizes or strides, NULL D (or
 * A, B with K > 0), size overflow, overlapping batches of D, or D
 * overlapping A or B; GEMM_TN_ERR_UNSUPPORTED for K > 2^21, N > 2^20 or
 * more than 2^31 - 1 workgroups; GEMM_TN_ERR_LAUNCH when the launch fails.
 * batch, M or N == 0 is a no-op; K == 0 writes zeros.
 */
#ifndef GEMM_F16ACC_H
#define GEMM_F16ACC_H

#include <stdint.h>

#include "gemm_tn.h"

#ifdef __cplusplus
extern "C" {
#endif

int gemm_tn_f16acc(int64_t batch, int64_t M, int64_t N, int64_t K,
                   const void *A, int64_t strideA, const void *B,
                   int64_t strideB, void *D, int64_t strideD, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F16ACC_H */
