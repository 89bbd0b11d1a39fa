/*
 * transpose_f32.h -- C ABI of the fp32 matrix transpose in the MI355X
 * (gfx950) GEMM library (libgemm_tn.so).
 *
 *     y[b][j][i] = x[b][i][j],   x: batch x M x N,  y: batch x N x M
 *
 * The operation of page "Mat Transpose CuTe 版代码学习" (chuoer47.github.io,
 * the reg kernel and its host wrappers: x is an M x N row-major matrix, y
 * the N x M row-major transpose, and a coordinate mask keeps the edge
 * tiles of ragged shapes in bounds).  The copy is exact: every output word
 * is an input word.
 *
 * Layout: x and y are packed row-major matrices of IEEE binary32; batch
 * entry b of x starts at x + b*M*N, of y at y + b*N*M.  16-byte-aligned
 * pointers with M and N multiples of 4 take 16-byte loads and stores;
 * anything else is handled element by element (same results).
 *
 * Ownership, asynchrony, threading and errors are as for gemm_tn (see
 * gemm_tn.h): device pointers owned by the caller, work enqueued on
 * `stream` (a hipStream_t), a gemm_tn_status returned, arguments checked
 * before any HIP call.  No memory is allocated.
 *
 * Errors: GEMM_TN_ERR_INVALID_ARG for negative sizes, NULL x or y with
 * batch*M*N > 0, size overflow, or x and y overlapping;
 * GEMM_TN_ERR_UNSUPPORTED for M or N above 2^23 (the kernel's 32-bit
 * offsets within a 64-row tile band); GEMM_TN_ERR_LAUNCH when the HIP
 * runtime rejects the launch.  batch, M or N == 0 is a no-op.
 */
#ifndef TRANSPOSE_F32_H
#define TRANSPOSE_F32_H

#include <stdint.h>

#include "gemm_tn.h"

#ifdef __cplusplus
extern "C" {
#endif

int transpose_f32(int64_t batch, int64_t M, int64_t N, const void *x,
                  void *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TRANSPOSE_F32_H */
