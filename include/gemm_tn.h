/*
 * gemm_tn.h -- C ABI of the MI355X (gfx950) half-precision TN GEMM library.
 *
 *     D = alpha * A * B^T + beta * C
 *
 * The operation is the one the CuTe tutorial kernel gemm_device computes
 * (page "gemm_device line-by-line walk-through", flagos.csdn.net, section 1:
 * C = alpha*A*B + beta*C with B addressed as an N x K matrix), in the TN
 * storage of page "cute(8) smem_gemm" (yuyanqi.com, kernel listing): A is
 * M x K row-major, B is N x K row-major, so both operands are contiguous
 * along K.  Readings where the pages are silent or disagree:
 *   - accumulation is fp32 (the first page's kernel accumulates in fp16;
 *     the fp32-accumulating atom of page "why retile_D", blog.qingsen.net,
 *     section 2, is the one followed);
 *   - C and D are separate arguments (C may equal D: every element of C is
 *     read by the thread that writes the same element of D, before it
 *     writes it);
 *   - C is not read when beta == 0 (it may then be NULL; NaN in C does not
 *     propagate); alpha is never special-cased;
 *   - the fp32 result alpha*acc + beta*c is rounded to the output type with
 *     round-to-nearest-even (fp16 overflow gives +-inf);
 *   - K == 0 gives D = beta*C (an empty sum); M == 0 or N == 0 is a no-op.
 *
 * Layout: every matrix is row-major.  gemm_tn and gemm_tn_strided_batched
 * take A as M x K and B as N x K with packed rows (lda = ldb = K,
 * ldc = ldd = N); gemm_tn_ex takes any row strides, and A or B may instead
 * be stored transposed (K x M, K x N), as gemm_device takes a stride per
 * matrix (page "gemm_device line-by-line walk-through", section 1: the
 * global tensors are built from a pointer, a shape and the strides dA, dB,
 * dC, so either mode of A and B may be the contiguous one).
 * Element types: A and B are IEEE binary16; C and D share `d_dtype`.
 *
 * Ownership and asynchrony: the caller owns every buffer; they are device
 * pointers (or any address the GPU can read/write, e.g. managed memory).
 * The library never frees or retains them.  Calls enqueue work on `stream`
 * (a hipStream_t, NULL for the default stream) and return at once; device
 * faults surface at the caller's next synchronisation.  The only memory the
 * library allocates itself is a per-(device, stream) fp32 workspace for the
 * split-K path (skinny problems with a long K, and the bottom tile rows of
 * problems whose whole-tile grid would leave a mostly idle last wave: those
 * rows are split along K while the rows above run as whole tiles); it is
 * grown on demand and kept until the process ends.
 *
 * Errors: every entry point returns a gemm_tn_status; the library never
 * exits or aborts.  Arguments are fully validated before any HIP call, so
 * an error return means nothing was enqueued.
 *
 * Thread safety: calls may come from several host threads, on one stream
 * or on several.  Calls on different streams that both take the split-K
 * path use different workspaces and do not race; calls on one stream share
 * its workspace in stream order (a call that must grow it waits for the
 * stream's earlier work before freeing the old buffer, and holds the
 * workspace until its own kernels are enqueued).
 */
#ifndef GEMM_TN_H
#define GEMM_TN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of C and D. */
typedef enum gemm_tn_dtype {
    GEMM_TN_F16 = 0, /* IEEE binary16 */
    GEMM_TN_F32 = 1  /* IEEE binary32 */
} gemm_tn_dtype;

/* Storage of an operand (gemm_tn_ex). */
typedef enum gemm_tn_layout {
    GEMM_TN_ROW_K = 0,  /* contiguous along K: A(m,k) = A[m*lda + k],
                           B(n,k) = B[n*ldb + k] (the TN layout) */
    GEMM_TN_ROW_MN = 1  /* contiguous along M / N: A(m,k) = A[k*lda + m],
                           B(n,k) = B[k*ldb + n] */
} gemm_tn_layout;

typedef enum gemm_tn_status {
    GEMM_TN_OK = 0,
    GEMM_TN_ERR_INVALID_ARG = 1, /* negative size, NULL where data is needed,
                                    bad dtype, a row stride shorter than its
                                    row, overlapping batches of D, size
                                    overflow */
    GEMM_TN_ERR_UNSUPPORTED = 2, /* sizes beyond the kernels' addressing
                                    range: K or an A/B row stride > 2^21
                                    (so M or N > 2^21 for an operand stored
                                    along M / N), N or a C/D row stride >
                                    2^20, or M > 2^31 - 1 */
    GEMM_TN_ERR_LAUNCH = 3,      /* the HIP runtime rejected a launch */
    GEMM_TN_ERR_WORKSPACE = 4,   /* the split-K workspace could not be
                                    allocated */
    GEMM_TN_ERR_SCRATCH = 5      /* gemm_tn_ex_noalloc: the problem's
                                    split-K plan needs more than
                                    GEMM_TN_NOALLOC_SCRATCH_BYTES */
} gemm_tn_status;

/* Size of the fixed per-GPU scratch of gemm_tn_ex_noalloc (64 MiB): the
   most partials any plan of the library's own choosing writes (one wave of
   256 x 256 fp32 tiles), so only a forced plan can need more. */
#define GEMM_TN_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)

/*
 * One GEMM.  M, N, K >= 0.
 *   A : M x K binary16, row-major (element (m,k) at A[m*K + k]); may be
 *       NULL only when M*K == 0.
 *   B : N x K binary16, row-major (element (n,k) at B[n*K + k]); may be
 *       NULL only when N*K == 0.
 *   C : M x N of d_dtype, row-major; read only when beta != 0 (then it must
 *       not be NULL when M*N > 0); may equal D.
 *   D : M x N of d_dtype, row-major; written (every element, nothing else).
 *   d_dtype : GEMM_TN_F16 or GEMM_TN_F32.
 *   stream  : hipStream_t to enqueue on.
 * Any element-aligned pointer is accepted; 16-byte-aligned A/B with K a
 * multiple of 8 select the vector loader, otherwise an element-granular
 * loader runs (slower, same results).
 */
int gemm_tn(int64_t M, int64_t N, int64_t K, float alpha, const void *A,
            const void *B, float beta, const void *C, void *D, int d_dtype,
            void *stream);

/*
 * `batch` independent GEMMs of the same shape, matrix i at
 *   A + i*strideA,  B + i*strideB,  C + i*strideC,  D + i*strideD
 * (strides in elements, >= 0; a zero A or B stride broadcasts one operand).
 * Batches of D must not overlap: strideD >= M*N when batch > 1.  The
 * batched score product S = Q * K^T of an attention head is this call with
 * A = Q, B = K (page "why retile_D", blog.qingsen.net, section 1: Q is the
 * A operand and K the B operand of the score GEMM).
 */
int gemm_tn_strided_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                            float alpha, const void *A, int64_t strideA,
                            const void *B, int64_t strideB, float beta,
                            const void *C, int64_t strideC, void *D,
                            int64_t strideD, int d_dtype, void *stream);

/*
 * The general form: gemm_tn_strided_batched with a row stride (leading
 * dimension, in elements) per matrix, so that any row-major sub-matrix of
 * a larger array can be an operand or the output, and with the storage of
 * A and B chosen by layout_a / layout_b (gemm_tn_layout):
 *   A(m,k) = A[i*strideA + m*lda + k],   lda >= K   (GEMM_TN_ROW_K)
 *            A[i*strideA + k*lda + m],   lda >= M   (GEMM_TN_ROW_MN)
 *   B(n,k) = B[i*strideB + n*ldb + k],   ldb >= K   (GEMM_TN_ROW_K)
 *            B[i*strideB + k*ldb + n],   ldb >= N   (GEMM_TN_ROW_MN)
 *   C(m,n) = C[i*strideC + m*ldc + n],   ldc >= N
 *   D(m,n) = D[i*strideD + m*ldd + n],   ldd >= N
 * Only the M x N elements of each D are written; the ldd - N elements
 * between rows are left untouched, and no padding of A, B or C is read.
 * Batches of D must not overlap: strideD >= (M - 1)*ldd + N when
 * batch > 1.  The 16-byte loaders need K-contiguous operands with lda and
 * ldb multiples of 8 (otherwise the element loader runs); 16-byte stores
 * need ldd (and ldc when C is read) to keep rows on 16-byte boundaries.
 * An unknown layout value is GEMM_TN_ERR_INVALID_ARG.
 */
int gemm_tn_ex(int64_t batch, int64_t M, int64_t N, int64_t K, float alpha,
               const void *A, int layout_a, int64_t lda, int64_t strideA,
               const void *B, int layout_b, int64_t ldb, int64_t strideB,
               float beta, const void *C, int64_t ldc, int64_t strideC,
               void *D, int64_t ldd, int64_t strideD, int d_dtype,
               void *stream);

/*
 * gemm_tn_ex for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results (bit for bit) as
 * gemm_tn_ex.  Where gemm_tn_ex would allocate or grow its per-stream
 * split-K workspace (skinny problems split along K, and the tail split of
 * a grid ending in a mostly idle wave), this entry point uses a fixed
 * device array of GEMM_TN_NOALLOC_SCRATCH_BYTES instead, one per GPU,
 * held until the process ends; it calls no hipMalloc or hipFree.
 *   - A problem whose plan needs more partials than that (splits x batch x
 *     M x round_up(N, 4) x 4 bytes, or the tail rows' share) returns
 *     GEMM_TN_ERR_SCRATCH and launches nothing.  The library's own plans
 *     never do; a plan forced through the GEMM_TN_FORCE environment
 *     variable (a tuning override read on every call) can.
 *   - Every call on one GPU shares that GPU's array: calls that overlap on
 *     one GPU (several streams or host threads at once) race on it, and
 *     the caller must order them.  Nothing in it has to start at zero: each
 *     call writes every partial it reads.
 *   - The array's device address is looked up once per device, on the
 *     first call with that device current.
 */
int gemm_tn_ex_noalloc(int64_t batch, int64_t M, int64_t N, int64_t K,
                       float alpha, const void *A, int layout_a, int64_t lda,
                       int64_t strideA, const void *B, int layout_b,
                       int64_t ldb, int64_t strideB, float beta,
                       const void *C, int64_t ldc, int64_t strideC, void *D,
                       int64_t ldd, int64_t strideD, int d_dtype,
                       void *stream);

/*
 * Name of the kernel configuration gemm_tn_ex would launch for this
 * problem (tile shape, loader, split-K factor, and the tail split: the
 * number of bottom tile rows split along K and into how many slices),
 * written NUL-terminated into buf (at most buflen bytes).  aligned16 != 0 means every matrix
 * pointer is 16-byte aligned.  Pure host logic, no HIP call.  Returns
 * GEMM_TN_OK or the status the GEMM call would return for these sizes.
 */
int gemm_tn_describe(int64_t batch, int64_t M, int64_t N, int64_t K,
                     int layout_a, int64_t lda, int layout_b, int64_t ldb,
                     int64_t ldc, int64_t ldd, int64_t strideA,
                     int64_t strideB, int64_t strideC, int64_t strideD,
                     float beta, int d_dtype, int aligned16, char *buf,
                     int64_t buflen);

/* Human-readable text of a status code (static storage). */
const char *gemm_tn_status_string(int status);

/* Library ABI version: (major << 16) | minor (currently 1.2). */
int gemm_tn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_TN_H */
