/*
 * CPU oracle for the fp16 TN GEMM  D = alpha * A * B^T + beta * C.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or table with the HIP
 * library; the only thing the two sides share is the seeded input bits.
 *
 * What it computes, and where that is defined:
 *   - the operation C = alpha*A*B + beta*C with A addressed (M,K) and B
 *     addressed (N,K): page "gemm_device line-by-line walk-through"
 *     (flagos.csdn.net), section 1 (the kernel's parameter list, the mA/mB
 *     views, the reference loops equivalent to gemm() and axpby());
 *   - the TN storage (A is M x K row-major, B is N x K row-major, D is M x N
 *     row-major): page "cute(8) smem_gemm" (yuyanqi.com), the kernel listing
 *     in "代码实现" (the make_stride(K,1) / make_stride(N,1) views);
 *   - C kept separate from D, fp32 accumulation, C unread when beta == 0:
 *     readings taken where the pages are silent or disagree (the first page
 *     accumulates in fp16 with no alpha/beta; the second updates C in place).
 *
 * Method: every fp16 input is decoded exactly to double (IEEE 754 binary16
 * definition), every product a*b is then exact in double (at most 22
 * significant bits), and the k-sum runs sequentially in double.  The fp64
 * rounding error is at most (K-1) * 2^-53 * sum|a*b|, far below the GPU
 * tolerance, so the result stands for the exact value.
 *
 * Built with gcc -O2 -ffp-contract=off (no fused multiply-add, no
 * fast-math); output rows are split across POSIX threads, each element is
 * computed by one thread in the serial order, so the thread count never
 * changes a result.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- IEEE 754 binary16 codec ------------------------------------------ */

/* bits s|e(5)|m(10):  e = 0 -> (-1)^s * m * 2^-24 (zero / subnormal);
 * 1 <= e <= 30 -> (-1)^s * (1024 + m) * 2^(e - 25);  e = 31 -> inf / NaN. */
double gemm_oracle_half_to_double(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = (m == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* Round-to-nearest, ties-to-even encode of a double to binary16.  The
 * rounding is done on the integer significand scaled to the target
 * quantum, so no intermediate float rounding is involved.  Values whose
 * rounded magnitude reaches 2^16 become infinity. */
uint16_t gemm_oracle_double_to_half(double x)
{
    if (isnan(x))
        return 0x7E00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a))
        return sign | 0x7C00;
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;                /* a in [2^e, 2^(e+1)) */
    if (e < -14)
        e = -14;                   /* subnormal range shares one quantum */
    double q = ldexp(1.0, e - 10); /* spacing of binary16 values near a */
    double t = a / q;              /* exact: q is a power of two */
    double fl = floor(t);
    double rem = t - fl;           /* exact */
    double n = fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0))
        n = fl + 1.0;
    /* n * q is the rounded magnitude; n may have carried to 2048 */
    double r = n * q;
    if (r >= 65536.0)
        return sign | 0x7C00;
    if (r < ldexp(1.0, -14))       /* subnormal or zero: field = n */
        return sign | (uint16_t)n;
    int re;
    frexp(r, &re);
    int be = re - 1;               /* r in [2^be, 2^(be+1)) */
    uint16_t mant = (uint16_t)(ldexp(r, 10 - be) - 1024.0);
    return sign | (uint16_t)((be + 15) << 10) | mant;
}

/* Round-to-nearest-even to binary32: C's conversion under the default
 * IEEE rounding mode is exactly that. */
float gemm_oracle_double_to_float(double x)
{
    return (float)x;
}

void gemm_oracle_decode_f16(const uint16_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = gemm_oracle_half_to_double(src[i]);
}

void gemm_oracle_encode_f16(const double *src, uint16_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = gemm_oracle_double_to_half(src[i]);
}

void gemm_oracle_encode_f32(const double *src, float *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = gemm_oracle_double_to_float(src[i]);
}

/* ---- the GEMM ---------------------------------------------------------- */

enum { ORACLE_C_F16 = 0, ORACLE_C_F32 = 1 };

static double load_c(const void *C, int c_dtype, int64_t idx)
{
    if (c_dtype == ORACLE_C_F16)
        return gemm_oracle_half_to_double(((const uint16_t *)C)[idx]);
    return (double)((const float *)C)[idx];
}

/* One output element: s = sum_k a(i,k) * b(j,k) in sequential k order, then
 * ref = alpha*s + beta*c (the c term only when beta != 0). */
static double element(const double *arow, const double *brow, int64_t bstep,
                      int64_t K, double alpha, double beta, const void *C,
                      int c_dtype, int64_t cidx)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k)
        s += arow[k] * brow[k * bstep];
    double r = alpha * s;
    if (beta != 0.0)
        r = r + beta * load_c(C, c_dtype, cidx);
    return r;
}

typedef struct {
    int64_t batch, M, N, K;
    double alpha, beta;
    const double *a, *b;     /* decoded operands */
    const void *C;
    int c_dtype;
    double *ref;
    int64_t row_begin, row_end;  /* flattened (batch, m) rows */
    int64_t next;                /* shared work counter */
    pthread_mutex_t lock;
} gemm_job;

static void *gemm_worker(void *p)
{
    gemm_job *job = (gemm_job *)p;
    for (;;) {
        pthread_mutex_lock(&job->lock);
        int64_t r = job->next++;
        pthread_mutex_unlock(&job->lock);
        r += job->row_begin;
        if (r >= job->row_end)
            break;
        int64_t bi = r / job->M;
        const double *arow = job->a + r * job->K;
        for (int64_t j = 0; j < job->N; ++j) {
            const double *brow = job->b + (bi * job->N + j) * job->K;
            int64_t bstep = 1;
            int64_t cidx = r * job->N + j;
            job->ref[(r - job->row_begin) * job->N + j] =
                element(arow, brow, bstep, job->K, job->alpha, job->beta,
                        job->C, job->c_dtype, cidx);
        }
    }
    return NULL;
}

/* Rows [row_begin, row_end) of the flattened (batch*M) x N result, written
 * to ref (row-major, (row_end-row_begin) x N).  A is batch x M x K fp16 bits,
 * B is batch x N x K fp16 bits, C (if beta != 0) batch x M x N in c_dtype.
 * Returns 0, or -1 on bad arguments / allocation failure. */
int gemm_oracle_tn_rows(int64_t batch, int64_t M, int64_t N, int64_t K,
                        double alpha, const uint16_t *A, const uint16_t *B,
                        double beta, const void *C, int c_dtype, double *ref,
                        int64_t row_begin, int64_t row_end, int nthreads)
{
    if (batch < 0 || M < 0 || N < 0 || K < 0 || row_begin < 0 ||
        row_end > batch * M || row_begin > row_end || nthreads < 1)
        return -1;
    if (beta != 0.0 && C == NULL)
        return -1;
    int64_t rows = row_end - row_begin;
    if (rows == 0 || N == 0)
        return 0;
    /* Decode the A rows needed and all of B for the batches touched. */
    int64_t b_first = row_begin / (M ? M : 1);
    int64_t b_last = (row_end - 1) / (M ? M : 1);
    double *a = (double *)malloc(sizeof(double) * (size_t)(batch * M * K + 1));
    double *b = (double *)malloc(sizeof(double) * (size_t)(batch * N * K + 1));
    if (!a || !b) {
        free(a);
        free(b);
        return -1;
    }
    gemm_oracle_decode_f16(A + row_begin * K, a + row_begin * K, rows * K);
    gemm_oracle_decode_f16(B + b_first * N * K, b + b_first * N * K,
                           (b_last - b_first + 1) * N * K);

    gemm_job job;
    memset(&job, 0, sizeof job);
    job.batch = batch; job.M = M; job.N = N; job.K = K;
    job.alpha = alpha; job.beta = beta;
    job.a = a; job.b = b; job.C = C; job.c_dtype = c_dtype; job.ref = ref;
    job.row_begin = row_begin; job.row_end = row_end; job.next = 0;
    pthread_mutex_init(&job.lock, NULL);
    if (nthreads > rows)
        nthreads = (int)rows;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[started], NULL, gemm_worker, &job) == 0)
            ++started;
    gemm_worker(&job);  /* the calling thread works too */
    for (int t = 0; t < started; ++t)
        pthread_join(th[t], NULL);
    pthread_mutex_destroy(&job.lock);
    free(th);
    free(a);
    free(b);
    return 0;
}

/* The whole result: ref is batch x M x N doubles. */
int gemm_oracle_tn(int64_t batch, int64_t M, int64_t N, int64_t K,
                   double alpha, const uint16_t *A, const uint16_t *B,
                   double beta, const void *C, int c_dtype, double *ref,
                   int nthreads)
{
    return gemm_oracle_tn_rows(batch, M, N, K, alpha, A, B, beta, C, c_dtype,
                               ref, 0, batch * M, nthreads);
}

/* Selected elements only: pts holds npts triples (b, i, j).  Used at sizes
 * where the full result would take too long; each value is the same
 * element() the full oracle computes. */
int gemm_oracle_tn_points(int64_t batch, int64_t M, int64_t N, int64_t K,
                          double alpha, const uint16_t *A, const uint16_t *B,
                          double beta, const void *C, int c_dtype,
                          const int64_t *pts, int64_t npts, double *out)
{
    if (batch < 0 || M < 0 || N < 0 || K < 0 || npts < 0)
        return -1;
    if (beta != 0.0 && C == NULL)
        return -1;
    double *arow = (double *)malloc(sizeof(double) * (size_t)(K + 1));
    double *brow = (double *)malloc(sizeof(double) * (size_t)(K + 1));
    if (!arow || !brow) {
        free(arow);
        free(brow);
        return -1;
    }
    int rc = 0;
    for (int64_t p = 0; p < npts; ++p) {
        int64_t bi = pts[3 * p], i = pts[3 * p + 1], j = pts[3 * p + 2];
        if (bi < 0 || bi >= batch || i < 0 || i >= M || j < 0 || j >= N) {
            rc = -1;
            break;
        }
        gemm_oracle_decode_f16(A + (bi * M + i) * K, arow, K);
        gemm_oracle_decode_f16(B + (bi * N + j) * K, brow, K);
        out[p] = element(arow, brow, 1, K, alpha, beta, C, c_dtype,
                         (bi * M + i) * N + j);
    }
    free(arow);
    free(brow);
    return rc;
}
