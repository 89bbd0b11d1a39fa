/*
 * A plain C program that uses the library through its C ABI only (no
 * Python, no torch): device memory from the HIP runtime, every entry point
 * called once on inputs whose results have a closed form, each result
 * checked on the host.  Exit status 0 when every check passes.
 *
 * Built by __graft_entry__.build() (gcc, host code only) and run by
 * tests/test_c_abi_gpu.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "attention_fwd.h"
#include "gemm_f16acc.h"
#include "gemm_tn.h"
#include "transpose_f32.h"

#define F16_ONE 0x3C00u
#define F16_TWO 0x4000u
#define F16_THREE 0x4200u

static int failures = 0;

#define HIP_OK(call)                                                        \
    do {                                                                    \
        hipError_t e_ = (call);                                             \
        if (e_ != hipSuccess) {                                             \
            fprintf(stderr, "%s:%d: %s failed: %s\n", __FILE__, __LINE__,   \
                    #call, hipGetErrorString(e_));                          \
            exit(2);                                                        \
        }                                                                   \
    } while (0)

static void expect(int ok, const char *what)
{
    printf("%-60s %s\n", what, ok ? "ok" : "FAILED");
    if (!ok)
        ++failures;
}

static void *dev_fill16(size_t n, uint16_t bits)
{
    uint16_t *h = malloc(n * 2);
    for (size_t i = 0; i < n; ++i)
        h[i] = bits;
    void *d;
    HIP_OK(hipMalloc(&d, n * 2));
    HIP_OK(hipMemcpy(d, h, n * 2, hipMemcpyHostToDevice));
    free(h);
    return d;
}

static void *dev_fill32(size_t n, float v)
{
    float *h = malloc(n * 4);
    for (size_t i = 0; i < n; ++i)
        h[i] = v;
    void *d;
    HIP_OK(hipMalloc(&d, n * 4));
    HIP_OK(hipMemcpy(d, h, n * 4, hipMemcpyHostToDevice));
    free(h);
    return d;
}

/* binary16 -> float for the few values read back here (normal numbers) */
static float f16_to_f32(uint16_t h)
{
    const int e = (h >> 10) & 31, m = h & 1023;
    const float s = (h & 0x8000) ? -1.0f : 1.0f;
    if (e == 0)
        return s * ldexpf((float)m, -24);
    return s * ldexpf((float)(1024 + m), e - 25);
}

int main(void)
{
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    const int v = gemm_tn_version();
    printf("libgemm_tn version %d.%d\n", v >> 16, v & 0xFFFF);

    /* 1. gemm_tn: A = 1, B = 2, C = 3, alpha = 0.5, beta = 1, fp32 D:
     *    every element is 0.5 * 2 * K + 3. */
    {
        const int64_t M = 512, N = 384, K = 640;
        void *A = dev_fill16(M * K, F16_ONE), *B = dev_fill16(N * K, F16_TWO);
        void *C = dev_fill32(M * N, 3.0f), *D = dev_fill32(M * N, -1.0f);
        int st = gemm_tn(M, N, K, 0.5f, A, B, 1.0f, C, D, GEMM_TN_F32,
                         stream);
        float *h = malloc(M * N * 4);
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipMemcpy(h, D, M * N * 4, hipMemcpyDeviceToHost));
        int ok = st == GEMM_TN_OK;
        for (int64_t i = 0; i < M * N && ok; ++i)
            ok = h[i] == 0.5f * 2.0f * (float)K + 3.0f;
        expect(ok, "gemm_tn 512x384x640, alpha 0.5, beta 1, fp32 D");
        free(h);
        hipFree(A), hipFree(B), hipFree(C), hipFree(D);
    }

    /* 2. gemm_tn_strided_batched: batch b has A = b + 1, B = 1, ragged K:
     *    every element of batch b is (b + 1) * K, exact in fp16. */
    {
        const int64_t batch = 3, M = 256, N = 256, K = 300;
        const uint16_t vals[3] = {F16_ONE, F16_TWO, F16_THREE};
        uint16_t *ha = malloc(batch * M * K * 2);
        for (int64_t b = 0; b < batch; ++b)
            for (int64_t i = 0; i < M * K; ++i)
                ha[b * M * K + i] = vals[b];
        void *A, *D;
        HIP_OK(hipMalloc(&A, batch * M * K * 2));
        HIP_OK(hipMemcpy(A, ha, batch * M * K * 2, hipMemcpyHostToDevice));
        void *B = dev_fill16(N * K, F16_ONE);
        HIP_OK(hipMalloc(&D, batch * M * N * 2));
        int st = gemm_tn_strided_batched(batch, M, N, K, 1.0f, A, M * K, B,
                                         0, 0.0f, NULL, 0, D, M * N,
                                         GEMM_TN_F16, stream);
        uint16_t *hd = malloc(batch * M * N * 2);
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipMemcpy(hd, D, batch * M * N * 2, hipMemcpyDeviceToHost));
        int ok = st == GEMM_TN_OK;
        for (int64_t b = 0; b < batch && ok; ++b)
            for (int64_t i = 0; i < M * N && ok; ++i)
                ok = f16_to_f32(hd[b * M * N + i]) == (float)((b + 1) * K);
        expect(ok, "gemm_tn_strided_batched 3x256x256x300, B broadcast");
        free(ha), free(hd);
        hipFree(A), hipFree(B), hipFree(D);
    }

    /* 3. gemm_tn_ex with A stored K x M (transposed) and padded rows. */
    {
        const int64_t M = 264, N = 200, K = 512, lda = M + 8;
        void *A = dev_fill16(K * lda, F16_ONE), *B = dev_fill16(N * K, F16_TWO);
        void *D = dev_fill32(M * N, -1.0f);
        int st = gemm_tn_ex(1, M, N, K, 0.25f, A, GEMM_TN_ROW_MN, lda, 0, B,
                            GEMM_TN_ROW_K, K, 0, 0.0f, NULL, N, 0, D, N, 0,
                            GEMM_TN_F32, stream);
        float *h = malloc(M * N * 4);
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipMemcpy(h, D, M * N * 4, hipMemcpyDeviceToHost));
        int ok = st == GEMM_TN_OK;
        for (int64_t i = 0; i < M * N && ok; ++i)
            ok = h[i] == 0.25f * 2.0f * (float)K;
        expect(ok, "gemm_tn_ex, A stored along M with padded rows");
        free(h);
        hipFree(A), hipFree(B), hipFree(D);
    }

    /* 4. transpose_f32: x[i][j] = i * N + j, y[j][i] must hold it. */
    {
        const int64_t M = 300, N = 200;
        float *hx = malloc(M * N * 4), *hy = malloc(M * N * 4);
        for (int64_t i = 0; i < M * N; ++i)
            hx[i] = (float)i;
        void *x, *y;
        HIP_OK(hipMalloc(&x, M * N * 4));
        HIP_OK(hipMalloc(&y, M * N * 4));
        HIP_OK(hipMemcpy(x, hx, M * N * 4, hipMemcpyHostToDevice));
        int st = transpose_f32(1, M, N, x, y, stream);
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipMemcpy(hy, y, M * N * 4, hipMemcpyDeviceToHost));
        int ok = st == GEMM_TN_OK;
        for (int64_t i = 0; i < M && ok; ++i)
            for (int64_t j = 0; j < N && ok; ++j)
                ok = hy[j * M + i] == hx[i * N + j];
        expect(ok, "transpose_f32 300x200");
        free(hx), free(hy);
        hipFree(x), hipFree(y);
    }

    /* 5. attention_fwd with Q = 0: every key weighs 1 / Lk, so O is the
     *    mean of V's rows (here V[j][x] = (x mod 4) / 4 in every row) and
     *    lse = log(Lk). */
    {
        const int64_t batch = 2, Lq = 100, Lk = 300, d = 64;
        void *Q = dev_fill16(batch * Lq * d, 0);
        void *Kd = dev_fill16(batch * Lk * d, F16_ONE);
        uint16_t *hv = malloc(batch * Lk * d * 2);
        const uint16_t quarter[4] = {0x0000, 0x3400, 0x3800, 0x3A00};
        for (int64_t i = 0; i < batch * Lk * d; ++i)
            hv[i] = quarter[(i % d) % 4];
        void *V, *O, *lse;
        HIP_OK(hipMalloc(&V, batch * Lk * d * 2));
        HIP_OK(hipMemcpy(V, hv, batch * Lk * d * 2, hipMemcpyHostToDevice));
        HIP_OK(hipMalloc(&O, batch * Lq * d * 4));
        HIP_OK(hipMalloc(&lse, batch * Lq * 4));
        int st = attention_fwd(batch, Lq, Lk, d, 0.125f, Q, Kd, V, O,
                               GEMM_TN_F32, lse, stream);
        float *ho = malloc(batch * Lq * d * 4), *hl = malloc(batch * Lq * 4);
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipMemcpy(ho, O, batch * Lq * d * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(hl, lse, batch * Lq * 4, hipMemcpyDeviceToHost));
        int ok = st == GEMM_TN_OK;
        for (int64_t i = 0; i < batch * Lq * d && ok; ++i)
            ok = fabsf(ho[i] - 0.25f * (float)((i % d) % 4)) <= 1e-6f;
        for (int64_t i = 0; i < batch * Lq && ok; ++i)
            ok = fabsf(hl[i] - logf((float)Lk)) <= 1e-5f;
        expect(ok, "attention_fwd, Q = 0: O = mean of V, lse = log Lk");
        free(hv), free(ho), free(hl);
        hipFree(Q), hipFree(Kd), hipFree(V), hipFree(O), hipFree(lse);
    }

    /* 6. gemm_tn_f16acc: A = B = 1, K = 4096: the fp16 accumulator steps
     *    by 16, every partial sum is an fp16 value, D = 4096. */
    {
        const int64_t M = 128, N = 128, K = 4096;
        void *A = dev_fill16(M * K, F16_ONE), *B = dev_fill16(N * K, F16_ONE);
        void *D;
        HIP_OK(hipMalloc(&D, M * N * 2));
        int st = gemm_tn_f16acc(1, M, N, K, A, 0, B, 0, D, 0, stream);
        uint16_t *hd = malloc(M * N * 2);
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipMemcpy(hd, D, M * N * 2, hipMemcpyDeviceToHost));
        int ok = st == GEMM_TN_OK;
        for (int64_t i = 0; i < M * N && ok; ++i)
            ok = f16_to_f32(hd[i]) == 4096.0f;
        expect(ok, "gemm_tn_f16acc 128x128x4096, ones");
        free(hd);
        hipFree(A), hipFree(B), hipFree(D);
    }

    /* 7. errors come back as status codes, with nothing enqueued */
    {
        int st = gemm_tn(-1, 4, 4, 1.0f, NULL, NULL, 0.0f, NULL, NULL,
                         GEMM_TN_F32, stream);
        const char *msg = gemm_tn_status_string(st);
        expect(st == GEMM_TN_ERR_INVALID_ARG && msg && strlen(msg) > 0,
               "gemm_tn(M = -1) returns GEMM_TN_ERR_INVALID_ARG");
        st = attention_fwd(1, 4, 4, 32, 1.0f, NULL, NULL, NULL, NULL,
                           GEMM_TN_F32, NULL, stream);
        expect(st != GEMM_TN_OK, "attention_fwd(d = 32) is rejected");
    }

    HIP_OK(hipStreamDestroy(stream));
    printf("%s\n", failures ? "c abi demo FAILED" : "c abi demo ok");
    return failures ? 1 : 0;
}
