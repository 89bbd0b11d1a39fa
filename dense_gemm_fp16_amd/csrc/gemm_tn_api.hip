// extern "C" entry points of the fp16 TN GEMM library (declared in
// include/gemm_tn.h): argument checks, configuration choice, the split-K
// workspace, and the launches.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <utility>

#include "gemm_tn.h"
#include "gemm_tn_launch.hpp"
#include "gemm_tn_plan.hpp"

namespace gtn {

hipError_t launch_splitk_reduce(const GemmArgs &a, bool out_f32, bool vec_out,
                                hipStream_t s)
{
    const int64_t work = (int64_t)a.batch * a.M * ((a.N + 3) / 4);
    const unsigned grid = (unsigned)((work + 255) / 256);
    void *fn;
    if (out_f32)
        fn = vec_out ? (void *)&splitk_reduce_kernel<float, true>
                     : (void *)&splitk_reduce_kernel<float, false>;
    else
        fn = vec_out ? (void *)&splitk_reduce_kernel<_Float16, true>
                     : (void *)&splitk_reduce_kernel<_Float16, false>;
    GemmArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, s);
}

namespace {

// Split-K workspace, one per (device, stream): calls on one stream run in
// order, so reusing its buffer is safe; distinct streams never share one.
// The caller holds `lock` (taken here) until its kernels are enqueued: a
// call from another thread that grows the buffer waits for the stream
// before freeing it, which covers only kernels already enqueued.
struct Workspace {
    void *ptr = nullptr;
    int64_t bytes = 0;
};
std::mutex g_ws_lock;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

int get_workspace(hipStream_t s, int64_t bytes, float **out,
                  std::unique_lock<std::mutex> &lock)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return GEMM_TN_ERR_LAUNCH;
    lock = std::unique_lock<std::mutex>(g_ws_lock);
    Workspace &w = g_ws[std::make_pair(dev, s)];
    if (w.bytes < bytes) {
        if (w.ptr) {
            // earlier work on this stream may still read the old buffer
            if (hipStreamSynchronize(s) != hipSuccess)
                return GEMM_TN_ERR_WORKSPACE;
            (void)hipFree(w.ptr);
            w.ptr = nullptr;
            w.bytes = 0;
        }
        int64_t want = bytes + bytes / 4;   // headroom for growth
        if (hipMalloc(&w.ptr, (size_t)want) != hipSuccess) {
            w.ptr = nullptr;
            (void)hipGetLastError();
            return GEMM_TN_ERR_WORKSPACE;
        }
        w.bytes = want;
    }
    *out = (float *)w.ptr;
    return GEMM_TN_OK;
}

// Scratch of gemm_tn_ex_noalloc: the split-K partials of callers that
// cannot allocate live in this fixed array instead of the per-stream
// workspace.  Each GPU the library runs on holds its own copy for the life
// of the process.  In host code `scratch` names a host-side stand-in, not
// device memory: its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device and kept in g_scratch_dev.
static __device__ __align__(256) char scratch[GEMM_TN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_lock;
void *g_scratch_dev[kMaxDevices];

// The current device's address of `scratch`, for a problem needing `bytes`
// of it.  No allocation: the array exists once the library's code object
// is loaded on the device.
int get_static_scratch(int64_t bytes, float **out)
{
    if (bytes > GEMM_TN_NOALLOC_SCRATCH_BYTES)
        return GEMM_TN_ERR_SCRATCH;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return GEMM_TN_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_lock);
    if (g_scratch_dev[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess ||
            ptr == nullptr) {
            (void)hipGetLastError();
            return GEMM_TN_ERR_LAUNCH;
        }
        g_scratch_dev[dev] = ptr;
    }
    *out = (float *)g_scratch_dev[dev];
    return GEMM_TN_OK;
}

bool aligned(const void *p, uintptr_t a)
{
    return ((uintptr_t)p % a) == 0;
}

// vec_in: 16-byte loads of A and B are possible; vec_out: 16-byte stores
// of D (and loads of C) are.
bool vector_inputs(bool aligned16, int64_t M, int64_t N, int64_t K,
                   const Lds &ld, int64_t sA, int64_t sB)
{
    const int64_t a_len = ld.a_mn ? M : K, b_len = ld.b_mn ? N : K;
    return aligned16 && a_len % 8 == 0 && b_len % 8 == 0 && ld.a % 8 == 0 &&
           ld.b % 8 == 0 && sA % 8 == 0 && sB % 8 == 0;
}

bool vector_outputs(bool d_aligned16, bool c_aligned16, int64_t N,
                    const Lds &ld, int64_t sC, int64_t sD, float beta, int es)
{
    return d_aligned16 && (N * es) % 16 == 0 && (ld.d * es) % 16 == 0 &&
           (sD * es) % 16 == 0 &&
           (beta == 0.0f ||
            (c_aligned16 && (ld.c * es) % 16 == 0 && (sC * es) % 16 == 0));
}

// The tile kernel (and, for split-K, the reduction) over the problem in a:
// `splits` slices of a.k_split, `grid` workgroups.
int launch_rows(const GemmArgs &a, const Plan &p, int splits, unsigned grid,
                bool out_f32, hipStream_t s)
{
    const bool split = splits > 1;
    if (split && a.ws == nullptr)
        return GEMM_TN_ERR_WORKSPACE;    // partials need somewhere to go
    hipError_t e;
    switch (p.tile) {
    case TILE_256:
        e = p.four_wave
                ? launch_tile256_w4(a, out_f32, split, p.vec_out, grid, s)
                : launch_tile256(a, p.loader, p.layout, out_f32, split,
                                 p.vec_out, grid, s);
        break;
    case TILE_128:
        e = launch_tile128(a, p.loader, p.layout, out_f32, split, p.vec_out,
                           grid, s);
        break;
    default:
        e = launch_tile64(a, p.loader, p.layout, out_f32, split, p.vec_out,
                          grid, s);
        break;
    }
    if (e == hipSuccess && split)
        e = launch_splitk_reduce(a, out_f32, p.vec_out, s);
    return e == hipSuccess ? GEMM_TN_OK : GEMM_TN_ERR_LAUNCH;
}

bool layout_ok(int layout)
{
    return layout == GEMM_TN_ROW_K || layout == GEMM_TN_ROW_MN;
}

int run(int64_t batch, int64_t M, int64_t N, int64_t K, float alpha,
        const void *A, int layout_a, int64_t lda, int64_t sA, const void *B,
        int layout_b, int64_t ldb, int64_t sB, float beta, const void *C,
        int64_t ldc, int64_t sC, void *D, int64_t ldd, int64_t sD,
        int d_dtype, void *stream, bool noalloc)
{
    if (!layout_ok(layout_a) || !layout_ok(layout_b))
        return GEMM_TN_ERR_INVALID_ARG;
    const Lds ld{lda, ldb, ldc, ldd, layout_a == GEMM_TN_ROW_MN,
                 layout_b == GEMM_TN_ROW_MN};
    int st = check_sizes(batch, M, N, K, ld, sA, sB, sC, sD, d_dtype);
    if (st != GEMM_TN_OK)
        return st;
    if (batch == 0 || M == 0 || N == 0)
        return GEMM_TN_OK;
    st = check_pointers(M, N, K, A, B, beta, C, D);
    if (st != GEMM_TN_OK)
        return st;

    const bool out_f32 = d_dtype == GEMM_TN_F32;
    const int es = out_f32 ? 4 : 2;
    const bool vec_in = vector_inputs(aligned(A, 16) && aligned(B, 16), M, N,
                                      K, ld, sA, sB);
    const bool vec_out = vector_outputs(aligned(D, 16), aligned(C, 16), N, ld,
                                        sC, sD, beta, es);
    const Plan p = make_plan(batch, M, N, K, ld, sA, sB, sC, sD, d_dtype,
                             vec_in, vec_out, getenv("GEMM_TN_FORCE"));
    if (p.status != GEMM_TN_OK)
        return p.status;

    hipStream_t s = (hipStream_t)stream;
    GemmArgs a;
    a.A = (const _Float16 *)A;
    a.B = (const _Float16 *)B;
    a.C = C;
    a.D = D;
    a.ws = nullptr;
    a.M = M;
    a.N = N;
    a.K = K;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.ldd = ldd;
    a.sA = sA;
    a.sB = sB;
    a.sC = sC;
    a.sD = sD;
    a.ws_ld = p.ws_ld;
    a.alpha = alpha;
    a.beta = beta;
    a.tiles_m = p.tiles_m;
    a.tiles_n = p.tiles_n;
    a.batch = (int)batch;
    a.splits = p.splits;
    a.k_split = (int)p.k_split;
    a.group_m = p.group_m;
    if (p.onek) {
        const hipError_t e = launch_onek(a, out_f32, (unsigned)p.grid, s);
        return e == hipSuccess ? GEMM_TN_OK : GEMM_TN_ERR_LAUNCH;
    }
    std::unique_lock<std::mutex> ws_lock;   // held until the launches
    if (p.splits > 1 || p.tail_rows > 0) {
        st = noalloc ? get_static_scratch(p.ws_bytes, &a.ws)
                     : get_workspace(s, p.ws_bytes, &a.ws, ws_lock);
        if (st != GEMM_TN_OK)
            return st;
    }
    if (p.tail_rows == 0)
        return launch_rows(a, p, p.splits, (unsigned)p.grid, out_f32, s);

    // Tail split: rows [0, m_tail) as whole tiles, rows [m_tail, M) as a
    // split-K problem of their own (operand A, C and D start at row m_tail
    // of every batch entry; the batch strides stay).
    const int64_t m_tail = (int64_t)(p.tiles_m - p.tail_rows) * p.bm;
    GemmArgs top = a;
    top.M = m_tail;
    top.tiles_m = p.tiles_m - p.tail_rows;
    top.splits = 1;
    top.k_split = (int)(cdiv(K, kBK) * kBK);
    st = launch_rows(top, p, 1, (unsigned)p.grid, out_f32, s);
    if (st != GEMM_TN_OK)
        return st;
    GemmArgs bot = a;
    bot.A = ld.a_mn ? a.A + m_tail : a.A + m_tail * lda;
    bot.C = C ? (const char *)C + m_tail * ldc * es : nullptr;
    bot.D = (char *)D + m_tail * ldd * es;
    bot.M = M - m_tail;
    bot.tiles_m = p.tail_rows;
    bot.splits = p.tail_splits;
    bot.k_split = (int)p.tail_k_split;
    return launch_rows(bot, p, p.tail_splits, (unsigned)p.tail_grid, out_f32,
                       s);
}

}  // namespace
}  // namespace gtn

extern "C" {

int gemm_tn(int64_t M, int64_t N, int64_t K, float alpha, const void *A,
            const void *B, float beta, const void *C, void *D, int d_dtype,
            void *stream)
{
    return gtn::run(1, M, N, K, alpha, A, GEMM_TN_ROW_K, K, 0, B,
                    GEMM_TN_ROW_K, K, 0, beta, C, N, 0, D, N, 0, d_dtype,
                    stream, false);
}

int gemm_tn_strided_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                            float alpha, const void *A, int64_t strideA,
                            const void *B, int64_t strideB, float beta,
                            const void *C, int64_t strideC, void *D,
                            int64_t strideD, int d_dtype, void *stream)
{
    return gtn::run(batch, M, N, K, alpha, A, GEMM_TN_ROW_K, K, strideA, B,
                    GEMM_TN_ROW_K, K, strideB, beta, C, N, strideC, D, N,
                    strideD, d_dtype, stream, false);
}

int gemm_tn_ex(int64_t batch, int64_t M, int64_t N, int64_t K, float alpha,
               const void *A, int layout_a, int64_t lda, int64_t strideA,
               const void *B, int layout_b, int64_t ldb, int64_t strideB,
               float beta, const void *C, int64_t ldc, int64_t strideC,
               void *D, int64_t ldd, int64_t strideD, int d_dtype,
               void *stream)
{
    return gtn::run(batch, M, N, K, alpha, A, layout_a, lda, strideA, B,
                    layout_b, ldb, strideB, beta, C, ldc, strideC, D, ldd,
                    strideD, d_dtype, stream, false);
}

int gemm_tn_ex_noalloc(int64_t batch, int64_t M, int64_t N, int64_t K,
                       float alpha, const void *A, int layout_a, int64_t lda,
                       int64_t strideA, const void *B, int layout_b,
                       int64_t ldb, int64_t strideB, float beta,
                       const void *C, int64_t ldc, int64_t strideC, void *D,
                       int64_t ldd, int64_t strideD, int d_dtype,
                       void *stream)
{
    return gtn::run(batch, M, N, K, alpha, A, layout_a, lda, strideA, B,
                    layout_b, ldb, strideB, beta, C, ldc, strideC, D, ldd,
                    strideD, d_dtype, stream, true);
}

int gemm_tn_describe(int64_t batch, int64_t M, int64_t N, int64_t K,
                     int layout_a, int64_t lda, int layout_b, int64_t ldb,
                     int64_t ldc, int64_t ldd, int64_t strideA,
                     int64_t strideB, int64_t strideC, int64_t strideD,
                     float beta, int d_dtype, int aligned16, char *buf,
                     int64_t buflen)
{
    if (!gtn::layout_ok(layout_a) || !gtn::layout_ok(layout_b)) {
        gtn::Plan bad;
        bad.status = GEMM_TN_ERR_INVALID_ARG;
        return gtn::describe_plan(bad, buf, buflen);
    }
    const gtn::Lds ld{lda, ldb, ldc, ldd, layout_a == GEMM_TN_ROW_MN,
                      layout_b == GEMM_TN_ROW_MN};
    const int es = d_dtype == GEMM_TN_F32 ? 4 : 2;
    const bool vec_in = gtn::vector_inputs(aligned16 != 0, M, N, K, ld,
                                           strideA, strideB);
    const bool vec_out = gtn::vector_outputs(aligned16 != 0, aligned16 != 0,
                                             N, ld, strideC, strideD, beta, es);
    const gtn::Plan p = gtn::make_plan(batch, M, N, K, ld, strideA, strideB,
                                       strideC, strideD, d_dtype, vec_in,
                                       vec_out, getenv("GEMM_TN_FORCE"));
    return gtn::describe_plan(p, buf, buflen);
}

const char *gemm_tn_status_string(int status)
{
    switch (status) {
    case GEMM_TN_OK:
        return "ok";
    case GEMM_TN_ERR_INVALID_ARG:
        return "invalid argument";
    case GEMM_TN_ERR_UNSUPPORTED:
        return "unsupported size";
    case GEMM_TN_ERR_LAUNCH:
        return "kernel launch failed";
    case GEMM_TN_ERR_WORKSPACE:
        return "split-K workspace allocation failed";
    case GEMM_TN_ERR_SCRATCH:
        return "problem needs more split-K scratch than "
               "gemm_tn_ex_noalloc's static maximum";
    default:
        return "unknown status";
    }
}

int gemm_tn_version(void) { return (1 << 16) | 2; }

}  // extern "C"
