// fp32 matrix transpose y = x^T for gfx950 (declared in include/
// transpose_f32.h).  One workgroup of 256 threads moves a 64 x 64 tile
// (tiles ordered per XCD down the columns of x, see the kernel):
//
//  * read: 16 consecutive lanes cover one 256-byte row segment of x with
//    16-byte loads (4 rows per wave instruction), as the pages' row2col
//    kernels keep the contiguous side coalesced;
//  * LDS: element (i, j) of the tile is stored at row i, column j ^ i -- the
//    XOR swizzle of page "Mat Transpose CuTe 版代码学习" (version 3: the
//    physical column c ^ r replaces padding).  With 64 banks of 4 bytes and
//    64-float rows, both the row-wise writes and the column-wise reads of a
//    wave hit 64 distinct banks;
//  * write: lanes gather 4 consecutive i of one column j and store them as
//    one 16-byte chunk of row j of y, 16 lanes per 256-byte segment,
//    non-temporally (y is written once).
//
// Edge tiles: rows past M, columns past N (and, transposed, their images)
// get out-of-range buffer offsets: loads read zero, stores are dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lds_layout.hpp"
#include "transpose_f32.h"

namespace {

using gtn::transpose_word;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 64;                 // tile edge
constexpr int kThreads = 256;
constexpr uint32_t kOob = 0x80000000u;  // beyond every record count below
constexpr int kNt = 2;                  // non-temporal store policy

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes)
{
    const uint32_t n = bytes <= 0 ? 0u
                     : (bytes >= 0x7FFFFFFF ? 0x7FFFFFFFu : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base),
                                             (short)0, (int)n, 0x00020000);
}

// VEC: 16-byte loads and stores (M, N multiples of 4, 16-byte aligned).
template <bool VEC>
__global__ void __launch_bounds__(kThreads)
transpose_f32_kernel(const float *x, float *y, int64_t M, int64_t N,
                     int tiles_m, int tiles_n)
{
    __shared__ float tile[kT * kT];
    const int t = threadIdx.x;
    // Workgroup id -> tile.  The hardware deals consecutive ids to the 8
    // XCDs in turn; the id is remapped so that each XCD takes a contiguous
    // range of tiles, and tiles are walked down the columns of x (tm
    // fastest).  Consecutive tiles of one XCD then write adjacent 256-byte
    // pieces of the same 64 rows of y, which the memory system merges; with
    // tn fastest those writes land 64 rows apart (measured at 8192^2: 76 us
    // against 102 us).
    const int per_batch = tiles_m * tiles_n;
    const int nwg = (int)gridDim.x, wg = (int)blockIdx.x;
    const int xq = nwg >> 3, xr = nwg & 7, xcd = wg & 7;
    const int logical = xcd * xq + (xcd < xr ? xcd : xr) + (wg >> 3);
    const int b = logical / per_batch;
    const int in_b = logical - b * per_batch;
    const int tn = in_b / tiles_m, tm = in_b - tn * tiles_m;
    const int64_t i0 = (int64_t)tm * kT, j0 = (int64_t)tn * kT;
    const int64_t rows_left = M - i0, cols_left = N - j0;

    // x: rows i0.., columns j0..; the record count ends at the last row's
    // N-th element, so rows past M read as zero.
    const __amdgpu_buffer_rsrc_t rx =
        rsrc(x + b * M * N + i0 * N + j0, ((rows_left - 1) * N + cols_left) * 4);
    const int c = t % 16;            // 4-float chunk within a tile row
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int r = t / 16 + 16 * k;
        if (VEC) {
            const uint32_t off = 4 * c < cols_left
                                     ? (uint32_t)((r * N + 4 * c) * 4)
                                     : kOob;
            const f32x4 v = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                tile[transpose_word<kT>(r, 4 * c + e)] = v[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t off = 4 * c + e < cols_left
                                         ? (uint32_t)((r * N + 4 * c + e) * 4)
                                         : kOob;
                tile[transpose_word<kT>(r, 4 * c + e)] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 0));
            }
        }
    }
    __syncthreads();

    // y: rows j0.. (columns of x), columns i0..
    const __amdgpu_buffer_rsrc_t ry =
        rsrc(y + b * N * M + j0 * M + i0, ((cols_left - 1) * M + rows_left) * 4);
    const int q = t % 16;            // 4-float chunk within a row of y
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int jj = t / 16 + 16 * k;
        // (a plain array: element-wise writes into an uninitialised
        // ext_vector_type value, read back element-wise, were miscompiled
        // into one LDS read per four elements)
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ii = 4 * q + e;
            v[e] = tile[transpose_word<kT>(ii, jj)];
        }
        if (VEC) {
            const uint32_t off = 4 * q < rows_left
                                     ? (uint32_t)((jj * M + 4 * q) * 4)
                                     : kOob;
            const f32x4 w = {v[0], v[1], v[2], v[3]};
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, w), ry, off, 0, kNt);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t off = 4 * q + e < rows_left
                                         ? (uint32_t)((jj * M + 4 * q + e) * 4)
                                         : kOob;
                __builtin_amdgcn_raw_buffer_store_b32(
                    __builtin_bit_cast(uint32_t, v[e]), ry, off, 0, kNt);
            }
        }
    }
}

bool overlap(const void *a, const void *b, int64_t bytes)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + (uintptr_t)bytes && y < x + (uintptr_t)bytes;
}

}  // namespace

extern "C" int transpose_f32(int64_t batch, int64_t M, int64_t N,
                             const void *x, void *y, void *stream)
{
    if (batch < 0 || M < 0 || N < 0)
        return GEMM_TN_ERR_INVALID_ARG;
    int64_t mn, total, bytes;
    if (__builtin_mul_overflow(M, N, &mn) ||
        __builtin_mul_overflow(mn, batch, &total) ||
        __builtin_mul_overflow(total, (int64_t)4, &bytes))
        return GEMM_TN_ERR_INVALID_ARG;
    if (total == 0)
        return GEMM_TN_OK;
    if (x == nullptr || y == nullptr || overlap(x, y, bytes))
        return GEMM_TN_ERR_INVALID_ARG;
    const int64_t kMax = int64_t(1) << 23;
    if (M > kMax || N > kMax)
        return GEMM_TN_ERR_UNSUPPORTED;
    const int64_t tiles_m = (M + kT - 1) / kT, tiles_n = (N + kT - 1) / kT;
    const int64_t grid = tiles_m * tiles_n * batch;
    if (grid > 0x7FFFFFFF)
        return GEMM_TN_ERR_UNSUPPORTED;
    const bool vec = ((uintptr_t)x % 16) == 0 && ((uintptr_t)y % 16) == 0 &&
                     M % 4 == 0 && N % 4 == 0;
    void *fn = vec ? (void *)&transpose_f32_kernel<true>
                   : (void *)&transpose_f32_kernel<false>;
    int tm = (int)tiles_m, tn = (int)tiles_n;
    const float *xf = (const float *)x;
    float *yf = (float *)y;
    void *args[] = {&xf, &yf, &M, &N, &tm, &tn};
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid),
                                         dim3(kThreads), args, 0,
                                         (hipStream_t)stream);
    return e == hipSuccess ? GEMM_TN_OK : GEMM_TN_ERR_LAUNCH;
}
