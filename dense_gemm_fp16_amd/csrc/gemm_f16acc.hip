// fp16-accumulating TN GEMM D = A * B^T for gfx950 (declared in
// include/gemm_f16acc.h).
//
// Page "cute(8) smem_gemm" (yuyanqi.com, kernel listing and section 2.3)
// builds its GEMM from an MMA atom with fp16 A, B, C and D, 16 deep in K:
// the accumulator is an fp16 value after every 16-deep step.  gfx950's
// MFMAs accumulate in fp32, so this kernel keeps that rule explicitly:
// v_mfma_f32_16x16x16_f16 adds one 16-deep step to the accumulator (whose
// values are fp16 numbers held in fp32), and the result is rounded back to
// fp16 (round to nearest even) before the next step.  The steps run in
// order of K, each over 16 consecutive k.
//
//  * Work: one workgroup of 4 waves (2 x 2, as the page's 2 x 2 MMA
//    arrangement) per 128 x 128 tile of D; each wave owns 64 x 64, a 4 x 4
//    grid of 16 x 16 accumulator blocks.
//  * K tiles of 32 (the page's kTileK) in two LDS stages; 16-byte chunk c of
//    row r stored at chunk c ^ ((r / 4) % 4), which keeps the 8-byte
//    fragment reads of a half wave (16 rows, one chunk) on distinct banks.
//  * Fragments: lane l holds row l % 16 and k = 4 (l / 16) .. + 3 of a
//    16-deep step, one ds_read_b64.  Operands are issued as (B, A), so a
//    lane's accumulators are 4 consecutive n of one m.
//  * Loads: 16-byte direct-to-LDS buffer loads when rows allow them (K a
//    multiple of 8, 16-byte aligned operands); otherwise each thread
//    gathers 8 halves with 2-byte loads and writes them to LDS.  Rows past
//    M or N and k past K read as zero (the extra terms add nothing).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_f16acc.h"
#include "gemm_tn_kernels.hpp"

namespace gtn {
namespace {

constexpr int kT = 128;         // tile edge
constexpr int kBKa = 32;        // K per LDS stage
constexpr int kThr = 256;
// Offsets within a tile stay below 2^29 bytes with these limits.
constexpr int64_t kAccMaxK = int64_t(1) << 21;
constexpr int64_t kAccMaxN = int64_t(1) << 20;

typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct AccArgs {
    const _Float16 *A, *B;
    _Float16 *D;
    int64_t M, N, K;
    int64_t sA, sB, sD;
    int tiles_m, tiles_n, batch;
};

template <bool DIRECT, bool VEC_OUT>
__global__ void __launch_bounds__(kThr) gemm_f16acc_kernel(AccArgs p)
{
    constexpr int TILE = kT * kBKa;                 // halves per operand tile
    __shared__ __attribute__((aligned(1024))) _Float16 lds[2 * 2 * TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // workgroup id -> (batch, tile); XCD x receives a contiguous range
    const int total = p.tiles_m * p.tiles_n * p.batch;
    const int wg = blockIdx.x;
    const int qq = total >> 3, rr = total & 7, x8 = wg & 7;
    const int logical = x8 * qq + (x8 < rr ? x8 : rr) + (wg >> 3);
    const int per_b = p.tiles_m * p.tiles_n;
    const int b = logical / per_b;
    const int t = logical - b * per_b;
    const int tm = t / p.tiles_n, tn = t - tm * p.tiles_n;
    const int64_t m0 = (int64_t)tm * kT, n0 = (int64_t)tn * kT;
    const int64_t M = p.M, N = p.N, K = p.K;

    const _Float16 *Ab = p.A + b * p.sA + m0 * K;
    const _Float16 *Bb = p.B + b * p.sB + n0 * K;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(Ab, ((M - m0 - 1) * K + K) * 2);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bb, ((N - n0 - 1) * K + K) * 2);

    // ---- global -> LDS -----------------------------------------------------
    // DIRECT: one wave instruction fills 16 rows of 64 bytes; lane l lands in
    // physical chunk l % 4 of row l / 4 of that group.
    auto issue = [&](int stage, int64_t k0) {
        GTN_LDS _Float16 *base = (GTN_LDS _Float16 *)lds + stage * 2 * TILE;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int grp = wave + 4 * h;           // 16-row group, 0..7
            const int row = grp * 16 + (lane >> 2);
            const int kc = swizzle_chunk<kBKa>(row, lane & 3) * 8;
            const bool in = k0 + kc < K;
            const uint32_t off_a = in ? (uint32_t)((row * K + k0 + kc) * 2)
                                      : kOutOfRange;
            const uint32_t off_b = off_a;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rA, (GTN_LDS void *)(base + grp * 16 * kBKa), 16, off_a, 0,
                0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rB, (GTN_LDS void *)(base + TILE + grp * 16 * kBKa), 16,
                off_b, 0, 0, 0);
        }
    };
    // Element loader: thread t owns chunk slots t and t + 256 of each
    // operand's 128 x 4 chunk grid.
    u32x4 regs[4];
    auto fetch = [&](int64_t k0) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const bool isA = x < 2;
            const int slot = tid + 256 * (x & 1);
            const int row = slot >> 2, ch = slot & 3;
            const __amdgpu_buffer_rsrc_t r = isA ? rA : rB;
            uint16_t e[8];
#pragma unroll
            for (int y = 0; y < 8; ++y) {
                const int64_t kk = k0 + ch * 8 + y;
                const uint32_t off = kk < K ? (uint32_t)((row * K + kk) * 2)
                                            : kOutOfRange;
                e[y] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
            }
            regs[x] = u32x4{e[0] | ((uint32_t)e[1] << 16),
                            e[2] | ((uint32_t)e[3] << 16),
                            e[4] | ((uint32_t)e[5] << 16),
                            e[6] | ((uint32_t)e[7] << 16)};
        }
    };
    auto store = [&](int stage) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const bool isA = x < 2;
            const int slot = tid + 256 * (x & 1);
            const int row = slot >> 2, ch = slot & 3;
            *(u32x4 *)(lds + stage * 2 * TILE + (isA ? 0 : TILE) + row * kBKa +
                       swizzle_chunk<kBKa>(row, ch) * 8) = regs[x];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One 16-deep step s of the stage: fragments, 16 MFMAs, fp16 rounding.
    const int fr = lane & 15, fg = lane >> 4;
    auto step = [&](int stage, int s) {
        const _Float16 *sA = lds + stage * 2 * TILE;
        const _Float16 *sB = sA + TILE;
        half4v af[4], bf[4];                        // 4 k per lane
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = *(const half4v *)(sA + tn_frag4_offset<kBKa>(
                                               wm * 64 + i * 16, lane, s));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bf[j] = *(const half4v *)(sB + tn_frag4_offset<kBKa>(
                                               wn * 64 + j * 16, lane, s));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4 a = __builtin_amdgcn_mfma_f32_16x16x16f16(bf[j], af[i],
                                                               acc[i][j], 0,
                                                               0, 0);
                // rn16 of the four sums, two per packed conversion
                const half2v lo = __builtin_convertvector(f32x2{a[0], a[1]},
                                                          half2v);
                const half2v hi = __builtin_convertvector(f32x2{a[2], a[3]},
                                                          half2v);
                acc[i][j] = f32x4{(float)lo[0], (float)lo[1], (float)hi[0],
                                  (float)hi[1]};
            }
    };

    const int ktiles = (int)((K + kBKa - 1) / kBKa);
    if (DIRECT) {
        if (ktiles > 0)
            issue(0, 0);
        for (int kt = 0; kt < ktiles; ++kt) {
            const int cur = kt & 1;
            wait_vmcnt<0>();
            wait_lgkmcnt<0>();
            block_sync();
            if (kt + 1 < ktiles)
                issue(cur ^ 1, (int64_t)(kt + 1) * kBKa);
            step(cur, 0);
            step(cur, 1);
        }
    } else {
        if (ktiles > 0) {
            fetch(0);
            store(0);
        }
        for (int kt = 0; kt < ktiles; ++kt) {
            const int cur = kt & 1;
            __syncthreads();
            const bool more = kt + 1 < ktiles;
            if (more)
                fetch((int64_t)(kt + 1) * kBKa);
            step(cur, 0);
            step(cur, 1);
            if (more)
                store(cur ^ 1);
        }
    }

    // ---- epilogue: the fp16 accumulators, 4 consecutive n per lane --------
    const __amdgpu_buffer_rsrc_t rD =
        make_rsrc(p.D + b * p.sD + m0 * N, ((M - m0 - 1) * N + N) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = wm * 64 + i * 16 + fr;
            const int n = wn * 64 + j * 16 + 4 * fg;
            const bool row_in = m0 + m < M;
            if (VEC_OUT) {
                const half4v h = {(_Float16)acc[i][j][0], (_Float16)acc[i][j][1],
                                  (_Float16)acc[i][j][2], (_Float16)acc[i][j][3]};
                const uint32_t off = row_in && n0 + n < N
                                         ? (uint32_t)((m * N + n0 + n) * 2)
                                         : kOutOfRange;
                __builtin_amdgcn_raw_buffer_store_b64(
                    __builtin_bit_cast(u32x2, h), rD, off, 0, 0);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t off =
                        row_in && n0 + n + e < N
                            ? (uint32_t)((m * N + n0 + n + e) * 2)
                            : kOutOfRange;
                    const _Float16 h = (_Float16)acc[i][j][e];
                    __builtin_amdgcn_raw_buffer_store_b16(
                        __builtin_bit_cast(uint16_t, h), rD, off, 0, 0);
                }
            }
        }
}

bool overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na > 0 && nb > 0 && x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

}  // namespace
}  // namespace gtn

extern "C" int gemm_tn_f16acc(int64_t batch, int64_t M, int64_t N, int64_t K,
                              const void *A, int64_t strideA, const void *B,
                              int64_t strideB, void *D, int64_t strideD,
                              void *stream)
{
    using namespace gtn;
    if (batch < 0 || M < 0 || N < 0 || K < 0)
        return GEMM_TN_ERR_INVALID_ARG;
    if (batch == 0 || M == 0 || N == 0)
        return GEMM_TN_OK;
    if (D == nullptr || (K > 0 && (A == nullptr || B == nullptr)))
        return GEMM_TN_ERR_INVALID_ARG;
    int64_t mk, nk, mn;
    if (__builtin_mul_overflow(M, K, &mk) || __builtin_mul_overflow(N, K, &nk) ||
        __builtin_mul_overflow(M, N, &mn))
        return GEMM_TN_ERR_INVALID_ARG;
    // batch strides: 0 broadcasts A or B; D's batches must not overlap
    if (strideA < 0 || strideB < 0 || strideD < 0)
        return GEMM_TN_ERR_INVALID_ARG;
    if (batch > 1 && ((strideA != 0 && strideA < mk) ||
                      (strideB != 0 && strideB < nk) || strideD < mn))
        return GEMM_TN_ERR_INVALID_ARG;
    if (K > kAccMaxK || N > kAccMaxN)
        return GEMM_TN_ERR_UNSUPPORTED;
    int64_t ea, eb, ed;
    if (__builtin_mul_overflow(batch - 1, strideA, &ea) ||
        __builtin_mul_overflow(batch - 1, strideB, &eb) ||
        __builtin_mul_overflow(batch - 1, strideD, &ed))
        return GEMM_TN_ERR_INVALID_ARG;
    int64_t bytes_a, bytes_b, bytes_d;
    if (__builtin_add_overflow(ea, mk, &bytes_a) ||
        __builtin_add_overflow(eb, nk, &bytes_b) ||
        __builtin_add_overflow(ed, mn, &bytes_d) ||
        __builtin_mul_overflow(bytes_a, (int64_t)2, &bytes_a) ||
        __builtin_mul_overflow(bytes_b, (int64_t)2, &bytes_b) ||
        __builtin_mul_overflow(bytes_d, (int64_t)2, &bytes_d))
        return GEMM_TN_ERR_INVALID_ARG;
    if (overlap(D, bytes_d, A, bytes_a) || overlap(D, bytes_d, B, bytes_b))
        return GEMM_TN_ERR_INVALID_ARG;
    const int64_t tiles_m = (M + kT - 1) / kT, tiles_n = (N + kT - 1) / kT;
    if (tiles_m * tiles_n > 0x7FFFFFFF / batch)
        return GEMM_TN_ERR_UNSUPPORTED;

    AccArgs a;
    a.A = (const _Float16 *)A;
    a.B = (const _Float16 *)B;
    a.D = (_Float16 *)D;
    a.M = M;
    a.N = N;
    a.K = K;
    a.sA = strideA;
    a.sB = strideB;
    a.sD = strideD;
    a.tiles_m = (int)tiles_m;
    a.tiles_n = (int)tiles_n;
    a.batch = (int)batch;
    const bool direct = K % 8 == 0 && (uintptr_t)A % 16 == 0 &&
                        (uintptr_t)B % 16 == 0 && strideA % 8 == 0 &&
                        strideB % 8 == 0;
    const bool vec_out = N % 4 == 0 && (uintptr_t)D % 8 == 0 &&
                         strideD % 4 == 0;
    void *fn = direct ? (vec_out ? (void *)&gemm_f16acc_kernel<true, true>
                                 : (void *)&gemm_f16acc_kernel<true, false>)
                      : (vec_out ? (void *)&gemm_f16acc_kernel<false, true>
                                 : (void *)&gemm_f16acc_kernel<false, false>);
    void *args[] = {&a};
    const hipError_t e = hipLaunchKernel(
        fn, dim3((unsigned)(tiles_m * tiles_n * batch)), dim3(kThr), args, 0,
        (hipStream_t)stream);
    return e == hipSuccess ? GEMM_TN_OK : GEMM_TN_ERR_LAUNCH;
}
