// HIP kernels of the fp16 TN GEMM  D = alpha * A * B^T + beta * C  for
// gfx950 (MI355X, CDNA4).
//
// One workgroup owns one BM x BN tile of D for one batch entry (and, with
// split-K, one slice of K), as the CTA does in page "cute(8) smem_gemm"
// (yuyanqi.com, kernel listing and section 6: a CTA walks the K dimension
// of its A rows and B rows in kTileK-wide steps, and an inner loop walks the
// MMA k-steps of each step).  The CDNA4 design of each stage:
//
//  * global -> LDS: 16-byte loads through buffer resources.  A row of a
//    BK = 64 tile is 128 bytes = 8 chunks of 16 bytes, so 8 consecutive
//    lanes read one full 128-byte line (coalesced).  Rows past M / N and
//    chunks past K get an out-of-range buffer offset, which the hardware
//    turns into zeros: that is the edge predication (page "Mat Transpose
//    CuTe 版代码学习", chuoer47.github.io, version 1: a per-element coordinate
//    mask decides which accesses happen).
//  * LDS layout: chunk c of row r is stored at chunk c ^ ((r >> SWZ) & 7)
//    of that row: an XOR swizzle of 16-byte groups, which keeps each group
//    contiguous for 128-bit reads while spreading one logical chunk of
//    consecutive rows over distinct banks (page "cute(8) smem_gemm",
//    section 3: Swizzle<B,M,S> XORs the row bits into the group index).
//  * LDS -> registers: v_mfma_f32_32x32x16_f16 takes, in each lane, 8
//    consecutive-k halves of one row of each operand; in TN storage that is
//    one ds_read_b128 per operand per lane, with no shuffle.
//  * MFMA: each wave owns a (BM/WM) x (BN/WN) sub-tile as a grid of 32 x 32
//    fp32 accumulator blocks.  The operands are issued as (B, A), so the
//    accumulator block is D^T: each lane then holds 4 consecutive n of one
//    m per group of 4 registers, which the epilogue stores as one 8- or
//    16-byte vector.
//  * Pipeline: two LDS stages; the loads of k-tile t+1 are issued before
//    the MFMAs of k-tile t, and one barrier per k-tile orders both the
//    read-after-write on stage t and the write-after-read on stage t+1.
//  * Epilogue: alpha * acc (+ beta * C when beta != 0) in fp32, rounded to
//    fp16 or fp32 with round-to-nearest-even, stored through buffer stores
//    whose out-of-range lanes are dropped.
//  * Split-K: slices write fp32 partial tiles to a workspace; a second
//    kernel sums them in slice order (deterministic) and applies the
//    epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gtn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define GTN_LDS __attribute__((address_space(3)))

// Buffer offsets at or above this value are out of range for every
// resource made by make_rsrc (whose record count is at most 0x7FFFFFFF).
constexpr uint32_t kOutOfRange = 0x80000000u;
// Word 3 of a gfx9 buffer descriptor: 32-bit data format, raw addressing.
constexpr int kRsrcWord3 = 0x00020000;

enum Loader { LOAD_DIRECT = 0, LOAD_VREG = 1, LOAD_ELEM = 2 };

struct GemmArgs {
    const _Float16 *A;
    const _Float16 *B;
    const void *C;
    void *D;
    float *ws;          // split-K partials: [split][batch][M][ws_ld] fp32
    int64_t M, N, K;
    int64_t sA, sB, sC, sD;   // batch strides in elements
    int64_t ws_ld;
    float alpha, beta;
    int tiles_m, tiles_n, batch, splits;
    int k_split;        // K extent of one split-K slice (multiple of BK)
    int group_m;        // tile rows per L2 group in the tile order
};

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base,
                                                   int64_t bytes)
{
    uint32_t n = bytes <= 0 ? 0u
               : (bytes >= 0x7FFFFFFF ? 0x7FFFFFFFu : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base),
                                             (short)0, (int)n, kRsrcWord3);
}

// Workgroup id -> (batch, split, tile_m, tile_n).
//
// The hardware hands consecutive workgroup ids to the 8 XCDs in turn; each
// XCD has its own L2.  The id is first remapped so that each XCD receives a
// contiguous range of logical tiles, then logical tiles are ordered in
// groups of `group_m` tile rows, column by column inside a group, so that a
// contiguous range covers a compact block of D sharing few A and B panels.
struct TileCoord {
    int b, s, tm, tn;
};

__device__ inline TileCoord map_tile(const GemmArgs &p)
{
    const int total = p.tiles_m * p.tiles_n * p.batch * p.splits;
    const int wg = blockIdx.x;
    const int q = total >> 3, r = total & 7, x = wg & 7;
    const int logical = x * q + (x < r ? x : r) + (wg >> 3);
    const int per_bs = p.tiles_m * p.tiles_n;
    const int tile = logical % per_bs;
    const int bs = logical / per_bs;
    TileCoord tc;
    tc.b = bs % p.batch;
    tc.s = bs / p.batch;
    const int per_group = p.group_m * p.tiles_n;
    const int g = tile / per_group;
    const int first_m = g * p.group_m;
    const int rows_in_group =
        (p.tiles_m - first_m) < p.group_m ? (p.tiles_m - first_m) : p.group_m;
    const int in_g = tile - g * per_group;
    tc.tm = first_m + in_g % rows_in_group;
    tc.tn = in_g / rows_in_group;
    return tc;
}

template <int SWZ>
__device__ __host__ constexpr int swizzle_chunk(int row, int chunk)
{
    return chunk ^ ((row >> SWZ) & 7);
}

template <typename OutT>
struct OutTraits;
template <>
struct OutTraits<_Float16> {
    static constexpr int bytes = 2;
};
template <>
struct OutTraits<float> {
    static constexpr int bytes = 4;
};

__device__ inline float load_out_elem(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                      _Float16 *)
{
    uint16_t v = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    return (float)__builtin_bit_cast(_Float16, v);
}
__device__ inline float load_out_elem(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                      float *)
{
    uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    return __builtin_bit_cast(float, v);
}
__device__ inline void store_out_elem(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                      float v, _Float16 *)
{
    _Float16 h = (_Float16)v;
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, h), r,
                                          off, 0, 0);
}
__device__ inline void store_out_elem(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                      float v, float *)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r,
                                          off, 0, 0);
}
__device__ inline f32x4 load_out_vec4(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                      _Float16 *)
{
    u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    half4 h = __builtin_bit_cast(half4, v);
    return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}
__device__ inline f32x4 load_out_vec4(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                      float *)
{
    u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return __builtin_bit_cast(f32x4, v);
}
__device__ inline void store_out_vec4(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                      f32x4 v, _Float16 *)
{
    half4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2],
               (_Float16)v[3]};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), r,
                                          off, 0, 0);
}
__device__ inline void store_out_vec4(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                      f32x4 v, float *)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r,
                                           off, 0, 0);
}

// ---------------------------------------------------------------------------
// Main kernel.
//   BM x BN x BK : workgroup tile; WM x WN waves; SWZ : swizzle row shift;
//   LOADER : LOAD_DIRECT (16-byte buffer loads straight into LDS),
//            LOAD_VREG (16-byte loads into VGPRs, then ds_write_b128),
//            LOAD_ELEM (2-byte loads, any K and any alignment);
//   OutT : _Float16 or float; SPLIT : write fp32 partials to the workspace;
//   VEC_OUT : D / C rows allow 4-element vector access (N % 4 == 0 and the
//             base pointers are aligned for it).
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int WM, int WN, int SWZ, int LOADER,
          typename OutT, bool SPLIT, bool VEC_OUT, int MIN_WAVES>
__global__ void __attribute__((amdgpu_flat_work_group_size(WM * WN * 64,
                                                           WM * WN * 64),
                               amdgpu_waves_per_eu(MIN_WAVES, 8)))
gemm_tn_kernel(GemmArgs p)
{
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MI = WTM / 32, NI = WTN / 32;
    constexpr int KSTEPS = BK / 16;
    constexpr int CHUNKS = BK / 8;            // 16-byte chunks per tile row
    constexpr int ROWS_PER_WAVE_LOAD = 64 / CHUNKS;
    constexpr int STAGE_HALVES = (BM + BN) * BK;
    static_assert(BK == 64, "the swizzle and loaders assume 128-byte rows");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile of 32x32 blocks");
    static_assert(BM % (ROWS_PER_WAVE_LOAD * WM * WN) == 0 &&
                      BN % (ROWS_PER_WAVE_LOAD * WM * WN) == 0,
                  "every wave issues the same number of tile loads");

    __shared__ __attribute__((aligned(1024))) _Float16 lds[2 * STAGE_HALVES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    const TileCoord tc = map_tile(p);
    const int64_t m0 = (int64_t)tc.tm * BM;
    const int64_t n0 = (int64_t)tc.tn * BN;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t k_begin = (int64_t)tc.s * p.k_split;
    const int64_t k_end = SPLIT ? (k_begin + p.k_split < K ? k_begin + p.k_split
                                                           : K)
                                : K;
    const int ktiles = k_end > k_begin ? (int)((k_end - k_begin + BK - 1) / BK)
                                       : 0;

    // Operand resources start at the tile's first row; rows past M (N) lie
    // beyond the record count and read as zero.
    const _Float16 *Ab = p.A + tc.b * p.sA + m0 * K;
    const _Float16 *Bb = p.B + tc.b * p.sB + n0 * K;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(Ab, (M - m0) * K * 2);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bb, (N - n0) * K * 2);

    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
            acc[i][j] = f32x16{};

    // ---- global -> LDS ----------------------------------------------------
    // LOAD_DIRECT: wave w fills 8-row groups w, w + WM*WN, ... of the A and
    // B tiles; lane l writes physical chunk l % 8 of row l / 8 of the group,
    // so it fetches the logical chunk that the swizzle puts there.
    constexpr int A_GROUPS = BM / ROWS_PER_WAVE_LOAD / (WM * WN);
    constexpr int B_GROUPS = BN / ROWS_PER_WAVE_LOAD / (WM * WN);
    // LOAD_VREG / LOAD_ELEM: thread t owns slots t, t + NT, ... of the
    // (BM + BN) x CHUNKS chunk grid (row-major), A rows first.
    constexpr int SLOTS = (BM + BN) * CHUNKS / NT;
    static_assert((BM + BN) * CHUNKS % NT == 0, "slots divide evenly");

    auto issue_direct = [&](int stage, int64_t k0) {
        GTN_LDS _Float16 *base =
            (GTN_LDS _Float16 *)(lds) + stage * STAGE_HALVES;
        const int rrow = lane / CHUNKS, pch = lane % CHUNKS;
#pragma unroll
        for (int g = 0; g < A_GROUPS; ++g) {
            const int grp = wave + g * WM * WN;
            const int row = grp * ROWS_PER_WAVE_LOAD + rrow;
            const int lch = swizzle_chunk<SWZ>(row, pch);
            const int64_t kk = k0 + lch * 8;
            const uint32_t off = kk < k_end
                                     ? (uint32_t)((row * K + kk) * 2)
                                     : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rA, (GTN_LDS void *)(base + grp * ROWS_PER_WAVE_LOAD * BK), 16,
                off, 0, 0, 0);
        }
#pragma unroll
        for (int g = 0; g < B_GROUPS; ++g) {
            const int grp = wave + g * WM * WN;
            const int row = grp * ROWS_PER_WAVE_LOAD + rrow;
            const int lch = swizzle_chunk<SWZ>(row, pch);
            const int64_t kk = k0 + lch * 8;
            const uint32_t off = kk < k_end
                                     ? (uint32_t)((row * K + kk) * 2)
                                     : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rB,
                (GTN_LDS void *)(base + BM * BK +
                                 grp * ROWS_PER_WAVE_LOAD * BK),
                16, off, 0, 0, 0);
        }
    };

    u32x4 stage_regs[LOADER == LOAD_DIRECT ? 1 : SLOTS];

    // Slot block i covers tile rows [i*RB, (i+1)*RB) of the A-then-B row
    // list; RB divides BM, so a block lies wholly in A or wholly in B and
    // the operand choice is a compile-time constant per i.
    constexpr int RB = NT / CHUNKS;
    static_assert(BM % RB == 0, "slot blocks do not straddle A and B");
    auto fetch_regs = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const bool isA = i * RB < BM;
            const int row = (isA ? i * RB : i * RB - BM) + tid / CHUNKS;
            const int lch = tid % CHUNKS;
            const __amdgpu_buffer_rsrc_t r = isA ? rA : rB;
            const int64_t kk = k0 + lch * 8;
            if (LOADER == LOAD_VREG) {
                const uint32_t off = kk < k_end
                                         ? (uint32_t)((row * K + kk) * 2)
                                         : kOutOfRange;
                stage_regs[i] = __builtin_amdgcn_raw_buffer_load_b128(r, off,
                                                                      0, 0);
            } else {
                uint16_t e[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const uint32_t off =
                        kk + x < k_end ? (uint32_t)((row * K + kk + x) * 2)
                                       : kOutOfRange;
                    e[x] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
                }
                stage_regs[i] = u32x4{e[0] | ((uint32_t)e[1] << 16),
                                      e[2] | ((uint32_t)e[3] << 16),
                                      e[4] | ((uint32_t)e[5] << 16),
                                      e[6] | ((uint32_t)e[7] << 16)};
            }
        }
    };

    auto store_regs = [&](int stage) {
        _Float16 *base = lds + stage * STAGE_HALVES;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const bool isA = i * RB < BM;
            const int row = (isA ? i * RB : i * RB - BM) + tid / CHUNKS;
            const int pch = swizzle_chunk<SWZ>(row, tid % CHUNKS);
            *(u32x4 *)(base + (isA ? 0 : BM * BK) + row * BK + pch * 8) =
                stage_regs[i];
        }
    };

    // ---- MFMA on one LDS stage -------------------------------------------
    auto compute = [&](int stage) {
        const _Float16 *sA = lds + stage * STAGE_HALVES;
        const _Float16 *sB = sA + BM * BK;
        const int frow = lane & 31;
        const int fhalf = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            half8 af[MI], bf[NI];
            const int ch = ks * 2 + fhalf;
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int row = wm * WTM + i * 32 + frow;
                af[i] = *(const half8 *)(sA + row * BK +
                                         swizzle_chunk<SWZ>(row, ch) * 8);
            }
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int row = wn * WTN + j * 32 + frow;
                bf[j] = *(const half8 *)(sB + row * BK +
                                         swizzle_chunk<SWZ>(row, ch) * 8);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        bf[j], af[i], acc[i][j], 0, 0, 0);
        }
    };

    // ---- main loop -------------------------------------------------------
    if (ktiles > 0) {
        if (LOADER == LOAD_DIRECT) {
            issue_direct(0, k_begin);
        } else {
            fetch_regs(k_begin);
            store_regs(0);
        }
    }
    for (int kt = 0; kt < ktiles; ++kt) {
        const int cur = kt & 1;
        if (LOADER == LOAD_DIRECT)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const bool more = kt + 1 < ktiles;
        const int64_t k_next = k_begin + (int64_t)(kt + 1) * BK;
        if (more) {
            if (LOADER == LOAD_DIRECT)
                issue_direct(cur ^ 1, k_next);
            else
                fetch_regs(k_next);
        }
        compute(cur);
        if (LOADER != LOAD_DIRECT && more)
            store_regs(cur ^ 1);
    }

    // ---- epilogue --------------------------------------------------------
    // Accumulator block (i, j), register 4g + e of lane l holds
    //   m = m0 + wm*WTM + i*32 + (l % 32)
    //   n = n0 + wn*WTN + j*32 + 8g + 4(l / 32) + e.
    const int em = lane & 31;
    const int en = (lane >> 5) * 4;
    if (SPLIT) {
        float *wsb = p.ws + ((int64_t)tc.s * p.batch + tc.b) * M * p.ws_ld +
                     m0 * p.ws_ld;
        const __amdgpu_buffer_rsrc_t rW =
            make_rsrc(wsb, (M - m0) * p.ws_ld * 4);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int lm = wm * WTM + i * 32 + em;
                    const int64_t n = n0 + wn * WTN + j * 32 + 8 * g + en;
                    const uint32_t off =
                        n < N ? (uint32_t)((lm * p.ws_ld + n) * 4)
                              : kOutOfRange;
                    f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1],
                               acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(u32x4, v), rW, off, 0, 0);
                }
        return;
    }

    constexpr int ES = OutTraits<OutT>::bytes;
    OutT *Db = (OutT *)p.D + tc.b * p.sD + m0 * N;
    const __amdgpu_buffer_rsrc_t rD = make_rsrc(Db, (M - m0) * N * ES);
    const bool use_c = p.beta != 0.0f;
    const OutT *Cb = use_c ? (const OutT *)p.C + tc.b * p.sC + m0 * N
                           : (const OutT *)p.D;
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(Cb, use_c ? (M - m0) * N * ES
                                                          : 0);
    const float alpha = p.alpha, beta = p.beta;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int lm = wm * WTM + i * 32 + em;
                const int64_t n = n0 + wn * WTN + j * 32 + 8 * g + en;
                f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1],
                           acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                v = v * alpha;
                if (VEC_OUT) {
                    const uint32_t off =
                        n < N ? (uint32_t)((lm * N + n) * ES) : kOutOfRange;
                    if (use_c) {
                        f32x4 c = load_out_vec4(rC, off, (OutT *)nullptr);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v[e] = __builtin_fmaf(beta, c[e], v[e]);
                    }
                    store_out_vec4(rD, off, v, (OutT *)nullptr);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t off =
                            n + e < N ? (uint32_t)((lm * N + n + e) * ES)
                                      : kOutOfRange;
                        float x = v[e];
                        if (use_c)
                            x = __builtin_fmaf(
                                beta, load_out_elem(rC, off, (OutT *)nullptr),
                                x);
                        store_out_elem(rD, off, x, (OutT *)nullptr);
                    }
                }
            }
}

// ---------------------------------------------------------------------------
// Split-K reduction: D = alpha * sum_s ws[s] + beta * C, slices summed in
// order s = 0, 1, ... so that the result does not depend on timing.  One
// thread per 4 consecutive outputs of a row.
// ---------------------------------------------------------------------------
template <typename OutT, bool VEC_OUT>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(GemmArgs p)
{
    const int64_t groups_per_row = (p.N + 3) / 4;
    const int64_t rows = (int64_t)p.batch * p.M;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= rows * groups_per_row)
        return;
    const int64_t row = gid / groups_per_row;
    const int64_t n = (gid - row * groups_per_row) * 4;
    const int64_t b = row / p.M, m = row - b * p.M;
    const int64_t slice = (int64_t)p.batch * p.M * p.ws_ld;
    const float *w = p.ws + row * p.ws_ld + n;
    f32x4 s = *(const f32x4 *)w;
    for (int k = 1; k < p.splits; ++k) {
        const f32x4 t = *(const f32x4 *)(w + k * slice);
        s = s + t;
    }
    constexpr int ES = OutTraits<OutT>::bytes;
    OutT *Drow = (OutT *)p.D + b * p.sD + m * p.N;
    const __amdgpu_buffer_rsrc_t rD = make_rsrc(Drow, p.N * ES);
    const bool use_c = p.beta != 0.0f;
    const OutT *Crow = use_c ? (const OutT *)p.C + b * p.sC + m * p.N
                             : (const OutT *)p.D;
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(Crow, use_c ? p.N * ES : 0);
    f32x4 v = s * p.alpha;
    if (VEC_OUT) {
        const uint32_t off = (uint32_t)(n * ES);
        if (use_c) {
            f32x4 c = load_out_vec4(rC, off, (OutT *)nullptr);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = __builtin_fmaf(p.beta, c[e], v[e]);
        }
        store_out_vec4(rD, off, v, (OutT *)nullptr);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t off =
                n + e < p.N ? (uint32_t)((n + e) * ES) : kOutOfRange;
            float x = v[e];
            if (use_c)
                x = __builtin_fmaf(p.beta,
                                   load_out_elem(rC, off, (OutT *)nullptr), x);
            store_out_elem(rD, off, x, (OutT *)nullptr);
        }
    }
}

}  // namespace gtn
