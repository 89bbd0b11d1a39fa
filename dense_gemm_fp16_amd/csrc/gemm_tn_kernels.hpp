// HIP kernels of the fp16 TN GEMM  D = alpha * A * B^T + beta * C  for
// gfx950 (MI355X, CDNA4).
//
// One workgroup owns one BM x BN tile of D for one batch entry (and, with
// split-K, one slice of K), as the CTA does in page "cute(8) smem_gemm"
// (yuyanqi.com, kernel listing and section 6: a CTA walks the K dimension
// of its A rows and B rows in kTileK-wide steps, and an inner loop walks the
// MMA k-steps of each step).  The CDNA4 design of each stage:
//
//  * global -> LDS: 16-byte buffer loads that write LDS directly
//    (buffer_load_dwordx4 ... lds), no VGPR staging.  A row of a BK = 64
//    tile is 128 bytes = 8 chunks of 16 bytes, so 8 consecutive lanes read
//    one full 128-byte line (coalesced).  Rows past M / N and chunks past K
//    get an out-of-range buffer offset, which the hardware turns into
//    zeros: that is the edge predication (page "Mat Transpose CuTe 版代码学习",
//    chuoer47.github.io, version 1: a per-element coordinate mask decides
//    which accesses happen).  Odd sizes, strides or alignments take an
//    element-wise loader into the same LDS layout.
//  * LDS layout: chunk c of row r is stored at chunk c ^ f(r) of that row:
//    an XOR swizzle of 16-byte groups, which keeps each group contiguous
//    for 128-bit reads while spreading one logical chunk of consecutive
//    rows over distinct banks (page "cute(8) smem_gemm", section 3:
//    Swizzle<B,M,S> XORs the row bits into the group index); f is chosen
//    for gfx950's 64-bank LDS (see swizzle_chunk).
//  * LDS -> registers: v_mfma_f32_16x16x32_f16 (and 32x32x16) takes, in
//    each lane, 8 consecutive-k halves of one row of each operand; in TN
//    storage that is one ds_read_b128 per operand per lane, with no
//    shuffle.  An operand stored along M / N is kept in LDS as rows of k
//    and read with the transposing ds_read_b64_tr_b16 (swizzle_mn).
//  * MFMA: each wave owns a (BM/WM) x (BN/WN) sub-tile as a grid of 16 x 16
//    (or 32 x 32) fp32 accumulator blocks.  The operands are issued as
//    (B, A), so the accumulator block is D^T: each lane then holds 4
//    consecutive n of one m per group of 4 registers.
//  * Pipeline: the 256 x 256 tile runs 8 waves in a ping-pong schedule
//    (two waves per SIMD, one loading while the other multiplies, A and B
//    in separate LDS rings); the smaller tiles interleave the next k-step's
//    fragment reads and a share of the tile loads with the MFMAs of the
//    current k-step, with one barrier per k-tile.
//  * Epilogue: alpha * acc (+ beta * C when beta != 0) in fp32, rounded to
//    fp16 or fp32 with round-to-nearest-even, staged through LDS and
//    written as whole 16-byte row pieces (element stores where the rows do
//    not allow them); out-of-range lanes are dropped.
//  * Split-K: slices write fp32 partial tiles to a workspace; a second
//    kernel sums them in slice order (deterministic) and applies the
//    epilogue.  The same path serves the bottom tile rows of a tail split.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_tn_config.hpp"
#include "lds_layout.hpp"

namespace gtn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
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
    int64_t lda, ldb, ldc, ldd;   // row strides in elements
    int64_t sA, sB, sC, sD;       // batch strides in elements
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

template <bool V>
struct Bool {
    static constexpr bool value = V;
};
template <int V>
struct Int {
    static constexpr int value = V;
    __device__ __host__ constexpr operator int() const { return V; }
};

// f(Int<0>{}), ..., f(Int<N - 1>{}) in order: a loop whose index is a
// compile-time constant inside the body (an immediate offset, say).
template <int N, int I = 0, typename F>
__device__ inline void static_for(F &&f)
{
    if constexpr (I < N) {
        f(Int<I>{});
        static_for<N, I + 1>(static_cast<F &&>(f));
    }
}

// s_waitcnt with only the vector-memory counter (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at "no wait").
template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) |
                               (15 << 8));
}
// s_waitcnt with only the LDS/scalar counter (lgkmcnt in bits 11:8).
template <int N>
__device__ inline void wait_lgkmcnt()
{
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (N << 8));
}

// Workgroup barrier with no implied memory wait.  __syncthreads() also
// releases every outstanding memory operation, which for the loads that
// write LDS directly means waiting for all of them, including prefetches
// meant to stay in flight across the barrier.  Callers wait explicitly for
// exactly what the barrier must order (lgkmcnt for LDS reads and writes,
// vmcnt for the direct-to-LDS loads of the tile about to be read); the
// empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ inline void block_sync()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ds_read_b64_tr_b16 at a constant byte offset from the LDS byte address
// `addr`, issued through inline asm.  The compiler builtin makes the
// compiler wait for every direct-to-LDS load still in flight before the
// read (it cannot tell that those loads fill other stages), which exposes
// a prefetch's whole HBM latency once per tile.  Callers order these reads
// against the tile loads with their own waits and barriers, and use the
// results only after an asm lgkmcnt(0) wait with the registers tied to it
// (lds_fence): the compiler does not track the asm reads, so it inserts no
// wait for them.
template <int OFF>
__device__ inline u32x2 ds_read_tr_asm(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "16-bit DS offset");
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                 : "=v"(r) : "v"(addr), "n"(OFF));
    return r;
}
// Makes `v` a new value defined here, after every asm statement before
// this one (a wait, say), so that no use of it is scheduled earlier.
template <typename T>
__device__ inline void tie_reg(T &v)
{
    asm volatile("" : "+v"(v));
}
// Waits for all LDS operations issued so far (as asm, which the compiler
// neither merges nor relaxes), then ties each register of `v` to the wait.
template <typename T, int N>
__device__ inline void lds_fence(T (&v)[N])
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int k = 0; k < N; ++k)
        tie_reg(v[k]);
}

// v_mfma_f32_16x16x32_f16 on accumulators held in the accumulation
// registers ("a" constraint), as asm so that the compiler can neither move
// the accumulators to ordinary registers nor reorder the MFMAs.  acc += the
// product of fragments b (16 columns) and a (16 rows); the _first form
// starts the sum at +0 (as acc = 0 + product would).  The compiler does not
// know these are MFMAs and so inserts none of their hazard padding: the
// operands a and b must come from LDS or memory loads (whose completion the
// compiler waits for), never from a vector-ALU write just before, and the
// results may be read only after after_mfma16_acc.
__device__ inline void mfma16_acc(f32x4 &acc, const half8 &b, const half8 &a)
{
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                 : "+a"(acc)
                 : "v"(b), "v"(a));
}
__device__ inline void mfma16_acc_first(f32x4 &acc, const half8 &b,
                                        const half8 &a)
{
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0"
                 : "=a"(acc)
                 : "v"(b), "v"(a));
}
// Wait states between the last asm MFMA and any read of its results (32,
// above what an 8-pass MFMA's result needs before a vector-ALU read), then
// every accumulator tied to the wait so that no read is scheduled before.
template <int MI, int NI>
__device__ inline void after_mfma16_acc(f32x4 (&acc)[MI][NI])
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
            asm volatile("" : "+a"(acc[i][j]));
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
// fp32 -> fp16, round to nearest even, of a value the compiler may not fold
// into the instruction that produced it.  Left alone, hipcc selects
// (_Float16)(x * alpha) as a mixed-precision FMA with a +0 addend
// (v_fma_mixlo_f16 d, alpha, x, 0), and -0 + +0 is +0: a product of -0
// (alpha < 0 times an exactly cancelling sum) came out as +0 at one
// accumulator of every 256-tile wave.  The empty asm makes the value opaque.
__device__ inline _Float16 to_half(float x)
{
    asm("" : "+v"(x));
    return (_Float16)x;
}
__device__ inline half4 to_half4(f32x4 v)
{
    return half4{to_half(v[0]), to_half(v[1]), to_half(v[2]), to_half(v[3])};
}

__device__ inline void store_out_elem(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                      float v, _Float16 *)
{
    _Float16 h = to_half(v);
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
    half4 h = to_half4(v);
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
//   BM x BN x BK : workgroup tile (BK = 32, 64 or 128); WM x WN waves;
//   STAGES : LDS ring depth of the direct loader (tile t + STAGES - 1 is in
//            flight while tile t is multiplied);
//   LOADER : LOAD_DIRECT (16-byte buffer loads straight into LDS),
//            LOAD_VREG (16-byte loads into VGPRs, then ds_write_b128),
//            LOAD_ELEM (2-byte loads, any K and any alignment); the two
//            register-staged loaders use a ring of two stages;
//   SCHED : with the direct loader, 0 = every wave interleaves its loads
//           with its MFMAs; 1 = ping-pong (8 waves, two per SIMD: in each
//           phase one wave of a SIMD multiplies a whole k-tile from
//           registers while the other issues loads and fragment reads);
//           2 = ping-pong with the tile loads split between the two wave
//           groups (A ring of three stages, B ring of two);
//           3 = four waves, one per SIMD, each multiplying a 128 x 128
//           quadrant with its accumulators in the accumulation registers,
//           tile loads and fragment reads at fixed slots between the MFMAs
//           (256 x 256 x 64 tiles of TN operands only);
//   MB : MFMA block edge, 32 (v_mfma_f32_32x32x16_f16) or 16
//        (v_mfma_f32_16x16x32_f16: the same work per cycle, in four times as
//        many instructions, at a lower power per flop on random data);
//   LAY : bit 0 / bit 1 set = A / B is stored contiguous along M / N.
//         The direct loader then loads its tile as k-rows and reads its
//         fragments with ds_read_b64_tr_b16; the element loader gathers
//         8 consecutive k of a row into the usual K-contiguous LDS tile;
//   OutT : _Float16 or float; SPLIT : write fp32 partials to the workspace;
//   VEC_OUT : rows of D (and C) start on 16-byte boundaries (N * element
//             size a multiple of 16, D / C 16-byte aligned): the tile is
//             written through LDS with 16-byte stores.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int LOADER,
          typename OutT, bool SPLIT, bool VEC_OUT, int MIN_WAVES, int SCHED,
          int MB, int LAY>
__global__ void __attribute__((amdgpu_flat_work_group_size(WM * WN * 64,
                                                           WM * WN * 64),
                               amdgpu_waves_per_eu(MIN_WAVES, 8)))
gemm_tn_kernel(GemmArgs p)
{
    constexpr int NW = WM * WN;
    constexpr int NT = NW * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    static_assert(MB == 32 || MB == 16, "MFMA blocks of 32x32 or 16x16");
    constexpr int MI = WTM / MB, NI = WTN / MB;
    // A fragment: lane l holds 8 consecutive k of row l % MB, at k offset
    // 8 * (l / MB) of a KM-wide k-step; QN lanes groups cover the k-step.
    constexpr int QN = 64 / MB;
    constexpr int KM = 8 * QN;
    constexpr int KSTEPS = BK / KM;
    // Accumulator registers per block, in groups of 4 consecutive n.
    constexpr int ACC = MB * MB / 64;
    constexpr int G = ACC / 4;
    constexpr int CHUNKS = BK / 8;            // 16-byte chunks per tile row
    constexpr int ROWS_PER_WAVE_LOAD = 64 / CHUNKS;
    constexpr int STAGE_HALVES = (BM + BN) * BK;
    static_assert(BK == 32 || BK == 64 || BK == 128,
                  "tile rows of 64, 128 or 256 bytes");
    static_assert(STAGES >= 2, "at least double buffering");
    static_assert(WTM % MB == 0 && WTN % MB == 0, "wave tile of MFMA blocks");
    static_assert(BK % KM == 0, "whole k-steps per tile");
    constexpr bool A_MN = (LAY & 1) != 0, B_MN = (LAY & 2) != 0;
    // Tiles held in LDS as k-rows (direct loader); the element loader
    // gathers operands stored along M / N into the K-contiguous tile.
    constexpr bool A_TR = A_MN && LOADER == LOAD_DIRECT;
    constexpr bool B_TR = B_MN && LOADER == LOAD_DIRECT;
    static_assert(LAY == 0 || LOADER == LOAD_ELEM ||
                      (LOADER == LOAD_DIRECT && MB == 16),
                  "operands stored along M / N: element loader, or direct "
                  "loader with 16x16 MFMA");
    static_assert(BM % (ROWS_PER_WAVE_LOAD * NW) == 0 &&
                      BN % (ROWS_PER_WAVE_LOAD * NW) == 0,
                  "every wave issues the same number of tile loads");
    // SCHED 2 keeps three stages of A and two of B (one more tile of A in
    // flight); the other schedules keep STAGES stages of A and B together.
    constexpr bool SPLIT_RING = SCHED == 2 && LOADER == LOAD_DIRECT;
    constexpr int A_STAGES = SPLIT_RING ? 3 : STAGES;
    constexpr int LDS_HALVES = SPLIT_RING ? (3 * BM + 2 * BN) * BK
                                          : STAGES * STAGE_HALVES;
    static_assert(LDS_HALVES * 2 <= 160 * 1024, "LDS budget");
    // Element offsets of the A and B tiles of a stage.
    auto a_base = [](int st) {
        return SPLIT_RING ? st * BM * BK : st * STAGE_HALVES;
    };
    auto b_base = [](int st) {
        return SPLIT_RING ? A_STAGES * BM * BK + st * BN * BK
                          : st * STAGE_HALVES + BM * BK;
    };

    __shared__ __attribute__((aligned(1024))) _Float16 lds[LDS_HALVES];

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
    const int64_t lda = p.lda, ldb = p.ldb;
    const _Float16 *Ab = p.A + tc.b * p.sA + m0 * lda;
    const _Float16 *Bb = p.B + tc.b * p.sB + n0 * ldb;
    // The record count ends at the last row's K-th element: rows past M
    // (N) start beyond it, so every element of theirs reads as zero.
    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(Ab, ((M - m0 - 1) * lda + K) * 2);
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc(Bb, ((N - n0 - 1) * ldb + K) * 2);

    typedef float accv __attribute__((ext_vector_type(ACC)));
    accv acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
            acc[i][j] = accv{};

    // ---- global -> LDS ----------------------------------------------------
    // LOAD_DIRECT: one buffer_load_dwordx4 ... lds of a wave fills
    // ROWS_PER_WAVE_LOAD whole tile rows (1 KiB, written contiguously from
    // the wave's LDS base); lane l lands in physical chunk l % CHUNKS of row
    // l / CHUNKS of that group, so it fetches the logical chunk the swizzle
    // maps there.  Wave w fills row groups w, w + NW, ... of A, then of B.
    constexpr bool FOUR_WAVE = SCHED == 3 && LOADER == LOAD_DIRECT;
    static_assert(!FOUR_WAVE || (BM == 256 && BN == 256 && BK == 64 &&
                                 WM == 2 && WN == 2 && STAGES == 2 &&
                                 MB == 16 && LAY == 0),
                  "four waves: 256 x 256 x 64 TN tiles, two stages");
    constexpr bool PINGPONG = (SCHED == 1 || SCHED == 2) &&
                              LOADER == LOAD_DIRECT;
    static_assert(!PINGPONG || (NW == 8 && STAGES == 2),
                  "ping-pong: two waves per SIMD, double-buffered LDS");
    // Waves that issue the tile loads: all of them, or the first half in
    // the ping-pong schedule.
    constexpr int NLOAD = PINGPONG ? NW / 2 : NW;
    constexpr int A_GROUPS = BM / ROWS_PER_WAVE_LOAD / NLOAD;
    constexpr int B_GROUPS = BN / ROWS_PER_WAVE_LOAD / NLOAD;
    static_assert(A_GROUPS * ROWS_PER_WAVE_LOAD * NLOAD == BM &&
                      B_GROUPS * ROWS_PER_WAVE_LOAD * NLOAD == BN,
                  "loading waves cover the tile");
    constexpr int LOADS_PER_TILE = A_GROUPS + B_GROUPS;
    const int rrow = lane / CHUNKS, pch = lane % CHUNKS;
    // Tile starting at k0 into LDS stage `stage` (issued by loading wave
    // lw); chunks at or past k_end (and every chunk once k0 >= k_end) read
    // as zero without touching memory.  Offsets are relative to the tile's
    // first row; rows past M / N fall beyond the record count and read as
    // zero.
    // Loads [x0, x1) of the tile's list (A row groups, then B row groups).
    // The swizzle repeats every 16 rows and a wave's row groups are
    // NLOAD * ROWS_PER_WAVE_LOAD rows apart, so every group of a wave shares
    // one per-lane chunk and offset; only a wave-uniform row stride differs.
    static_assert((NLOAD * ROWS_PER_WAVE_LOAD) % 16 == 0,
                  "a wave's row groups share the swizzle phase");
    // An operand stored along M (N): the tile is BK rows of k, each BM (BN)
    // elements; a 1 KiB load covers 1024 / (2*BM) rows.  Its resource
    // starts at row k0, column m0 (n0) and ends with row k_end - 1, so
    // offsets stay within 32 bits; rows past K and chunks past M (N, a
    // multiple of 8 on this path) read as zero.
    auto mn_rsrc = [&](const _Float16 *X, int64_t sX, int64_t ld, int64_t c0,
                       int64_t cols, int64_t k0) {
        const int64_t rows = k_end - k0;
        return make_rsrc(X + tc.b * sX + k0 * ld + c0,
                         rows > 0 ? ((rows - 1) * ld + cols - c0) * 2 : 0);
    };
    // Per-lane offsets of the loads of one wave into such a tile: the
    // wave's load groups are RG k-rows apart, a multiple of 8, so the
    // swizzle (a function of the row mod 16) takes at most two values, for
    // even and odd groups; a group adds a wave-uniform row stride.
    struct MnLanes {
        uint32_t even, odd;   // offset of group 0 / group 1 minus the stride
        int rk0;              // k-row of this lane in group 0
        bool c_even, c_odd;   // the lane's chunk lies before M (N)
    };
    auto mn_lanes = [&](auto cr_tag, int lw, int64_t ld, int64_t cols_left) {
        constexpr int CR = decltype(cr_tag)::value;
        constexpr int RPL = 64 / CR;              // k-rows per 1 KiB load
        constexpr int RG = NLOAD * RPL;
        static_assert(RG % 8 == 0, "two swizzle phases per wave");
        MnLanes m;
        m.rk0 = lw * RPL + lane / CR;
        const int ce = swizzle_mn<CR>(m.rk0, lane % CR);
        const int co = swizzle_mn<CR>(m.rk0 + RG, lane % CR);
        m.even = (uint32_t)((m.rk0 * ld + ce * 8) * 2);
        m.odd = (uint32_t)((m.rk0 * ld + co * 8) * 2);
        m.c_even = ce * 8 < cols_left;
        m.c_odd = co * 8 < cols_left;
        return m;
    };
    auto mn_offset = [&](auto cr_tag, const MnLanes &m, int g, int64_t k0,
                         int64_t ld) {
        constexpr int CR = decltype(cr_tag)::value;
        constexpr int RG = NLOAD * (64 / CR);
        const bool ok = (g & 1) ? m.c_odd : m.c_even;
        return ok && k0 + m.rk0 + g * RG < k_end
                   ? ((g & 1) ? m.odd : m.even) + (uint32_t)(g * RG * ld) * 2
                   : kOutOfRange;
    };
    auto issue_part = [&](int stage, int64_t k0, int lw, int x0, int x1) {
        GTN_LDS _Float16 *ldsp = (GTN_LDS _Float16 *)(lds);
        const int64_t rem64 = k_end - k0;
        const int rem = rem64 < 0 ? 0 : (rem64 > BK ? BK : (int)rem64);
        __amdgpu_buffer_rsrc_t rAt = rA, rBt = rB;
        MnLanes ma{}, mb{};
        if constexpr (A_TR) {
            rAt = mn_rsrc(p.A, p.sA, lda, m0, M, k0);
            ma = mn_lanes(Int<BM / 8>{}, lw, lda, M - m0);
        }
        if constexpr (B_TR) {
            rBt = mn_rsrc(p.B, p.sB, ldb, n0, N, k0);
            mb = mn_lanes(Int<BN / 8>{}, lw, ldb, N - n0);
        }
        const uint32_t kb = (uint32_t)(k0 < K ? k0 : K) * 2;
        const int row0 = lw * ROWS_PER_WAVE_LOAD + rrow;
        const int kc = swizzle_chunk<BK>(row0, pch) * 8;
        const uint32_t lane_off_a = (uint32_t)(row0 * lda + kc) * 2 + kb;
        const uint32_t lane_off_b = (uint32_t)(row0 * ldb + kc) * 2 + kb;
        const bool valid = kc < rem;
        const uint32_t group_stride_a =
            (uint32_t)(NLOAD * ROWS_PER_WAVE_LOAD * lda) * 2;
        const uint32_t group_stride_b =
            (uint32_t)(NLOAD * ROWS_PER_WAVE_LOAD * ldb) * 2;
#pragma unroll
        for (int x = 0; x < LOADS_PER_TILE; ++x) {
            if (x < x0 || x >= x1)
                continue;
            const bool isA = x < A_GROUPS;
            const int g = isA ? x : x - A_GROUPS;
            uint32_t off =
                !valid ? kOutOfRange
                : isA  ? lane_off_a + (uint32_t)g * group_stride_a
                       : lane_off_b + (uint32_t)g * group_stride_b;
            if (isA && A_TR)
                off = mn_offset(Int<BM / 8>{}, ma, g, k0, lda);
            if (!isA && B_TR)
                off = mn_offset(Int<BN / 8>{}, mb, g, k0, ldb);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                isA ? rAt : rBt,
                (GTN_LDS void *)(ldsp + (isA ? a_base(stage) : b_base(stage)) +
                                 (lw + g * NLOAD) * ROWS_PER_WAVE_LOAD * BK),
                16, off, 0, 0, 0);
        }
    };
    auto issue_direct = [&](int stage, int64_t k0, int lw) {
        issue_part(stage, k0, lw, 0, LOADS_PER_TILE);
    };

    // LOAD_VREG / LOAD_ELEM: thread t owns chunk slots t, t + NT, ... of the
    // (BM + BN) x CHUNKS grid (row-major, A rows first).  Slot block i
    // covers rows [i*RB, (i+1)*RB); RB divides BM, so a block lies wholly in
    // A or wholly in B and the operand is a compile-time choice per i.
    constexpr int SLOTS = (BM + BN) * CHUNKS / NT;
    constexpr int RB = NT / CHUNKS;
    static_assert((BM + BN) * CHUNKS % NT == 0, "slots divide evenly");
    static_assert(BM % RB == 0, "slot blocks do not straddle A and B");
    u32x4 stage_regs[LOADER == LOAD_DIRECT ? 1 : SLOTS];

    // The element loader reads an operand stored along M (N) through the
    // same per-k-tile resource as the direct loader (mn_rsrc above).
    auto fetch_regs = [&](int64_t k0) {
        __amdgpu_buffer_rsrc_t rAk = rA, rBk = rB;
        if constexpr (LOADER == LOAD_ELEM && A_MN)
            rAk = mn_rsrc(p.A, p.sA, lda, m0, M, k0);
        if constexpr (LOADER == LOAD_ELEM && B_MN)
            rBk = mn_rsrc(p.B, p.sB, ldb, n0, N, k0);
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const bool isA = i * RB < BM;
            const int row = (isA ? i * RB : i * RB - BM) + tid / CHUNKS;
            const int lch = tid % CHUNKS;
            const __amdgpu_buffer_rsrc_t r = isA ? rAk : rBk;
            const int64_t ld = isA ? lda : ldb;
            const int64_t kk = k0 + lch * 8;
            if (LOADER == LOAD_VREG) {
                const uint32_t off = kk < k_end
                                         ? (uint32_t)((row * ld + kk) * 2)
                                         : kOutOfRange;
                stage_regs[i] = __builtin_amdgcn_raw_buffer_load_b128(r, off,
                                                                      0, 0);
            } else {
                const bool mn = isA ? A_MN : B_MN;
                const bool row_in = row < (isA ? M - m0 : N - n0);
                uint16_t e[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const uint32_t off =
                        kk + x >= k_end ? kOutOfRange
                        : !mn           ? (uint32_t)((row * ld + kk + x) * 2)
                        : row_in ? (uint32_t)(((kk - k0 + x) * ld + row) * 2)
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
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const bool isA = i * RB < BM;
            const int row = (isA ? i * RB : i * RB - BM) + tid / CHUNKS;
            const int pch = swizzle_chunk<BK>(row, tid % CHUNKS);
            *(u32x4 *)(lds + (isA ? a_base(stage) : b_base(stage)) +
                       row * BK + pch * 8) = stage_regs[i];
        }
    };

    // ---- LDS -> registers, and the MFMAs of one KM-wide k-step ---------
    // Fragment of an operand tile stored along M (N) (BK rows of W
    // elements): rows c0 .. c0 + 15, the 32 k of k-step ks.  Each
    // ds_read_b64_tr_b16 gives lane i of every 16-lane group the 4 values
    // (k, c0 + i), k = kb .. kb + 3, when lane j of the group points at
    // (kb + j / 4, c0 + 4 (j % 4)); lane group g takes k = 8g .. 8g + 7 of
    // the k-step in two such reads.
    // Rows 32 ks + 8 g + 4 r + (i / 4): the swizzle reads row bits 0, 1
    // and 3 only, which 32 ks and 4 r (bit 2 is clear below) leave alone,
    // so one address per fragment serves both reads of every k-step, with
    // the rest in the instruction's offset.  Fragment f of the wave's
    // columns cbase + 16 f has byte offset ((2 cbase + 32 f) ^ 32 h) within
    // the row (2 h the row's swizzle), and 2 cbase, 32 f and the rest of the
    // address occupy disjoint bits, so every fragment's address is one
    // per-lane base XOR 32 f: one register per operand instead of one per
    // fragment.  The reads go through asm (ds_read_tr_asm); the fragments
    // are used after frags_ready().
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(const GTN_LDS void *)lds;
    auto read_tr = [&](auto w_tag, int tile, int cbase, int f, auto ks_tag) {
        constexpr int W = decltype(w_tag)::value;
        constexpr int KS = decltype(ks_tag)::value;
        static_assert(KM == 32 && MB == 16, "k-steps of 32, 16-wide blocks");
        const uint32_t base = lds_addr + (uint32_t)(tile * 2) +
                              tr_read_offset<W>(lane, cbase);
        const uint32_t addr = base ^ (uint32_t)(32 * f);
        const u32x2 lo = ds_read_tr_asm<KS * 32 * W * 2>(addr);
        const u32x2 hi = ds_read_tr_asm<(KS * 32 + 4) * W * 2>(addr);
        return __builtin_bit_cast(half8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    };
    // Fragments read by ds_read_tr_asm are usable after this: a wait for
    // all LDS reads, then the registers tied to it (no-op for TN tiles,
    // whose plain LDS reads the compiler waits for itself).
    auto frags_ready = [&](half8 (&af)[MI], half8 (&bf)[NI]) {
        if constexpr (A_TR || B_TR) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if constexpr (A_TR) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    tie_reg(af[i]);
            }
            if constexpr (B_TR) {
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    tie_reg(bf[j]);
            }
        }
    };
    // Fragments are read in the order the MFMAs below consume them (B0, A0,
    // then B1.., then A1..), so the first MFMAs of a k-step depend only on
    // the oldest reads of the previous one.
    auto read_frags2 = [&](int sta, int stb, auto ks, half8 (&af)[MI],
                           half8 (&bf)[NI]) {
        const _Float16 *sA = lds + a_base(sta);
        const _Float16 *sB = lds + b_base(stb);
        auto rd_a = [&](int i) {
            if constexpr (A_TR) {
                af[i] = read_tr(Int<BM>{}, a_base(sta), wm * WTM, i, ks);
            } else {
                af[i] = *(const half8 *)(sA + tn_frag_offset<BK, MB>(
                                                  wm * WTM + i * MB, lane, ks));
            }
        };
        auto rd_b = [&](int j) {
            if constexpr (B_TR) {
                bf[j] = read_tr(Int<BN>{}, b_base(stb), wn * WTN, j, ks);
            } else {
                bf[j] = *(const half8 *)(sB + tn_frag_offset<BK, MB>(
                                                  wn * WTN + j * MB, lane, ks));
            }
        };
        rd_b(0);
        rd_a(0);
#pragma unroll
        for (int j = 1; j < NI; ++j)
            rd_b(j);
#pragma unroll
        for (int i = 1; i < MI; ++i)
            rd_a(i);
    };
    auto read_frags = [&](int stage, auto ks, half8 (&af)[MI],
                          half8 (&bf)[NI]) {
        read_frags2(stage, stage, ks, af, bf);
    };
    auto mfma = [](const half8 &b, const half8 &a, const accv &c) {
        if constexpr (MB == 32)
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(b, a, c, 0, 0, 0);
    };
    auto mma = [&](const half8 (&af)[MI], const half8 (&bf)[NI]) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
                acc[i][j] = mfma(bf[j], af[i], acc[i][j]);
    };
    // Instruction order inside one k-step (the compiler otherwise waits on
    // each fragment right before its first MFMA): the next k-step's
    // fragment reads and this k-step's share of tile loads go out one each
    // after an MFMA, from the start of the k-step.
    constexpr int FRAGS = MI + NI;
    constexpr int MFMAS = MI * NI;

    // ---- main loop -------------------------------------------------------
    if constexpr (FOUR_WAVE) {
        // One wave per SIMD multiplies a 128 x 128 quadrant: per k-tile two
        // k-steps of 64 MFMAs (8 x 8 blocks), with one LDS read (1 KiB a
        // wave) or tile load slotted after given MFMAs instead of in phases:
        //   k-step 0 of tile t: after MFMA 4f + 1 the read of fragment f of
        //     k-step 1 (f = 0..15), after MFMA 4x + 3 tile load x of tile
        //     t + 1 into the other stage (x = 0..15: A row groups, then B);
        //   k-step 1 of tile t: after MFMA 47 each wave waits for its own
        //     loads of tile t + 1 and for its LDS reads, and passes the
        //     tile's one barrier: tile t + 1 is then whole in LDS, and every
        //     read of tile t's stage, which the loads of tile t + 2 refill
        //     next, is done; after MFMAs 48..63 the reads of tile t + 1's
        //     k-step 0 fragments.
        // Fragments are read in the order of first use (A 0, B 0..7,
        // A 1..7), and the loads of a tile have the rest of k-step 0 and
        // most of k-step 1 (about 1000 MFMA cycles) to land.  Past the last
        // tile the loads read zeros without touching memory (or, in the
        // fast form below, the last tile again), so the loop has no branch;
        // an empty K range multiplies one tile of zeros.
        // The accumulators (8 x 8 x 4 registers) live in the accumulation
        // registers through asm MFMAs (mfma16_acc): left to the compiler,
        // tiles of this size copy accumulators between the two register
        // files inside the loop.  The compiler waits for the fragment reads
        // before the asm (plain LDS loads, whose registers it tracks); the
        // results are read only after the padding below (after_mfma16_acc).
        half8 fa0[MI], fb0[NI], fa1[MI], fb1[NI];
        // Every fragment block starts on a multiple of 16 rows, where the
        // swizzle repeats, so a read's address is one per-lane offset per
        // k-step plus a wave-uniform part (stage, quadrant) and a constant
        // (the block): tn_frag_offset(16 b, l, ks) = 16 b BK +
        // tn_frag_offset(0, l, ks), checked on the host for every b, l, ks.
        // Written so, the compiler keeps two address registers per operand
        // instead of one per block.
        const int frag_off[2] = {tn_frag_offset<BK, MB>(0, lane, 0),
                                 tn_frag_offset<BK, MB>(0, lane, 1)};
        auto rd_a = [&](int st, int ks, int i) {
            return *(const half8 *)(lds + a_base(st) + wm * WTM * BK +
                                    frag_off[ks] + i * MB * BK);
        };
        auto rd_b = [&](int st, int ks, int j) {
            return *(const half8 *)(lds + b_base(st) + wn * WTN * BK +
                                    frag_off[ks] + j * MB * BK);
        };
        // Read number f (0..15) of a k-step's fragments.
        auto rd = [&](auto f_tag, int st, int ks, half8 (&af)[MI],
                      half8 (&bf)[NI]) {
            constexpr int f = decltype(f_tag)::value;
            if constexpr (f == 0)
                af[0] = rd_a(st, ks, 0);
            else if constexpr (f <= NI)
                bf[f - 1] = rd_b(st, ks, f - 1);
            else
                af[f - NI] = rd_a(st, ks, f - NI);
        };
        constexpr int BAR_AT = GTN_W4_BARRIER_AT;
        constexpr int LOAD_FIRST = GTN_W4_LOAD_FIRST;
        constexpr int LOAD_EVERY = GTN_W4_LOAD_EVERY;
        static_assert(MI == 8 && NI == 8 && LOADS_PER_TILE == 16,
                      "16 fragment reads and 16 tile loads per k-step");
        static_assert(BAR_AT + 16 < 64, "the reads after the barrier fit");
        static_assert(LOAD_FIRST + 15 * LOAD_EVERY < 64,
                      "the tile loads fit in k-step 0");
        // Tile loads.  Load x (A row groups 0..7, then B's) of wave w puts
        // rows 32 g + 8 w .. + 7 of group g = x % 8 into LDS, lane l
        // fetching, for physical chunk l % 8 of row 8 w + l / 8 (mod 32),
        // the logical chunk the swizzle maps there (as issue_part does).
        // A workgroup whose 256 rows of A and of B lie inside M and N and
        // whose K range is whole k-tiles takes the FAST form: the lane's
        // row and chunk in the offset register, the group's rows and the k
        // offset in the scalar offset, no per-lane arithmetic.  Any other
        // (edges, a K tail) puts the whole offset in the offset register,
        // where the record count stops rows past M (N), and sends chunks at
        // or past k_end out of range.
        GTN_LDS _Float16 *ldsp = (GTN_LDS _Float16 *)(lds);
        const int lrow = wave * 8 + (lane >> 3);
        const int lkc = swizzle_chunk<BK>(lrow, lane & 7) * 8;
        const uint32_t lane_a = (uint32_t)(lrow * lda + lkc) * 2;
        const uint32_t lane_b = (uint32_t)(lrow * ldb + lkc) * 2;
        const uint32_t grp_a = (uint32_t)(32 * lda) * 2;
        const uint32_t grp_b = (uint32_t)(32 * ldb) * 2;
        const bool rows_full = M - m0 >= BM && N - n0 >= BN;
        auto load = [&](auto fast, int stage, int64_t k0, int x) {
            const bool isA = x < 8;
            const int g = x & 7;
            GTN_LDS _Float16 *dst = ldsp +
                                    (isA ? a_base(stage) : b_base(stage)) +
                                    (g * 32 + wave * 8) * BK;
            const uint32_t lane_off = isA ? lane_a : lane_b;
            const uint32_t grp = (isA ? grp_a : grp_b) * (uint32_t)g;
            if constexpr (decltype(fast)::value) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    isA ? rA : rB, (GTN_LDS void *)dst, 16, lane_off,
                    grp + (uint32_t)k0 * 2, 0, 0);
            } else {
                const uint32_t off = k0 + lkc < k_end
                                         ? lane_off + grp + (uint32_t)k0 * 2
                                         : kOutOfRange;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    isA ? rA : rB, (GTN_LDS void *)dst, 16, off, 0, 0, 0);
            }
        };
        // k-step 0 of the tile in stage `cur` (fragments in fa0 / fb0);
        // FIRST: the tile's MFMAs start the sums; FAST: the loads of the
        // tile at k_next take the fast form.
        auto kstep0 = [&](auto first, auto fast, int cur, int64_t k_next) {
            static_for<64>([&](auto t) {
                constexpr int x = decltype(t)::value;
                constexpr int i = x / NI, j = x % NI;
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (decltype(first)::value)
                    mfma16_acc_first(acc[i][j], fb0[j], fa0[i]);
                else
                    mfma16_acc(acc[i][j], fb0[j], fa0[i]);
                if constexpr (x % 4 == 1)
                    rd(Int<x / 4>{}, cur, 1, fa1, fb1);
                if constexpr (x >= LOAD_FIRST &&
                              (x - LOAD_FIRST) % LOAD_EVERY == 0 &&
                              (x - LOAD_FIRST) / LOAD_EVERY < 16) {
                    constexpr int l = (x - LOAD_FIRST) / LOAD_EVERY;
                    load(fast, cur ^ 1, k_next, l);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        // k-step 1 of the tile in stage `cur`, then k-step 0's fragments of
        // the next tile from stage cur ^ 1.
        auto kstep1 = [&](int cur) {
            static_for<64>([&](auto t) {
                constexpr int x = decltype(t)::value;
                constexpr int i = x / NI, j = x % NI;
                __builtin_amdgcn_sched_barrier(0);
                mfma16_acc(acc[i][j], fb1[j], fa1[i]);
                if constexpr (x == BAR_AT) {
                    wait_vmcnt<0>();
                    wait_lgkmcnt<0>();
                    block_sync();
                }
                if constexpr (x > BAR_AT && x - BAR_AT <= 16)
                    rd(Int<x - BAR_AT - 1>{}, cur ^ 1, 0, fa0, fb0);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        const int nt = ktiles > 0 ? ktiles : 1;
        // The whole pipeline in one load form.  Past the last tile the fast
        // form loads the last tile again (into the stage nobody reads
        // again, within the operands), the other form reads zeros without
        // touching memory; either way the loop has no branch inside.
        auto pipeline = [&](auto fast) {
            constexpr bool F = decltype(fast)::value;
            auto k_of = [&](int t) {
                return k_begin + (int64_t)(F && t >= nt ? nt - 1 : t) * BK;
            };
            static_for<16>([&](auto x) { load(fast, 0, k_begin, x); });
            wait_vmcnt<0>();
            block_sync();
            static_for<16>([&](auto f) { rd(f, 0, 0, fa0, fb0); });
            kstep0(Bool<true>{}, fast, 0, k_of(1));
            for (int kt = 1; kt < nt; ++kt) {
                kstep1((kt - 1) & 1);
                kstep0(Bool<false>{}, fast, kt & 1, k_of(kt + 1));
            }
            kstep1((nt - 1) & 1);
        };
        if (rows_full && ktiles > 0 && (k_end - k_begin) % BK == 0)
            pipeline(Bool<true>{});
        else
            pipeline(Bool<false>{});
        after_mfma16_acc(acc);
    } else if constexpr (PINGPONG) {
        // Waves 0..3 (group 0) and 4..7 (group 1) share the SIMDs pairwise.
        // Each wave alternates a load phase (group 0 also issues the global
        // loads of the next tile; then fragments of the whole current tile
        // are read into registers) and a compute phase (all MFMAs of the
        // tile).  Group 1 runs one phase behind group 0, so in every phase
        // one wave per SIMD multiplies while the other loads.  Phases end
        // with a workgroup barrier:
        //   tile t in LDS  <- group 0 waits for its loads of tile t at the
        //                     end of its compute phase of tile t-1;
        //   stage reuse    <- group 1 reads tile t-1 in the phase before
        //                     group 0 starts the loads of tile t+1 into it.
        const int grp = wave >= NW / 2 ? 1 : 0;
        const int lw = wave - grp * (NW / 2);
        half8 fa[KSTEPS][MI], fb[KSTEPS][NI];
        if (SCHED == 2) {
            // Split ring: group 0 loads B one tile ahead (2 stages), group 1
            // loads A two tiles ahead (3 stages), so each load phase carries
            // half of a tile's traffic and every load has at least two
            // phases to land.
            //   B(t+1) lands <- group 0 waits at the end of its compute
            //                   phase of tile t;
            //   A(t+1) lands <- group 1 waits (leaving A(t+2) in flight) at
            //                   the end of its load phase of tile t.
            if (ktiles > 0) {
                if (grp == 0) {
                    issue_part(0, k_begin, lw, A_GROUPS, LOADS_PER_TILE);
                } else {
                    issue_part(0, k_begin, lw, 0, A_GROUPS);
                    issue_part(1, k_begin + BK, lw, 0, A_GROUPS);
                }
                // Tile 0 is all the first barrier must publish: A(1) may
                // stay in flight (group 1's wait at the end of its first
                // load phase covers it before tile 1 is read).
                if (grp == 1)
                    wait_vmcnt<A_GROUPS>();
                else
                    wait_vmcnt<0>();
                block_sync();
                if (grp == 1)
                    block_sync();
            }
            int sa = 0, sb = 0;
            for (int kt = 0; kt < ktiles; ++kt) {
                // load phase
                if (grp == 0)
                    issue_part(sb ^ 1, k_begin + (int64_t)(kt + 1) * BK, lw,
                               A_GROUPS, LOADS_PER_TILE);
                else
                    issue_part(sa == 0 ? 2 : sa - 1,
                               k_begin + (int64_t)(kt + 2) * BK, lw, 0,
                               A_GROUPS);
                static_for<KSTEPS>([&](auto ks) {
                    read_frags2(sa, sb, ks, fa[ks], fb[ks]);
                });
                wait_lgkmcnt<0>();
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
                    frags_ready(fa[ks], fb[ks]);
                if (grp == 1)
                    wait_vmcnt<A_GROUPS>();
                block_sync();
                // compute phase, at the waves' common priority: raising
                // the multiplying wave's priority cost 8k cycles per
                // launch at 4096 x 4096 x 8192 (counters, one box)
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
                    mma(fa[ks], fb[ks]);
                if (grp == 0)
                    wait_vmcnt<0>();
                block_sync();
                sa = sa == 2 ? 0 : sa + 1;
                sb ^= 1;
            }
            if (ktiles > 0 && grp == 0)
                block_sync();
            wait_vmcnt<0>();
        } else {
        if (ktiles > 0) {
            if (grp == 0)
                issue_direct(0, k_begin, lw);
            wait_vmcnt<0>();
            block_sync();
            if (grp == 1)
                block_sync();
        }
        for (int kt = 0; kt < ktiles; ++kt) {
            const int cur = kt & 1;
            // load phase
            if (grp == 0)
                issue_direct(cur ^ 1, k_begin + (int64_t)(kt + 1) * BK, lw);
            static_for<KSTEPS>([&](auto ks) {
                read_frags(cur, ks, fa[ks], fb[ks]);
            });
            wait_lgkmcnt<0>();
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
                frags_ready(fa[ks], fb[ks]);
            block_sync();
            // compute phase
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
                mma(fa[ks], fb[ks]);
            __builtin_amdgcn_s_setprio(0);
            if (grp == 0)
                wait_vmcnt<0>();
            block_sync();
        }
        if (ktiles > 0 && grp == 0)
            block_sync();
        }
    } else if constexpr (LOADER == LOAD_DIRECT) {
        // Tiles t .. t + STAGES - 1 are in LDS or in flight.  Fragments of
        // k-step s + 1 are read while the MFMAs of k-step s run.  At the
        // last k-step of tile t each wave waits for its own loads of tile
        // t + 1 and passes the one barrier of the tile (after which no wave
        // reads stage t % STAGES again and all of tile t + 1 is in LDS),
        // then reads the first fragments of tile t + 1 while the last MFMAs
        // of tile t are still in the pipe.
        // With three or more stages the loads of tile t + STAGES - 1 go into
        // the stage freed at the previous barrier and are spread over the
        // k-steps of tile t (a burst of them stalls the issuing waves on the
        // per-CU fill rate); with two stages they go, after the barrier,
        // into the stage just freed.
        static_assert(KSTEPS % 2 == 0,
                      "fragment double buffer returns to slot 0 each tile");
        constexpr bool SPREAD = STAGES >= 3;
        constexpr int PER = SPREAD ? LOADS_PER_TILE / KSTEPS : 0;
        static_assert(!SPREAD || PER * KSTEPS == LOADS_PER_TILE,
                      "loads split evenly over the k-steps");
        constexpr int PRO = SPREAD ? STAGES - 1 : STAGES;   // prologue tiles
        constexpr int WAIT_N = SPREAD
            ? (STAGES - 3) * LOADS_PER_TILE + (KSTEPS - 1) * PER
            : (STAGES - 2) * LOADS_PER_TILE;
        if (ktiles > 0) {
#pragma unroll
            for (int s = 0; s < PRO; ++s)
                issue_direct(s, k_begin + (int64_t)s * BK, wave);
            wait_vmcnt<(PRO - 1) * LOADS_PER_TILE>();
            block_sync();
        }
        half8 fa[2][MI], fb[2][NI];
        if (ktiles > 0)
            read_frags(0, Int<0>{}, fa[0], fb[0]);
        int cur = 0;
        for (int kt = 0; kt < ktiles; ++kt) {
            const int refill = cur == 0 ? STAGES - 1 : cur - 1;
            const int64_t k_refill = k_begin + (int64_t)(kt + STAGES - 1) * BK;
            static_for<KSTEPS - 1>([&](auto ks) {
                __builtin_amdgcn_sched_barrier(0);
                frags_ready(fa[ks & 1], fb[ks & 1]);
                if (SPREAD)
                    issue_part(refill, k_refill, wave, ks * PER,
                               (ks + 1) * PER);
                read_frags(cur, Int<decltype(ks)::value + 1>{},
                           fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
                mma(fa[ks & 1], fb[ks & 1]);
#pragma unroll
                for (int x = 0; x < MFMAS; ++x) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (x < FRAGS)
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    if (x < PER)
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            constexpr int LAST = (KSTEPS - 1) & 1;
            constexpr int LAST_LOADS = SPREAD ? PER : LOADS_PER_TILE;
            const int nxt = cur + 1 == STAGES ? 0 : cur + 1;
            wait_vmcnt<WAIT_N>();
            wait_lgkmcnt<0>();
            frags_ready(fa[LAST], fb[LAST]);
            block_sync();
            if (SPREAD)
                issue_part(refill, k_refill, wave, (KSTEPS - 1) * PER,
                           LOADS_PER_TILE);
            else
                issue_direct(cur, k_begin + (int64_t)(kt + STAGES) * BK, wave);
            read_frags(nxt, Int<0>{}, fa[LAST ^ 1], fb[LAST ^ 1]);
            mma(fa[LAST], fb[LAST]);
#pragma unroll
            for (int x = 0; x < MFMAS; ++x) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (x < FRAGS)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                if (x < LAST_LOADS)
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            cur = nxt;
        }
        // The last iteration read k-step 0 of the tile after the last one.
        // Nothing uses those fragments, but transposing reads are asm, which
        // the compiler neither waits for nor keeps the registers of once
        // their values are dead: without this wait and tie, a read still in
        // flight could land in registers the epilogue has taken over.
        frags_ready(fa[((KSTEPS - 1) & 1) ^ 1], fb[((KSTEPS - 1) & 1) ^ 1]);
        wait_vmcnt<0>();
    } else {
        if (ktiles > 0) {
            fetch_regs(k_begin);
            store_regs(0);
        }
        for (int kt = 0; kt < ktiles; ++kt) {
            const int cur = kt & 1;
            __syncthreads();
            const bool more = kt + 1 < ktiles;
            if (more)
                fetch_regs(k_begin + (int64_t)(kt + 1) * BK);
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                half8 af[MI], bf[NI];
                read_frags(cur, ks, af, bf);
                mma(af, bf);
            }
            if (more)
                store_regs(cur ^ 1);
        }
    }

    // ---- epilogue --------------------------------------------------------
    // Accumulator block (i, j), register 4g + e of lane l holds
    //   m = m0 + wm*WTM + i*MB + (l % MB)
    //   n = n0 + wn*WTN + j*MB + 4*QN*g + 4(l / MB) + e.
    // Each lane therefore owns 4 consecutive n of MB different rows; stored
    // straight from registers every instruction would touch MB rows with a
    // few bytes each.  Instead every wave turns its sub-tile around in its
    // own slice of LDS (free once the main loop is done) and writes whole
    // 256-byte row segments with 16-byte stores.
    const int em = lane % MB;
    const int en = (lane / MB) * 4;
    constexpr int ES = SPLIT ? 4 : OutTraits<OutT>::bytes;
    constexpr int LDS_BYTES = LDS_HALVES * 2;
    constexpr int REGION = LDS_BYTES / NW;            // bytes per wave
    constexpr int ROW_BYTES = WTN * ES;
    constexpr int CPR = ROW_BYTES / 16;               // 16-byte chunks per row
    constexpr int FIT = REGION / ROW_BYTES / 32 * 32;
    // rows per pass: as many as the slice holds, at most GTN_EPI_MAX_RPP
    constexpr int RPP_FIT = FIT < WTM ? FIT : WTM;
    constexpr int RPP =
        RPP_FIT < GTN_EPI_MAX_RPP ? RPP_FIT : GTN_EPI_MAX_RPP;
    constexpr int PASSES = WTM / RPP;
    static_assert(RPP >= 32 && WTM % RPP == 0, "LDS slice holds 32-row bands");
    static_assert(RPP * CPR % 64 == 0, "whole waves of 16-byte chunks");
    // Staged rows are laid out by stage_offset (lds_layout.hpp): the rows
    // a store instruction writes spread over distinct banks.
    char *region = (char *)lds + wave * REGION;

    // Fp32 results of the block in output precision, then into the slice.
    // BARE: finish returns the accumulators themselves, which no product
    // precedes, so the conversion needs no barrier (to_half).
    auto stage_pass = [&](int pass, auto finish, auto bare) {
#pragma unroll
        for (int ii = 0; ii < RPP / MB; ++ii) {
            const int i = pass * (RPP / MB) + ii;
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1],
                               acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                    v = finish(i, j, g, v);
                    const int r = ii * MB + em;
                    const int col = j * MB + 4 * QN * g + en;  // element column
                    const int cb = col * ES;                  // byte column
                    char *dst = region + stage_offset<ROW_BYTES>(r, cb);
                    if constexpr (ES == 4) {
                        *(f32x4 *)dst = v;
                    } else if constexpr (decltype(bare)::value) {
                        *(half4 *)dst = __builtin_convertvector(v, half4);
                    } else {
                        half4 h = to_half4(v);
                        *(half4 *)dst = h;
                    }
                }
        }
    };
    // Slice rows back out, 16 bytes per lane, row-contiguous.
    // A lane keeps its 16-byte column c = lane % CPR in every iteration
    // (CPR divides 64), and its row advances by 64 / CPR: one column check
    // and one 32-bit offset per pass, then an add per store (offsets are
    // below 2^31: the resource starts at the tile's first row, and rows
    // and columns are limited to 2^20 elements).  A column past n_limit
    // starts at kOutOfRange, which the adds keep out of range.
    // The LDS reads take stage_read_period addresses and constant offsets.
    static_assert(64 % CPR == 0, "a lane's column is fixed across stores");
    constexpr int RPER = stage_read_period<ROW_BYTES>();
    auto drain_pass = [&](int pass, __amdgpu_buffer_rsrc_t rOut, int64_t ld,
                          int64_t n_limit) {
        const int c = lane % CPR;
        const int64_t n = n0 + wn * WTN + c * (16 / ES);
        const int lm0 = wm * WTM + pass * RPP + lane / CPR;
        const uint32_t base =
            n < n_limit ? (uint32_t)((lm0 * ld + n) * ES) : kOutOfRange;
        const uint32_t step = (uint32_t)(64 / CPR * ld * ES);
        int roff[RPER];
#pragma unroll
        for (int q = 0; q < RPER; ++q)
            roff[q] = stage_read_offset<ROW_BYTES>(lane, q);
#pragma unroll
        for (int it = 0; it < RPP * CPR / 64; ++it) {
            const u32x4 v = *(const u32x4 *)(
                region + roff[it % RPER] +
                (it / RPER) * (RPER * (64 / CPR) * ROW_BYTES));
            __builtin_amdgcn_raw_buffer_store_b128(
                v, rOut, base + (uint32_t)it * step, 0, GTN_TILE_STORE_CPOL);
        }
    };

    // Without 16-byte rows, beta == 0 still stages D through LDS (then one
    // element per lane, consecutive lanes on consecutive elements of a row).
    const bool staged = SPLIT || VEC_OUT || p.beta == 0.0f;
    if (staged) {
        // All waves are done with the pipeline's LDS (and its last loads).
        wait_vmcnt<0>();
        __syncthreads();
    }
    if (SPLIT) {
        float *wsb = p.ws + ((int64_t)tc.s * p.batch + tc.b) * M * p.ws_ld +
                     m0 * p.ws_ld;
        const __amdgpu_buffer_rsrc_t rW =
            make_rsrc(wsb, (M - m0) * p.ws_ld * 4);
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
            stage_pass(pass, [](int, int, int, f32x4 v) { return v; },
                       Bool<true>{});
            drain_pass(pass, rW, p.ws_ld, N);
        }
        return;
    }

    const int64_t ldc = p.ldc, ldd = p.ldd;
    OutT *Db = (OutT *)p.D + tc.b * p.sD + m0 * ldd;
    const __amdgpu_buffer_rsrc_t rD =
        make_rsrc(Db, ((M - m0 - 1) * ldd + N) * ES);
    const bool use_c = p.beta != 0.0f;
    const OutT *Cb = use_c ? (const OutT *)p.C + tc.b * p.sC + m0 * ldc
                           : (const OutT *)p.D;
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(Cb, use_c ? ((M - m0 - 1) * ldc + N) * ES : 0);
    const float alpha = p.alpha, beta = p.beta;

    if (VEC_OUT) {
        // alpha (and beta * C, read in the accumulator layout) in fp32, one
        // rounding to the output type, then the coalesced write-out.
        auto with_c = [&](int i, int j, int g, f32x4 v) {
            const int lm = wm * WTM + i * MB + em;
            const int64_t n = n0 + wn * WTN + j * MB + 4 * QN * g + en;
            const uint32_t off =
                n < N ? (uint32_t)((lm * ldc + n) * ES) : kOutOfRange;
            const f32x4 c = load_out_vec4(rC, off, (OutT *)nullptr);
            v = v * alpha;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = __builtin_fmaf(beta, c[e], v[e]);
            return v;
        };
        auto no_c = [&](int, int, int, f32x4 v) { return v * alpha; };
        // alpha = 1 skips the multiply (x * 1 = x for every x): a vector
        // instruction per accumulator, which on the 256 tile's two waves
        // per SIMD is about 1000 cycles of the epilogue
        auto as_is = [](int, int, int, f32x4 v) { return v; };
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
            if (use_c)
                stage_pass(pass, with_c, Bool<false>{});
            else if (alpha == 1.0f)
                stage_pass(pass, as_is, Bool<true>{});
            else
                stage_pass(pass, no_c, Bool<false>{});
            drain_pass(pass, rD, ldd, N);
        }
        return;
    }

    // Rows whose length or alignment rules out 16-byte stores, beta == 0:
    // the same LDS staging, then each store instruction writes 64
    // consecutive elements of a row (whole lines) where the accumulator
    // layout would write 4-byte pieces 16 bytes apart in 16 rows.
    if (!use_c) {
        constexpr int EPR = WTN;                    // elements per staged row
        static_assert(RPP * EPR % 64 == 0, "whole waves of elements");
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
            stage_pass(pass, [&](int, int, int, f32x4 v) { return v * alpha; },
                       Bool<false>{});
#pragma unroll
            for (int it = 0; it < RPP * EPR / 64; ++it) {
                const int idx = it * 64 + lane;
                const int r = idx / EPR, ce = idx % EPR;
                const int cb = ce * ES;               // byte column
                const char *src = region + stage_offset<ROW_BYTES>(r, cb);
                const int lm = wm * WTM + pass * RPP + r;
                const int64_t n = n0 + wn * WTN + ce;
                const uint32_t off =
                    n < N ? (uint32_t)((lm * ldd + n) * ES) : kOutOfRange;
                if constexpr (ES == 4)
                    __builtin_amdgcn_raw_buffer_store_b32(
                        *(const uint32_t *)src, rD, off, 0, GTN_TILE_STORE_CPOL);
                else
                    __builtin_amdgcn_raw_buffer_store_b16(
                        *(const uint16_t *)src, rD, off, 0, GTN_TILE_STORE_CPOL);
            }
        }
        return;
    }

    // With C (beta != 0 here): element by element, straight from the
    // accumulators.  The value converted is fma(beta, c, alpha * acc), not a
    // bare product, so it takes the plain conversion: to_half's asm would
    // hold every value in its own register, and on the 256 tile that spills.
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int lm = wm * WTM + i * MB + em;
                const int64_t n = n0 + wn * WTN + j * MB + 4 * QN * g + en;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool in = n + e < N;
                    const uint32_t offd =
                        in ? (uint32_t)((lm * ldd + n + e) * ES) : kOutOfRange;
                    const uint32_t offc =
                        in ? (uint32_t)((lm * ldc + n + e) * ES) : kOutOfRange;
                    const float x = __builtin_fmaf(
                        beta, load_out_elem(rC, offc, (OutT *)nullptr),
                        acc[i][j][4 * g + e] * alpha);
                    if constexpr (ES == 2)
                        __builtin_amdgcn_raw_buffer_store_b16(
                            __builtin_bit_cast(uint16_t, (_Float16)x), rD,
                            offd, 0, 0);
                    else
                        store_out_elem(rD, offd, x, (OutT *)nullptr);
                }
            }
}

// ---------------------------------------------------------------------------
// Split-K reduction: D = alpha * sum_s ws[s] + beta * C, slices summed in
// order s = 0, 1, ... so that the result does not depend on timing.  One
// thread per 4 consecutive outputs of a row.  The loads of eight slices are
// issued before they are added (still in slice order): with few outputs
// and many slices the thread's chain of loads, one at a time, set the time
// (about 0.4 us per slice from the L2).
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
    int k = 1;
    for (; k + 8 <= p.splits; k += 8) {
        f32x4 t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            t[u] = *(const f32x4 *)(w + (k + u) * slice);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            s = s + t[u];
    }
    for (; k < p.splits; ++k)
        s = s + *(const f32x4 *)(w + k * slice);
    constexpr int ES = OutTraits<OutT>::bytes;
    OutT *Drow = (OutT *)p.D + b * p.sD + m * p.ldd;
    const __amdgpu_buffer_rsrc_t rD = make_rsrc(Drow, p.N * ES);
    const bool use_c = p.beta != 0.0f;
    const OutT *Crow = use_c ? (const OutT *)p.C + b * p.sC + m * p.ldc
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
