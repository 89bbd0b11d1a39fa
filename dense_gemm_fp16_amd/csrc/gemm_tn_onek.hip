// Persistent kernel for products whose K fits one k-tile (K <= 64): the
// batched attention-score product S = Q K^T at head dimension 64 is one
// (page "为什么 cutlass_cute_tutorial_zh.md 中要用 retile_D",
// blog.qingsen.net, section 1: Q is the A and K the B operand of a TN score
// GEMM; section 3: head dimension 64).
//
// Such a product is bound by writing D: 64 x 1024 x 1024 fp32 scores are
// 256 MiB against 16 MiB of operands.  With one tile per workgroup, every
// workgroup first waits for its operands (a load round trip) and only then
// writes; the two workgroups of a CU run in step, so each of a CU's rounds
// exposes that round trip.  Here one workgroup per CU walks a run of tiles
// and keeps the next tile's operands in flight while the current tile's
// stores drain:
//
//  * operands: LDS buffers of one 128 x 128 x 64 k-tile each (A and B,
//    32 KiB), filled by the direct-to-LDS 16-byte loads with the GEMM's
//    swizzle; tile i + DEPTH's loads are issued right after the barrier
//    that opens tile i;
//  * math: 4 waves of 64 x 64, v_mfma_f32_16x16x32_f16 with operands
//    issued (B, A), as in the tile kernels;
//  * epilogue: alpha (+ beta C) in fp32, one rounding, staged per wave in
//    LDS and written as 16-byte row pieces with the streaming store policy.
//
// The vector-memory counter drains in issue order, so at the top of a tile
// waiting until only the operations issued after its loads (later tiles'
// loads, earlier tiles' stores) are outstanding means that its loads have
// landed.
//
// Tiles go to XCDs in contiguous runs, in row order within a batch entry:
// the 32 workgroups of an XCD write neighbouring row pieces of the same
// rows of D.
#include "gemm_tn_launch.hpp"

namespace gtn {
namespace {

constexpr int kOkBM = 128, kOkBN = 128, kOkBK = 64;

// Tiles whose operands are in flight while a tile is multiplied and
// written, and the cache policy of the output stores.  Measured on the
// 64 x 1024 x 1024 x 64 score product (HIP events, interleaved, one box):
// one tile ahead with streaming stores 44.8 us; two tiles ahead 46.6 us;
// default-policy stores 56.2 / 58.5 us; a plain fill of the same 256 MiB
// 38.5 us.
#ifndef GTN_ONEK_DEPTH
#define GTN_ONEK_DEPTH 1
#endif
#ifndef GTN_ONEK_CPOL
#define GTN_ONEK_CPOL GTN_STORE_CPOL
#endif

template <typename OutT>
__global__ void __launch_bounds__(256) gemm_onek_kernel(GemmArgs p)
{
    // operand buffers: the current tile and DEPTH tiles in flight
    constexpr int DEPTH = GTN_ONEK_DEPTH;
    constexpr int NBUF = DEPTH + 1;
    constexpr int ES = OutTraits<OutT>::bytes;
    constexpr int OP = (kOkBM + kOkBN) * kOkBK;       // halves per buffer
    constexpr int WT = 64;                            // wave tile edge
    constexpr int ROW_BYTES = WT * ES;                // staged row
    constexpr int REGION = WT * ROW_BYTES;            // staged bytes per wave
    constexpr int CPR = ROW_BYTES / 16;               // 16-byte chunks per row
    constexpr int STORES = WT * CPR / 64;             // store instructions
    constexpr int LOADS = OP * 2 / 1024 / 4;          // 1 KiB loads per wave
    static_assert(NBUF * OP * 2 + 4 * REGION <= 160 * 1024, "LDS budget");
    static_assert(DEPTH * (STORES + LOADS) < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char lds[NBUF * OP * 2 +
                                                       4 * REGION];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // This workgroup's tiles: XCD x = blockIdx % 8 owns a contiguous run of
    // logical tiles, walked by its workgroups in turn.
    const int per_b = p.tiles_m * p.tiles_n;
    const int total = per_b * p.batch;
    const int xcds = gridDim.x < 8 ? (int)gridDim.x : 8;
    const int x = blockIdx.x % xcds;
    const int slot = blockIdx.x / xcds;
    const int slots = (gridDim.x - x + xcds - 1) / xcds;   // WGs on XCD x
    const int q = total / xcds, r = total % xcds;
    const int first = x * q + (x < r ? x : r);
    const int run = q + (x < r ? 1 : 0);
    const int count = slot < run ? (run - slot + slots - 1) / slots : 0;

    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t lda = p.lda, ldb = p.ldb, ldd = p.ldd, ldc = p.ldc;
    const float alpha = p.alpha, beta = p.beta;
    const bool use_c = beta != 0.0f;

    struct Tile {
        int b;
        int64_t m0, n0;
    };
    auto tile_of = [&](int i) {
        const int logical = first + slot + i * slots;
        Tile t;
        t.b = logical / per_b;
        const int in_b = logical - t.b * per_b;
        t.m0 = (int64_t)(in_b / p.tiles_n) * kOkBM;
        t.n0 = (int64_t)(in_b % p.tiles_n) * kOkBN;
        return t;
    };

    // Loads of one tile into buffer `buf`: load g of wave w fills rows
    // 8 (4 g + w) .. + 7 of A (g < 4) or of B (g >= 4); lane l lands in
    // physical chunk l % 8 of row l / 8 and fetches the logical chunk the
    // swizzle maps there; chunks past K and rows past M / N read as zero.
    const int lrow = 8 * wave + (lane >> 3);
    const int lk = swizzle_chunk<kOkBK>(lrow, lane & 7) * 8;
    // Tile i of the run into buffer i % NBUF.  Positions past the run issue
    // the same number of loads, all out of range (zeros), so the waits
    // below count exactly.
    auto issue = [&](int i) {
        const Tile t = tile_of(i < count ? i : 0);
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(
            p.A + t.b * p.sA + t.m0 * lda, ((M - t.m0 - 1) * lda + K) * 2);
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(
            p.B + t.b * p.sB + t.n0 * ldb, ((N - t.n0 - 1) * ldb + K) * 2);
        GTN_LDS char *base = (GTN_LDS char *)lds + (i % NBUF) * OP * 2;
        const bool kin = lk < K && i < count;
#pragma unroll
        for (int g = 0; g < LOADS; ++g) {
            const bool isA = g < LOADS / 2;
            const int row = lrow + 32 * (isA ? g : g - LOADS / 2);
            const int64_t ld = isA ? lda : ldb;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                isA ? rA : rB,
                (GTN_LDS void *)(base + (isA ? 0 : kOkBM * kOkBK * 2) +
                                 (row - (lane >> 3)) * kOkBK * 2),
                16, kin ? (uint32_t)((row * ld + lk) * 2) : kOutOfRange, 0, 0,
                0);
        }
    };

    char *region = lds + NBUF * OP * 2 + wave * REGION;
    static_assert(64 % CPR == 0, "a lane's column is fixed across stores");
    constexpr int RPER = stage_read_period<ROW_BYTES>();
    int roff[RPER];
#pragma unroll
    for (int q = 0; q < RPER; ++q)
        roff[q] = stage_read_offset<ROW_BYTES>(lane, q);
    if (count > 0) {
#pragma unroll
        for (int i = 0; i < DEPTH; ++i)
            issue(i);
    }
    for (int i = 0; i < count; ++i) {
        const Tile t = tile_of(i);
        // Tile i's loads landed.  Issued after them: the loads of the tiles
        // up to i + DEPTH - 1 (issued in the prologue, or after the barriers
        // of tiles i - DEPTH + 1 .. i - 1) and the stores of the tiles
        // since i - DEPTH.
        if (i == 0)
            wait_vmcnt<(DEPTH - 1) * LOADS>();
        else if (DEPTH == 2 && i == 1)
            wait_vmcnt<LOADS + STORES>();
        else
            wait_vmcnt<(DEPTH - 1) * LOADS + DEPTH * STORES>();
        // every wave's share of tile i is in LDS, and every wave is done
        // reading the buffer of tile i - 1, which tile i + DEPTH takes
        block_sync();
        issue(i + DEPTH);

        const _Float16 *sA =
            (const _Float16 *)(lds + (i % NBUF) * OP * 2);
        const _Float16 *sB = sA + kOkBM * kOkBK;
        f32x4 acc[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kOkBK / 32; ++ks) {
            half8 af[4], bf[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *(const half8 *)(sB + tn_frag_offset<kOkBK, 16>(
                                                  wn * WT + 16 * j, lane, ks));
#pragma unroll
            for (int a = 0; a < 4; ++a)
                af[a] = *(const half8 *)(sA + tn_frag_offset<kOkBK, 16>(
                                                  wm * WT + 16 * a, lane, ks));
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        bf[j], af[a], acc[a][j], 0, 0, 0);
        }

        // Epilogue.  Block (a, j), lane l: row wm*64 + 16a + l % 16,
        // columns wn*64 + 16j + 4 (l / 16) .. + 3.
        OutT *Db = (OutT *)p.D + t.b * p.sD + t.m0 * ldd;
        const __amdgpu_buffer_rsrc_t rD =
            make_rsrc(Db, ((M - t.m0 - 1) * ldd + N) * ES);
        const OutT *Cb = use_c ? (const OutT *)p.C + t.b * p.sC + t.m0 * ldc
                               : (const OutT *)p.D;
        const __amdgpu_buffer_rsrc_t rC =
            make_rsrc(Cb, use_c ? ((M - t.m0 - 1) * ldc + N) * ES : 0);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = 16 * a + (lane & 15);
                const int cc = 16 * j + 4 * (lane >> 4);
                f32x4 v = acc[a][j] * alpha;
                if (use_c) {
                    const int64_t n = t.n0 + wn * WT + cc;
                    const int m = wm * WT + rr;
                    const f32x4 cv = load_out_vec4(
                        rC, n < N ? (uint32_t)((m * ldc + n) * ES) : kOutOfRange,
                        (OutT *)nullptr);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = __builtin_fmaf(beta, cv[e], v[e]);
                }
                char *dst = region + stage_offset<ROW_BYTES>(rr, cc * ES);
                if constexpr (ES == 4) {
                    *(f32x4 *)dst = v;
                } else {
                    const half4 h = to_half4(v);
                    *(half4 *)dst = h;
                }
            }
        // A lane keeps its 16-byte column in every store (CPR divides 64)
        // and its row advances by 64 / CPR: one column check and one 32-bit
        // offset per tile (below 2^31: the resource starts at the tile's
        // first row), an add per store; the staged rows are read at
        // stage_read_period addresses plus constants.
        {
            const int c = lane % CPR;
            const int64_t n = t.n0 + wn * WT + c * (16 / ES);
            const int m = wm * WT + lane / CPR;
            const uint32_t base =
                n < N ? (uint32_t)((m * ldd + n) * ES) : kOutOfRange;
            const uint32_t step = (uint32_t)(64 / CPR * ldd * ES);
#pragma unroll
            for (int it = 0; it < STORES; ++it) {
                const u32x4 v = *(const u32x4 *)(
                    region + roff[it % RPER] +
                    (it / RPER) * (RPER * (64 / CPR) * ROW_BYTES));
                __builtin_amdgcn_raw_buffer_store_b128(
                    v, rD, base + (uint32_t)it * step, 0, GTN_ONEK_CPOL);
            }
        }
    }
    wait_vmcnt<0>();
}

}  // namespace

hipError_t launch_onek(const GemmArgs &a, bool out_f32, unsigned grid,
                       hipStream_t s)
{
    void *fn = out_f32 ? (void *)&gemm_onek_kernel<float>
                       : (void *)&gemm_onek_kernel<_Float16>;
    GemmArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, s);
}

}  // namespace gtn
