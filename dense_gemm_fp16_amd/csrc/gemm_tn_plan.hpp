// Host-side argument checking and kernel-configuration choice for the fp16
// TN GEMM.  Pure C++: no HIP call is made here, so every error path can be
// exercised on a machine without a GPU.
#pragma once

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gemm_tn.h"
#include "gemm_tn_config.hpp"

namespace gtn {

// Loader kinds (must match the kernel template's Loader enum).
enum { PLAN_LOAD_DIRECT = 0, PLAN_LOAD_VREG = 1, PLAN_LOAD_ELEM = 2 };
// Tile shapes, all with BK = 64 and 2 x 2 waves.
enum { TILE_256 = 0, TILE_128 = 1, TILE_64 = 2, NUM_TILES = 3 };

constexpr int kTileDim[NUM_TILES] = {256, 128, 64};
constexpr int kTileBK[NUM_TILES] = {GTN_T256_BK, GTN_T128_BK, GTN_T64_BK};
constexpr int kTileStages[NUM_TILES] = {GTN_T256_STAGES, GTN_T128_STAGES,
                                        GTN_T64_STAGES};
// Ring depth and k-tile depth of split-K slices (differ on the 64 tile
// only).
constexpr int kTileSplitStages[NUM_TILES] = {
    GTN_T256_STAGES, GTN_T128_STAGES, GTN_T64_SPLIT_STAGES};
constexpr int kTileSplitBK[NUM_TILES] = {GTN_T256_BK, GTN_T128_BK,
                                         GTN_T64_SPLIT_BK};
constexpr int kTileWM[NUM_TILES] = {GTN_T256_WM, 2, 2};
constexpr int kTileWN[NUM_TILES] = {GTN_T256_WN, 2, 2};
constexpr int kTileSched[NUM_TILES] = {GTN_T256_SCHED, 0, 0};
constexpr int kTileMfma[NUM_TILES] = {GTN_T256_MFMA, GTN_T128_MFMA,
                                      GTN_T64_MFMA};
constexpr int kTileDirectLays[NUM_TILES] = {
    GTN_T256_DIRECT_LAYS, GTN_T128_DIRECT_LAYS, GTN_T64_DIRECT_LAYS};
constexpr bool kTileElemLays[NUM_TILES] = {
    GTN_T256_ELEM_LAYS, GTN_T128_ELEM_LAYS, GTN_T64_ELEM_LAYS};
// Workgroups of each tile that fit on one CU at once, as the tail split
// counts them (LDS-limited: the 256 tile's rings take 160 KiB, the 128
// tile's and the 64 tile's split-K rings 64 KiB of the 160 KiB).
constexpr int kTileWgsPerCu[NUM_TILES] = {1, 2, 2};
constexpr int kBK = 64;   // split-K slices are multiples of every tile's BK
constexpr int kCUs = 256;  // MI355X compute units (8 XCDs x 32)

// Addressing limits: the kernels form 32-bit byte offsets relative to the
// first row of a tile (at most 256 rows), so an operand row stride (and K)
// may be at most 2^21 fp16 elements and an output row stride (and N) at
// most 2^20 elements.
constexpr int64_t kMaxK = int64_t(1) << 21;
constexpr int64_t kMaxN = int64_t(1) << 20;
constexpr int64_t kMaxM = (int64_t(1) << 31) - 1;

// Vector loader used when alignment allows it.
constexpr int kDefaultVecLoader = PLAN_LOAD_DIRECT;

struct Plan {
    int status = GEMM_TN_OK;
    bool noop = false;       // nothing to compute (batch, M or N is 0)
    int tile = TILE_64;
    int bm = 64, bn = 64;
    int loader = PLAN_LOAD_ELEM;
    bool a_mn = false, b_mn = false;   // operand stored along M / N
    int layout = 0;          // kernel layout bits (LAY of the kernel)
    bool vec_out = false;
    int splits = 1;
    int64_t k_split = 0;
    int group_m = 8;
    int tiles_m = 0, tiles_n = 0;
    int64_t grid = 0;
    int64_t ws_ld = 0;
    int64_t ws_bytes = 0;
    // Tail split: the last tail_rows tile rows of every batch entry run as
    // a separate split-K problem with tail_splits slices of tail_k_split,
    // so that a last, mostly idle wave of whole tiles becomes one wave of
    // partial tiles; the rows above run as whole tiles (grid counts them).
    int tail_rows = 0;
    int tail_splits = 1;
    int64_t tail_k_split = 0;
    int64_t tail_grid = 0;
    // Persistent one-k-tile kernel (K <= kOneK, 128 x 128 tiles, `grid`
    // workgroups walking tiles_m * tiles_n * batch tiles).
    bool onek = false;
    // The 256 tile of TN operands with direct loads and 16-byte output rows
    // runs on four waves, one per SIMD (2 x 2 quadrants of 128 x 128),
    // instead of eight.
    bool four_wave = false;
};

constexpr int64_t kOneK = 64;           // deepest K the one-k-tile kernel takes
constexpr int64_t kOneKMinTiles = 512;  // fewer tiles: one per workgroup

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Cost model for problems with K of at least kModelMinK and 16-byte loads:
// the estimated time, in microseconds, of a tile and split-K choice (on the
// 256 tile unsplit, with its tail split, tail_split_of).  Fitted on TN
// operands; the other layouts' kernels rank the choices alike.
//   - A workgroup costs kKtileUs[tile] per k-tile of its slice plus
//     kFixedUs[tile] (its first loads and its epilogue); the 64 tile's
//     split-K slices run on another kernel (four stages of 64-deep
//     k-tiles), at kKtileUs64Split per k-tile.
//   - On the 256 tile (one workgroup per CU) a wave costs one workgroup's
//     time, and a last wave holding a fraction f of the CUs' workgroups
//     kShortWave[tile] + (1 - kShortWave[tile]) * f of it: with fewer CUs
//     busy the chip holds a higher clock.
//   - On the 128 and 64 tiles (two per CU) a CU holding L workgroups takes
//     L / 2 workgroup times, plus kShortWave[tile] of one for an odd L (a
//     workgroup alone on its CU).
//   - A split adds kReduceUs (the reduction's launch), kReduceSliceUs per
//     slice (each reduction thread reads the slices eight at a time), and
//     the write and read-back of its fp32 partials at kPartialBytesPerUs.
// The constants are a least-squares fit, on the log of the time, to 886
// timed tile / split choices on 42 shapes from 64^2 x 65536 to 3072^2 x
// 4096.  Timed again with `bench.py --plan-grid`, the least estimate's
// choice is 2.9 % slower than the fastest on average over those shapes (18 %
// at worst, 512^2 x 2048) and as fast as the fastest over 20 other shapes
// up to 3072^2 x 8192; the rules used before were 17 % and 25 % slower on
// average (71 % and 111 % at worst).
constexpr int64_t kModelMinK = 512;     // eight k-tiles
constexpr int64_t kModelMinSliceK = 512;   // eight k-tiles per slice at least
// Split factors tried: every one to 16, then about four per octave to 512.
constexpr int kModelSplits[] = {1,  2,  3,  4,   5,   6,   7,   8,   9,
                                10, 11, 12, 13,  14,  15,  16,  20,  24,
                                28, 32, 40, 48,  56,  64,  80,  96,  112,
                                128, 160, 192, 224, 256, 320, 384, 448, 512};
constexpr double kKtileUs[NUM_TILES] = {1.250, 0.805, 0.384};
constexpr double kKtileUs64Split = 0.357;
constexpr double kFixedUs[NUM_TILES] = {5.88, 3.64, 1.57};
constexpr double kShortWave[NUM_TILES] = {0.739, 0.665, 0.729};
constexpr double kReduceUs = 5.48;
constexpr double kReduceSliceUs = 0.0888;
constexpr double kPartialBytesPerUs = 8.40e6;
// Largest split-K workspace the model plans for: the fixed scratch of the
// no-allocation entry point, so that both entry points plan alike.
constexpr int64_t kModelMaxPartialBytes = GEMM_TN_NOALLOC_SCRATCH_BYTES;

// Bytes of fp32 partials a split into `splits` slices writes (rows padded
// to four elements, as the workspace lays them out).
inline int64_t partial_bytes(int64_t batch, int64_t M, int64_t N,
                             int64_t splits)
{
    return splits * batch * M * (cdiv(N, 4) * 4) * 4;
}

// Tail split of a grid of whole tiles.  With whole tiles only, a last wave
// holding less than half a wave's tiles (a wave: every CU running as many
// workgroups as fit) leaves most CUs idle for a whole tile's time.  Instead
// the fewest bottom tile rows that hold that remainder are split along K
// (at least four k-tiles per slice, at most a wave of workgroups), and the
// rows above run as whole tiles.  More slices shorten the tail's compute
// (about a tile's time / slices) but each adds a round trip of fp32
// partials for every tail tile (written, then read by the reduction): about
// sqrt(9 * k-tiles / tail tiles) slices balance the two.  Measured on the
// 256 tile at K = 4096 (interleaved medians): 4352^2, 34 tail tiles: 142.7
// / 140.7 / 141.5 / 142.7 / 146.2 us for 3 / 4 / 5 / 6 / 7 slices (the
// formula: 4); 6144^2, 72 tail tiles: 255.8 / 253.8 us for 2 / 3 (the
// formula: 3).  Taken only for tiles that run one workgroup per CU: where
// two fit, the last wave's tiles run at twice the speed, and measured on
// 3072^3 (128 tiles) the extra launch and reduction cost more than the tail
// they save.  force_rows >= 0 and force_splits >= 2 override the choice;
// rows = 0 means no tail split.
struct TailSplit {
    int rows = 0;
    int64_t splits = 1;
    int64_t k_split = 0;
};

inline TailSplit tail_split_of(int tile, int64_t batch, int64_t tiles_m,
                               int64_t tiles_n, int64_t K, int force_rows,
                               int force_splits)
{
    TailSplit t;
    const int64_t row_tiles = tiles_n * batch;
    const int64_t ntiles = tiles_m * row_tiles;
    const int64_t slots = (int64_t)kCUs * kTileWgsPerCu[tile];
    const int64_t full = ntiles / slots, rem = ntiles % slots;
    int64_t rows = 0;
    if (kTileWgsPerCu[tile] == 1 && full >= 1 && rem > 0 && rem <= slots / 2)
        rows = cdiv(rem, row_tiles);
    if (force_rows >= 0)
        rows = force_rows;
    if (rows <= 0 || rows >= tiles_m)
        return t;
    const int64_t tail_tiles = rows * row_tiles;
    int64_t ts = slots / tail_tiles;
    const int64_t ktiles = cdiv(K, kBK);
    int64_t balance = 1;                // round(sqrt(9 * ktiles / tail_tiles))
    while ((2 * balance + 1) * (2 * balance + 1) * tail_tiles <= 36 * ktiles)
        ++balance;
    if (balance < ts)
        ts = balance;
    if (force_splits >= 2)
        ts = force_splits;
    const int64_t max_splits = K / (4 * kBK) > 1 ? K / (4 * kBK) : 1;
    if (ts > max_splits)
        ts = max_splits;
    if (ts < 2)
        return t;
    const int64_t k_split = cdiv(cdiv(K, ts), kBK) * kBK;
    ts = cdiv(K, k_split);
    if (ts < 2)
        return t;
    t.rows = (int)rows;
    t.splits = ts;
    t.k_split = k_split;
    return t;
}

// Estimated time of `wgs` workgroups of `ktiles` k-tiles each on `tile`
// (split_kernel: the split-K instantiation, which differs on the 64 tile).
inline double waves_us(int tile, int64_t wgs, int64_t ktiles,
                       bool split_kernel)
{
    const double per_k = tile == TILE_64 && split_kernel ? kKtileUs64Split
                                                          : kKtileUs[tile];
    const double wg_us = (double)ktiles * per_k + kFixedUs[tile];
    double waves;
    if (kTileWgsPerCu[tile] == 1) {
        waves = (double)(wgs / kCUs);
        if (wgs % kCUs != 0)
            waves += kShortWave[tile] + (1.0 - kShortWave[tile]) *
                                            (double)(wgs % kCUs) / kCUs;
    } else {
        const int64_t per_cu = cdiv(wgs, kCUs);
        waves = (double)(per_cu / 2) + (per_cu % 2 ? kShortWave[tile] : 0.0);
    }
    return waves * wg_us;
}

// Estimated time of the reduction of `slices` slices of `bytes` of partials.
inline double reduce_us(int64_t slices, int64_t bytes)
{
    return kReduceUs + kReduceSliceUs * (double)slices +
           2.0 * (double)bytes / kPartialBytesPerUs;
}

// Estimated time of `tile` with K in `splits` slices; with one slice on a
// tile that takes a tail split (force_tail_rows as in tail_split_of), of
// the whole tiles above the tail, the tail's slices, and their reduction.
inline double estimate_us(int tile, int64_t batch, int64_t M, int64_t N,
                          int64_t K, int64_t splits, int force_tail_rows)
{
    const int64_t dim = kTileDim[tile];
    const int64_t tiles_m = cdiv(M, dim), tiles_n = cdiv(N, dim);
    const int64_t ntiles = tiles_m * tiles_n * batch;
    const int64_t ktiles = cdiv(cdiv(K, splits), kBK);
    const int64_t slices = cdiv(K, ktiles * kBK);
    if (slices == 1) {
        const TailSplit t = tail_split_of(tile, batch, tiles_m, tiles_n, K,
                                          force_tail_rows, -1);
        if (t.rows > 0) {
            const int64_t tail_tiles = t.rows * tiles_n * batch;
            const int64_t tail_m = M - (tiles_m - t.rows) * dim;
            return waves_us(tile, ntiles - tail_tiles, ktiles, false) +
                   waves_us(tile, tail_tiles * t.splits,
                            t.k_split / kBK, true) +
                   reduce_us(t.splits, t.splits * batch * tail_m *
                                           (cdiv(N, 4) * 4) * 4);
        }
    }
    return waves_us(tile, ntiles * slices, ktiles, slices > 1) +
           (slices > 1 ? reduce_us(slices,
                                   partial_bytes(batch, M, N, slices))
                       : 0.0);
}

// Tile and split-K factor of least estimated time, among the tiles set in
// tile_mask (bit t: tile t has a kernel for the operands' layout).  The
// 256 tile is tried when M and N are at least 256; splits while the slices
// keep kModelMinSliceK and the partials fit in kModelMaxPartialBytes; a
// factor that rounds to the slices of a smaller one is skipped.  Returns
// false (and leaves tile and splits) when no tile is allowed.
inline bool choose_by_cost(int64_t batch, int64_t M, int64_t N, int64_t K,
                           int force_tail_rows, unsigned tile_mask,
                           int *tile, int64_t *splits)
{
    if (M < 256 || N < 256)
        tile_mask &= ~(1u << TILE_256);
    double best = 0.0;
    bool found = false;
    for (int t = 0; t < NUM_TILES; ++t) {
        if (!((tile_mask >> t) & 1u))
            continue;
        for (const int s : kModelSplits) {
            if (s > 1 && s * kModelMinSliceK > K)
                break;
            if (cdiv(K, cdiv(cdiv(K, s), kBK) * kBK) != s)
                continue;
            if (s > 1 && partial_bytes(batch, M, N, s) > kModelMaxPartialBytes)
                break;
            const double us =
                estimate_us(t, batch, M, N, K, s, force_tail_rows);
            if (!found || us < best) {
                best = us;
                found = true;
                *tile = t;
                *splits = s;
            }
        }
    }
    return found;
}

inline bool mul_ok(int64_t a, int64_t b, int64_t *out)
{
    return !__builtin_mul_overflow(a, b, out);
}

// Row strides (in elements) of the four matrices, and whether A (B) is
// stored K x M (K x N) row-major -- contiguous along M (N) -- instead of
// M x K (N x K).
struct Lds {
    int64_t a, b, c, d;
    bool a_mn = false, b_mn = false;
};

// Size, stride and dtype checks (no pointers involved).  Every row stride
// is at least its row length; batches of D may not overlap.
inline int check_sizes(int64_t batch, int64_t M, int64_t N, int64_t K,
                       const Lds &ld, int64_t sA, int64_t sB, int64_t sC,
                       int64_t sD, int d_dtype)
{
    if (batch < 0 || M < 0 || N < 0 || K < 0)
        return GEMM_TN_ERR_INVALID_ARG;
    if (d_dtype != GEMM_TN_F16 && d_dtype != GEMM_TN_F32)
        return GEMM_TN_ERR_INVALID_ARG;
    if (sA < 0 || sB < 0 || sC < 0 || sD < 0)
        return GEMM_TN_ERR_INVALID_ARG;
    // Stored rows and row lengths of A and B.
    const int64_t a_rows = ld.a_mn ? K : M, a_len = ld.a_mn ? M : K;
    const int64_t b_rows = ld.b_mn ? K : N, b_len = ld.b_mn ? N : K;
    if (ld.a < a_len || ld.b < b_len || ld.c < N || ld.d < N)
        return GEMM_TN_ERR_INVALID_ARG;
    // Element extents of one matrix: (rows - 1) * ld + row length.
    int64_t ea, eb, ed, t;
    auto extent = [&](int64_t rows, int64_t l, int64_t len, int64_t *out) {
        if (rows == 0 || len == 0) {
            *out = 0;
            return true;
        }
        return mul_ok(rows - 1, l, out) && !__builtin_add_overflow(*out, len, out);
    };
    if (!extent(a_rows, ld.a, a_len, &ea) ||
        !extent(b_rows, ld.b, b_len, &eb) || !extent(M, ld.d, N, &ed) ||
        !extent(M, ld.c, N, &t))
        return GEMM_TN_ERR_INVALID_ARG;
    if (ea > t)
        t = ea;
    if (eb > t)
        t = eb;
    if (ed > t)
        t = ed;
    if (!mul_ok(t, 4, &t))
        return GEMM_TN_ERR_INVALID_ARG;
    if (batch > 1) {
        if (sD < ed)
            return GEMM_TN_ERR_INVALID_ARG;  // batches of D would overlap
        const int64_t strides[4] = {sA, sB, sC, sD};
        for (int i = 0; i < 4; ++i) {
            int64_t span;
            if (!mul_ok(strides[i], batch - 1, &span) ||
                __builtin_add_overflow(span, ea + eb + ed, &span) ||
                !mul_ok(span, 4, &span))
                return GEMM_TN_ERR_INVALID_ARG;
        }
    }
    if (batch == 0 || M == 0 || N == 0)
        return GEMM_TN_OK;
    if (K > kMaxK || N > kMaxN || M > kMaxM)
        return GEMM_TN_ERR_UNSUPPORTED;
    if (ld.a > kMaxK || ld.b > kMaxK || ld.c > kMaxN || ld.d > kMaxN)
        return GEMM_TN_ERR_UNSUPPORTED;
    return GEMM_TN_OK;
}

inline int check_pointers(int64_t M, int64_t N, int64_t K, const void *A,
                          const void *B, float beta, const void *C,
                          const void *D)
{
    if (M == 0 || N == 0)
        return GEMM_TN_OK;
    if (D == nullptr)
        return GEMM_TN_ERR_INVALID_ARG;
    if (K > 0 && (A == nullptr || B == nullptr))
        return GEMM_TN_ERR_INVALID_ARG;
    if (beta != 0.0f && C == nullptr)
        return GEMM_TN_ERR_INVALID_ARG;
    return GEMM_TN_OK;
}

// Optional override for tuning sweeps and tests: "tile=256|128|64,
// loader=0|1|2,split=S,group=G,tail=R,tail_split=T,onek=0|1,w4=0|1" (any
// subset, comma separated; tail=0 turns the tail split off; onek=1 takes
// the persistent one-k-tile kernel wherever it applies, onek=0 never; w4=0
// runs the 256 tile of TN operands on eight waves).  Unknown keys are
// ignored; a loader that the operands' alignment does not allow is ignored.
struct Override {
    int tile = -1, loader = -1, split = -1, group = -1, tail = -1,
        tail_split = -1, onek = -1, w4 = -1;
};

inline Override parse_override(const char *s)
{
    Override o;
    if (s == nullptr)
        return o;
    char buf[256];
    strncpy(buf, s, sizeof buf - 1);
    buf[sizeof buf - 1] = 0;
    char *save = nullptr;   // strtok_r: calls may come from several threads
    for (char *tok = strtok_r(buf, ",", &save); tok;
         tok = strtok_r(nullptr, ",", &save)) {
        char *eq = strchr(tok, '=');
        if (!eq)
            continue;
        *eq = 0;
        const int v = atoi(eq + 1);
        if (!strcmp(tok, "tile"))
            o.tile = v == 256 ? TILE_256 : v == 128 ? TILE_128
                   : v == 64  ? TILE_64  : -1;
        else if (!strcmp(tok, "loader"))
            o.loader = (v >= 0 && v <= 2) ? v : -1;
        else if (!strcmp(tok, "split"))
            o.split = v >= 1 ? v : -1;
        else if (!strcmp(tok, "group"))
            o.group = v >= 1 ? v : -1;
        else if (!strcmp(tok, "tail"))
            o.tail = v >= 0 ? v : -1;
        else if (!strcmp(tok, "tail_split"))
            o.tail_split = v >= 2 ? v : -1;
        else if (!strcmp(tok, "onek"))
            o.onek = v == 0 || v == 1 ? v : -1;
        else if (!strcmp(tok, "w4"))
            o.w4 = v == 0 || v == 1 ? v : -1;
    }
    return o;
}

// Choose the kernel configuration.  vec_in: A and B 16-byte aligned, their
// row lengths (K, or M / N when stored along M / N) and row and batch
// strides multiples of 8.  vec_out: every row of D
// (and of C when it is read) starts on a 16-byte boundary and holds a
// whole number of 16-byte chunks.
inline Plan make_plan(int64_t batch, int64_t M, int64_t N, int64_t K,
                      const Lds &ld, int64_t sA, int64_t sB, int64_t sC,
                      int64_t sD, int d_dtype, bool vec_in, bool vec_out,
                      const char *override_spec)
{
    Plan p;
    p.status = check_sizes(batch, M, N, K, ld, sA, sB, sC, sD, d_dtype);
    if (p.status != GEMM_TN_OK)
        return p;
    if (batch == 0 || M == 0 || N == 0) {
        p.noop = true;
        return p;
    }
    const Override o = parse_override(override_spec);

    auto tiles = [&](int t) {
        return cdiv(M, kTileDim[t]) * cdiv(N, kTileDim[t]) * batch;
    };
    // Largest tile that still gives every compute unit work.  The 256-wide
    // tile needs one 128 KiB LDS double buffer per CU, so it is used only
    // when there are about as many tiles as CUs and more than one k-tile.
    int tile;
    if (M >= 256 && N >= 256 && K > kBK && tiles(TILE_256) >= kCUs * 3 / 4)
        tile = TILE_256;
    else if (tiles(TILE_128) >= kCUs)
        tile = TILE_128;
    else
        tile = TILE_64;
    if (o.tile >= 0)
        tile = o.tile;
    // Operands stored along M / N: the loader that will run (direct when
    // the rows allow 16-byte loads) must have a kernel for this layout on
    // the tile, else the next smaller tile is taken.
    const int layout = (ld.a_mn ? 1 : 0) | (ld.b_mn ? 2 : 0);
    int loader = vec_in ? kDefaultVecLoader : PLAN_LOAD_ELEM;
    if (o.loader >= 0 && (vec_in || o.loader == PLAN_LOAD_ELEM))
        loader = o.loader;
    if (layout != 0 && loader == PLAN_LOAD_VREG)
        loader = PLAN_LOAD_ELEM;
    auto has_kernel = [&](int t) -> bool {
        if (loader == PLAN_LOAD_DIRECT)
            return ((kTileDirectLays[t] >> layout) & 1) != 0;
        if (loader == PLAN_LOAD_ELEM)
            return layout == 0 || kTileElemLays[t];
        return layout == 0;
    };
    while (!has_kernel(tile) && tile + 1 < NUM_TILES)
        ++tile;
    if (!has_kernel(tile) && loader == PLAN_LOAD_DIRECT) {
        loader = PLAN_LOAD_ELEM;     // no direct kernel for the layout
        tile = o.tile >= 0 ? o.tile : tile;
        while (!has_kernel(tile) && tile + 1 < NUM_TILES)
            ++tile;
    }
    // K of 512 or more with 16-byte loads, any layout: tile and split-K
    // factor from the cost model (a forced tile, split or tail split keeps
    // the rules above and below).
    int64_t model_splits = 0;
    if (o.tile < 0 && o.split < 1 && o.tail < 1 &&
        loader == PLAN_LOAD_DIRECT && K >= kModelMinK) {
        unsigned mask = 0;
        for (int t = 0; t < NUM_TILES; ++t)
            mask |= has_kernel(t) ? 1u << t : 0u;
        int mt = tile;
        int64_t ms = 0;
        if (choose_by_cost(batch, M, N, K, o.tail, mask, &mt, &ms)) {
            tile = mt;
            model_splits = ms;
        }
    }
    // K within one k-tile, many tiles, 16-byte loads and stores: the
    // persistent one-k-tile kernel (128 x 128 tiles), which keeps the next
    // tile's operands in flight while a tile's results are written.
    {
        const int64_t t128 = tiles(TILE_128);
        const bool able = K > 0 && K <= kOneK && layout == 0 &&
                          loader == PLAN_LOAD_DIRECT && vec_out &&
                          o.split < 2 && o.tail < 1;
        const bool want = o.onek >= 0 ? o.onek == 1
                                      : o.tile < 0 && t128 >= kOneKMinTiles;
        if (able && want) {
            p.onek = true;
            p.tile = TILE_128;
            p.bm = p.bn = 128;
            p.loader = loader;
            p.vec_out = true;
            p.tiles_m = (int)cdiv(M, 128);
            p.tiles_n = (int)cdiv(N, 128);
            p.splits = 1;
            p.k_split = kBK;
            p.group_m = 1;
            p.grid = t128 < kCUs ? t128 : kCUs;
            return p;
        }
    }
    p.tile = tile;
    p.bm = p.bn = kTileDim[tile];
    p.tiles_m = (int)cdiv(M, p.bm);
    p.tiles_n = (int)cdiv(N, p.bn);
    const int64_t ntiles = (int64_t)p.tiles_m * p.tiles_n * batch;

    // Split K when the tiles alone leave CUs idle and K is long: as many
    // slices as one wave of the tile holds (at least four k-tiles each).
    int64_t splits = 1;
    if (model_splits > 0)
        splits = model_splits;
    else if (ntiles < kCUs && K >= 1024) {
        const int64_t wave = (int64_t)kCUs * kTileWgsPerCu[tile];
        splits = wave / ntiles > 1 ? wave / ntiles : 1;
    }
    if (o.split >= 1)
        splits = o.split;
    else if (o.tail >= 1)
        splits = 1;      // a forced tail split replaces the whole-K split
    const int64_t max_splits = K / (4 * kBK) > 1 ? K / (4 * kBK) : 1;
    if (splits > max_splits)
        splits = max_splits;
    if (splits > 1) {
        p.k_split = cdiv(cdiv(K, splits), kBK) * kBK;
        splits = cdiv(K, p.k_split);
    }
    p.splits = (int)splits;
    if (p.splits == 1)
        p.k_split = cdiv(K, kBK) * kBK;

    p.loader = loader;
    p.four_wave = tile == TILE_256 && loader == PLAN_LOAD_DIRECT &&
                  layout == 0 && vec_out && o.w4 != 0;
    p.a_mn = ld.a_mn;
    p.b_mn = ld.b_mn;
    p.layout = layout;
    p.vec_out = vec_out;
    p.group_m = tile == TILE_256 ? 4 : 8;
    // With one or two k-tiles the operands are small next to D and the
    // writes of D dominate: tiles in row order, so that consecutive tiles
    // of an XCD write neighbouring pieces of the same rows (the batched
    // 1024 x 1024 x 64 score product: 47.2 against 49.4 us with groups of
    // 8 tile rows).
    if (K <= 2 * kBK)
        p.group_m = 1;
    if (o.group >= 1)
        p.group_m = o.group;

    // Tail split (tail_split_of) of a grid of whole tiles.
    const int64_t row_tiles = (int64_t)p.tiles_n * batch;
    if (p.splits == 1) {
        const TailSplit t = tail_split_of(tile, batch, p.tiles_m, p.tiles_n,
                                          K, o.tail, o.tail_split);
        if (t.rows > 0) {
            p.tail_rows = t.rows;
            p.tail_splits = (int)t.splits;
            p.tail_k_split = t.k_split;
            p.tail_grid = t.rows * row_tiles * t.splits;
        }
    }

    p.grid = (ntiles - (int64_t)p.tail_rows * row_tiles) * p.splits;
    if (p.grid + p.tail_grid > 0x7FFFFFFF) {
        p.status = GEMM_TN_ERR_UNSUPPORTED;
        return p;
    }
    if (p.splits > 1 || p.tail_rows > 0)
        p.ws_ld = cdiv(N, 4) * 4;
    if (p.splits > 1)
        p.ws_bytes = (int64_t)p.splits * batch * M * p.ws_ld * 4;
    if (p.tail_rows > 0) {
        const int64_t tail_m = M - (int64_t)(p.tiles_m - p.tail_rows) * p.bm;
        p.ws_bytes = (int64_t)p.tail_splits * batch * tail_m * p.ws_ld * 4;
    }
    (void)d_dtype;
    return p;
}

inline int describe_plan(const Plan &p, char *buf, int64_t buflen)
{
    static const char *loaders[] = {"direct", "vreg", "elem"};
    static const char *scheds[] = {"interleaved", "pingpong", "pingpong-split"};
    if (buf == nullptr || buflen <= 0)
        return p.status;
    if (p.status != GEMM_TN_OK) {
        snprintf(buf, (size_t)buflen, "error:%d", p.status);
        return p.status;
    }
    if (p.noop) {
        snprintf(buf, (size_t)buflen, "noop");
        return p.status;
    }
    if (p.onek) {
        snprintf(buf, (size_t)buflen,
                 "tile=128x128x64 stages=2 waves=2x2 mfma=16x16 "
                 "sched=persistent-onek loader=direct a_along=k b_along=k "
                 "split=1 k_split=64 vec_out=1 group_m=1 grid=%lld "
                 "tail_rows=0 tail_split=1 tail_k_split=0 tail_grid=0",
                 (long long)p.grid);
        return p.status;
    }
    snprintf(buf, (size_t)buflen,
             "tile=%dx%dx%d stages=%d waves=%dx%d mfma=%dx%d sched=%s "
             "loader=%s a_along=%s b_along=%s split=%d k_split=%lld "
             "vec_out=%d group_m=%d grid=%lld tail_rows=%d tail_split=%d "
             "tail_k_split=%lld tail_grid=%lld",
             p.bm, p.bn,
             p.splits > 1 ? kTileSplitBK[p.tile] : kTileBK[p.tile],
             p.splits > 1 ? kTileSplitStages[p.tile] : kTileStages[p.tile],
             p.four_wave ? 2 : kTileWM[p.tile],
             p.four_wave ? 2 : kTileWN[p.tile], kTileMfma[p.tile],
             kTileMfma[p.tile],
             p.four_wave                    ? "four-wave"
             : p.loader == PLAN_LOAD_DIRECT ? scheds[kTileSched[p.tile]]
                                            : "staged",
             loaders[p.loader], p.a_mn ? "m" : "k", p.b_mn ? "n" : "k",
             p.splits,
             (long long)p.k_split, p.vec_out ? 1 : 0, p.group_m,
             (long long)p.grid, p.tail_rows, p.tail_splits,
             (long long)p.tail_k_split, (long long)p.tail_grid);
    return p.status;
}

}  // namespace gtn
