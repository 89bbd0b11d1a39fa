// LDS layouts of the GEMM, attention and transpose kernels, and the per-lane
// LDS addresses of their fragment reads: plain constexpr integer functions.
//
// Each tile keeps its rows whole and permutes 16-byte chunks within a row
// by an XOR with a function of the row (page "cute(8) smem_gemm",
// yuyanqi.com, section 3 "Swizzle 详解": Swizzle<B,M,S> XORs row bits into
// the column group so that the lanes served together reach distinct banks,
// with no padding).  The functions are chosen for gfx950's LDS: 64 banks of
// 4 bytes; a ds_read_b128 / ds_write_b128 is served 16 lanes (256 bytes) at
// a time, a 64-bit access 32 lanes at a time.
//
// Nothing here touches a HIP type or builtin: the kernels call these
// functions, and a host test compiles this header as ordinary C++ (with
// __host__ / __device__ defined empty) to check that every map is a
// bijection per row and that every lane group of every access reaches
// distinct bank slots.
#pragma once

#include <stdint.h>

namespace gtn {

// Tile with BK-element (2*BK-byte) rows, K contiguous.  A 256-byte line of
// LDS holds R = 128 / BK rows; XORing the chunk index with (row / R) mod
// CHUNKS makes the R rows of a line and the CHUNKS lines of a 16-row group
// land in distinct 16-byte slots for every logical chunk.  (Measured on
// MI355X: zero SQ_LDS_BANK_CONFLICT in the main loop with this map, half of
// all LDS cycles in conflict with row mod 8, the map a 32-bank LDS wants.)
template <int BK>
__device__ __host__ constexpr int swizzle_chunk(int row, int chunk)
{
    return chunk ^ ((row / (128 / BK)) % (BK / 8));
}

// Element offset (in halves) of the 16 bytes a lane reads for an MFMA
// fragment of an MB-row block whose first row is row0, at k-step ks of a
// K-contiguous tile: lane l takes row row0 + l % MB and k chunk
// ks * (64 / MB) + l / MB (8 consecutive k per lane, 64 / MB lanes across
// a k-step).
template <int BK, int MB>
__device__ __host__ constexpr int tn_frag_offset(int row0, int lane, int ks)
{
    return (row0 + lane % MB) * BK +
           swizzle_chunk<BK>(row0 + lane % MB, ks * (64 / MB) + lane / MB) * 8;
}

// The same for a 16x16x16 MFMA fragment (4 consecutive k per lane, 8
// bytes): lane l takes row row0 + l % 16 and k = 16 ks + 4 (l / 16).
template <int BK>
__device__ __host__ constexpr int tn_frag4_offset(int row0, int lane, int ks)
{
    return (row0 + lane % 16) * BK +
           swizzle_chunk<BK>(row0 + lane % 16, (16 * ks + 4 * (lane / 16)) >> 3) *
               8 +
           ((16 * ks + 4 * (lane / 16)) & 7);
}

// Tile of an operand stored along M (N): BK rows of k, each CR = W / 8
// chunks of 16 bytes (8 consecutive m).  Its fragments are read with
// ds_read_b64_tr_b16, where lane group g of a wave reads rows
// 8g + 4r + (0..3) of a k-step, 32 bytes each; a half wave thus touches 8
// rows {0..3, 8..11} (+4, +16, +32 ...) at one pair of chunks (c, c+1),
// and XORing the chunk with 2*h(row) (h distinct over those 8 rows, and
// kept below CR so the pair stays adjacent and in its 256-byte line) puts
// them in distinct bank slots.  With 128-byte rows two rows share a
// 256-byte line by parity, so h only has to separate rows of one parity.
template <int CR>
__device__ __host__ constexpr int swizzle_mn(int row, int chunk)
{
    static_assert(CR == 8 || CR % 16 == 0, "rows of 128 bytes or 256n");
    return CR >= 16
               ? chunk ^ (2 * ((row & 3) | (((row >> 3) & 1) << 2)))
               : chunk ^ (2 * (((row >> 1) & 1) | (((row >> 3) & 1) << 1)));
}

// Byte offset, within a W-element k-row tile, of the first of the two
// transposing reads that give a lane its 8 k of fragment 0 of the columns
// cbase .. cbase + 15 (k-step 0).  Lane i of 16-lane group g points at
// k-row 8g + i / 4, column cbase + 4 (i % 4); the second read is 4 rows
// further, and k-step s adds 32 s rows.  The swizzle reads row bits 0, 1
// and 3 only, which 32 s and 4 leave alone, so these offsets serve every
// read as constant offsets.  Fragment f (columns cbase + 16 f) sits at this
// offset XOR 32 f: its chunk pair is 2 f further, and 2 cbase, 32 f and the
// rest of the offset occupy disjoint bits, so the XOR with the swizzle
// commutes (checked for every tile, lane and fragment by the host test).
template <int W>
__device__ __host__ constexpr uint32_t tr_read_offset(int lane, int cbase)
{
    return (uint32_t)(((8 * ((lane & 63) >> 4) + ((lane & 15) >> 2)) * W) * 2) +
           (uint32_t)(16 * ((lane & 3) >> 1) + 8 * (lane & 1)) +
           (uint32_t)((2 * cbase) ^
                      (swizzle_mn<W / 8>(8 * ((lane & 63) >> 4) +
                                             ((lane & 15) >> 2),
                                         0) *
                       16));
}

// Epilogue staging of a wave's sub-tile: rows of ROW_BYTES bytes (a row of
// results in the staged type), written in the accumulator layout (16
// lanes, one per row, at one 8- or 16-byte column piece) and read back 16
// bytes per lane along the rows.  Chunk c of staged row r sits at chunk
// c ^ ((r / LINE_ROWS) % X), LINE_ROWS rows per 256-byte line, so that the
// rows written together spread over distinct slots.
template <int ROW_BYTES>
__device__ __host__ constexpr int stage_chunk(int r, int c)
{
    constexpr int CPR = ROW_BYTES / 16;
    constexpr int LINE_ROWS = ROW_BYTES >= 256 ? 1 : 256 / ROW_BYTES;
    constexpr int X = CPR < 16 ? CPR : 16;
    return c ^ ((r / LINE_ROWS) % X);
}

// Byte offset of byte column cb of staged row r.
template <int ROW_BYTES>
__device__ __host__ constexpr int stage_offset(int r, int cb)
{
    return r * ROW_BYTES + stage_chunk<ROW_BYTES>(r, cb / 16) * 16 + cb % 16;
}

// Row reads of the staging: read `it` of a wave takes 16 bytes at row
// it * RS + lane / CPR, chunk lane % CPR (RS = 64 / CPR rows per read).
template <int ROW_BYTES>
__device__ __host__ constexpr int stage_read_offset(int lane, int it)
{
    constexpr int CPR = ROW_BYTES / 16;
    return stage_offset<ROW_BYTES>(it * (64 / CPR) + lane / CPR,
                                   (lane % CPR) * 16);
}
// The swizzle term of those rows repeats every stage_read_period reads, so
// stage_read_offset(l, it) = stage_read_offset(l, it % P) +
// (it / P) * P * RS * ROW_BYTES: P address registers and constant offsets
// (checked on the host for every lane and read).
template <int ROW_BYTES>
__device__ __host__ constexpr int stage_read_period()
{
    constexpr int CPR = ROW_BYTES / 16;
    constexpr int RS = 64 / CPR;
    constexpr int LINE_ROWS = ROW_BYTES >= 256 ? 1 : 256 / ROW_BYTES;
    constexpr int X = CPR < 16 ? CPR : 16;
    static_assert(RS % LINE_ROWS == 0, "reads cover whole 256-byte lines");
    int a = X, b = RS / LINE_ROWS;          // P = X / gcd(X, RS / LINE_ROWS)
    while (b != 0) {
        const int t = a % b;
        a = b;
        b = t;
    }
    return X / a;
}

// V tile of the attention kernel (64-element = 128-byte rows of keys), read
// with ds_read_b64_tr_b16: a half wave reads 8 consecutive key rows at one
// pair of 16-byte chunks (c, c + 1), c even.  Rows of one parity share a
// 256-byte bank line; XORing the chunk with 2 * ((row / 2) % 4) puts the 4
// rows of each parity on distinct chunk pairs, so the 32 lanes hit 64
// distinct banks.
__device__ __host__ constexpr int v_swizzle(int row)
{
    return 2 * ((row >> 1) & 3);
}

// Byte offset, within a V tile of D-element rows, of a lane's first
// transposing read for column block dj: key row 4 (lane / 16) +
// (lane % 16) / 4, column 16 dj + 4 (lane % 4); the other reads of the
// block are 16, 32 and 48 rows further (constant offsets: the swizzle
// reads row bits 1-2 only).
template <int D>
__device__ __host__ constexpr uint32_t v_read_offset(int lane, int dj)
{
    return (uint32_t)(((4 * ((lane & 63) >> 4) + ((lane & 15) >> 2)) * D +
                       (((dj * 16 + 4 * (lane & 3)) >> 3) ^
                        v_swizzle(4 * ((lane & 63) >> 4) +
                                  ((lane & 15) >> 2))) *
                           8 +
                       ((dj * 16 + 4 * (lane & 3)) & 7)) *
                      2);
}

// fp32 transpose tile of T x T words: element (i, j) at row i, word j ^ i
// (page "Mat Transpose CuTe 版代码学习", chuoer47.github.io, version 3: an
// XOR of the column with the row in place of padding).
template <int T>
__device__ __host__ constexpr int transpose_word(int i, int j)
{
    return i * T + (j ^ i);
}

}  // namespace gtn
