// Host check of the kernels' LDS layouts (dense_gemm_fp16_amd/csrc/
// lds_layout.hpp, compiled here as plain C++).  For every tile shape the
// kernels instantiate, it checks:
//
//  * each swizzle is a bijection of a row's chunks (every LDS slot filled by
//    exactly one logical chunk, every logical chunk fetched once);
//  * every lane group of every LDS access reaches distinct banks, in the
//    model of gfx950's LDS the layouts were built for: 64 banks of 4 bytes,
//    128-bit accesses served 16 lanes at a time, 64-bit ones 32 lanes at a
//    time, 32- and 16-bit ones a whole wave (lanes reading the same word
//    share it);
//  * the transposing reads' per-lane base XOR 32 f, plus the k-step
//    offsets, equals the address the swizzle defines for each element of
//    every fragment (and likewise for the attention V tile);
//  * every 64- and 128-bit access is aligned to its size.
//
// The bank model follows page "cute(8) smem_gemm" (yuyanqi.com) section 3
// ("bank conflict" and its check in 3.7): lanes served in one cycle must
// not touch two different words of one bank.  Prints one line per failure
// (the first 40) and exits non-zero if any check fails.
#include <stdint.h>
#include <stdio.h>

#include "lds_layout.hpp"

using namespace gtn;

static long g_checks = 0, g_fail = 0;

static void fail(const char *what, int a, int b, int c, int d)
{
    if (g_fail++ < 40)
        fprintf(stderr, "FAIL %s (%d %d %d %d)\n", what, a, b, c, d);
}

// addr[l]: byte address of lane l's access of `bytes` bytes (one wave
// instruction).  Returns true when no lane group served together touches
// two different words of one bank.
static bool conflict_free(const uint32_t *addr, int bytes)
{
    const int per = bytes >= 16 ? 16 : bytes == 8 ? 32 : 64;
    const int words = bytes < 4 ? 1 : bytes / 4;
    for (int g0 = 0; g0 < 64; g0 += per) {
        int64_t word_of_bank[64];
        for (int b = 0; b < 64; ++b)
            word_of_bank[b] = -1;
        for (int l = g0; l < g0 + per; ++l)
            for (int w = 0; w < words; ++w) {
                const int64_t word = addr[l] / 4 + w;
                const int bank = (int)(word % 64);
                if (word_of_bank[bank] >= 0 && word_of_bank[bank] != word)
                    return false;
                word_of_bank[bank] = word;
            }
    }
    return true;
}

static void check_access(const uint32_t *addr, int bytes, const char *what,
                         int a, int b, int c, int d)
{
    ++g_checks;
    if (!conflict_free(addr, bytes))
        fail(what, a, b, c, d);
    if (bytes >= 8)
        for (int l = 0; l < 64; ++l)
            if (addr[l] % (uint32_t)(bytes > 16 ? 16 : bytes) != 0) {
                fail("misaligned access", a, b, c, d);
                break;
            }
}

template <typename F>
static void check_bijection(int chunks, F &&map, const char *what, int row)
{
    ++g_checks;
    bool seen[64] = {};
    for (int c = 0; c < chunks; ++c) {
        const int p = map(c);
        if (p < 0 || p >= chunks || seen[p]) {
            fail(what, row, c, p, chunks);
            return;
        }
        seen[p] = true;
    }
}

// ---- the GEMM tiles ------------------------------------------------------
// BM x BN x BK tile, WM x WN waves, MB x MB MFMA blocks.
template <int BM, int BN, int BK, int WM, int WN, int MB>
static void gemm_tile()
{
    constexpr int NW = WM * WN, NT = NW * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MI = WTM / MB, NI = WTN / MB;
    constexpr int KSTEPS = BK / (8 * (64 / MB));
    constexpr int CHUNKS = BK / 8;
    uint32_t addr[64];

    // K-contiguous tiles: the direct loader's lane lands in physical chunk
    // c of its row and fetches logical chunk swizzle_chunk(row, c).
    for (int row = 0; row < (BM > BN ? BM : BN); ++row)
        check_bijection(CHUNKS,
                        [&](int c) { return swizzle_chunk<BK>(row, c); },
                        "swizzle_chunk not a bijection", row);
    // Fragment reads (ds_read_b128), A rows then B rows of every wave.
    for (int w = 0; w < NW; ++w)
        for (int ks = 0; ks < KSTEPS; ++ks) {
            for (int i = 0; i < MI; ++i) {
                for (int l = 0; l < 64; ++l)
                    addr[l] = 2u * (uint32_t)tn_frag_offset<BK, MB>(
                                       (w / WN) * WTM + i * MB, l, ks);
                check_access(addr, 16, "A fragment read", BM, w, ks, i);
            }
            for (int j = 0; j < NI; ++j) {
                for (int l = 0; l < 64; ++l)
                    addr[l] = 2u * (uint32_t)tn_frag_offset<BK, MB>(
                                       (w % WN) * WTN + j * MB, l, ks);
                check_access(addr, 16, "B fragment read", BN, w, ks, j);
            }
        }
    // Every MB-row block starts where the swizzle repeats (16 rows), so a
    // block's fragment offsets are the first block's shifted by whole rows
    // (the four-wave kernel reads with one per-lane offset per k-step).
    if (MB == 16)
        for (int ks = 0; ks < KSTEPS; ++ks)
            for (int b = 0; b < (BM > BN ? BM : BN) / MB; ++b)
                for (int l = 0; l < 64; ++l) {
                    ++g_checks;
                    if (tn_frag_offset<BK, MB>(b * MB, l, ks) !=
                        b * MB * BK + tn_frag_offset<BK, MB>(0, l, ks))
                        fail("fragment offset not block-invariant", b, l, ks,
                             BK);
                }
    // Register-staged loaders: thread t writes chunk slot t of each block of
    // NT / CHUNKS rows (A rows first), 16 bytes to its swizzled chunk.
    constexpr int RB = NT / CHUNKS;
    for (int blk = 0; blk < (BM + BN) / RB; ++blk)
        for (int w = 0; w < NW; ++w) {
            for (int l = 0; l < 64; ++l) {
                const int t = w * 64 + l;
                const int row = blk * RB + t / CHUNKS;     // A rows, then B
                addr[l] = 2u * (uint32_t)(row * BK +
                                          swizzle_chunk<BK>(row, t % CHUNKS) *
                                              8);
            }
            check_access(addr, 16, "staged tile store", BM, blk, w, 0);
        }
}

// Operand tile stored along M (N): BK rows of k, W elements each, read by
// the transposing loads of a wave whose columns start at cbase, F
// fragments of 16 columns, KSTEPS k-steps of 32.
template <int W, int BK>
static void mn_tile(int cbase, int F)
{
    constexpr int CR = W / 8;
    uint32_t addr[64];
    for (int row = 0; row < BK; ++row)
        check_bijection(CR, [&](int c) { return swizzle_mn<CR>(row, c); },
                        "swizzle_mn not a bijection", row);
    // the kernels' LDS tiles start on 1 KiB boundaries
    for (uint32_t tile = 0; tile < 3 * 1024 * 64; tile += 1024 * 16)
        for (int f = 0; f < F; ++f)
            for (int ks = 0; ks < BK / 32; ++ks)
                for (int half = 0; half < 2; ++half) {
                    const uint32_t off = (uint32_t)((32 * ks + 4 * half) * W * 2);
                    for (int l = 0; l < 64; ++l) {
                        addr[l] =
                            ((tile + tr_read_offset<W>(l, cbase)) ^ (32u * f)) +
                            off;
                        // the element the swizzle puts there
                        const int row = 8 * (l >> 4) + ((l & 15) >> 2) +
                                        32 * ks + 4 * half;
                        const int col = cbase + 16 * f + 4 * (l & 3);
                        const uint32_t want =
                            tile + (uint32_t)(row * W * 2 +
                                              swizzle_mn<CR>(row, col / 8) * 16 +
                                              (col % 8) * 2);
                        ++g_checks;
                        if (addr[l] != want)
                            fail("transposing read address != layout", W, cbase,
                                 f, l);
                    }
                    check_access(addr, 8, "transposing read", W, cbase, f, ks);
                }
}

// Epilogue staging of a WTM x WTN wave sub-tile with ES-byte results.
template <int WTM, int WTN, int ES, int MB>
static void epilogue()
{
    constexpr int ROW_BYTES = WTN * ES, CPR = ROW_BYTES / 16;
    constexpr int QN = 64 / MB, G = MB * MB / 64 / 4;
    uint32_t addr[64];
    // writes in the accumulator layout: 4 consecutive n of one m per lane
    for (int ii = 0; ii < WTM / MB; ++ii)
        for (int j = 0; j < WTN / MB; ++j)
            for (int g = 0; g < G; ++g) {
                for (int l = 0; l < 64; ++l) {
                    const int r = ii * MB + l % MB;
                    const int col = j * MB + 4 * QN * g + (l / MB) * 4;
                    addr[l] = (uint32_t)stage_offset<ROW_BYTES>(r, col * ES);
                }
                check_access(addr, 4 * ES, "epilogue staging write", WTN, ES,
                             ii, j);
            }
    // 16-byte row reads, and their split into a periodic per-lane part and
    // a constant
    constexpr int P = stage_read_period<ROW_BYTES>();
    for (int it = 0; it < WTM * CPR / 64; ++it)
        for (int l = 0; l < 64; ++l) {
            ++g_checks;
            if (stage_read_offset<ROW_BYTES>(l, it) !=
                stage_read_offset<ROW_BYTES>(l, it % P) +
                    (it / P) * P * (64 / CPR) * ROW_BYTES)
                fail("staged row read offset not periodic", WTN, ES, it, l);
        }
    for (int it = 0; it < WTM * CPR / 64; ++it) {
        for (int l = 0; l < 64; ++l) {
            const int idx = it * 64 + l;
            addr[l] = (uint32_t)stage_offset<ROW_BYTES>(idx / CPR,
                                                        (idx % CPR) * 16);
        }
        check_access(addr, 16, "epilogue row read", WTN, ES, it, 0);
    }
    // element reads (rows without 16-byte alignment)
    for (int it = 0; it < WTM * WTN / 64; ++it) {
        for (int l = 0; l < 64; ++l) {
            const int idx = it * 64 + l;
            addr[l] =
                (uint32_t)stage_offset<ROW_BYTES>(idx / WTN, (idx % WTN) * ES);
        }
        check_access(addr, ES, "epilogue element read", WTN, ES, it, 0);
    }
    // every staged byte has one home in the wave's slice
    for (int r = 0; r < WTM; ++r)
        check_bijection(CPR,
                        [&](int c) { return stage_chunk<ROW_BYTES>(r, c); },
                        "stage_chunk not a bijection", r);
}

// ---- fp16-accumulating GEMM: 128 x 128 x 32, 2 x 2 waves, 16-row blocks,
// 4 k per lane ---------------------------------------------------------------
static void f16acc_tile()
{
    constexpr int BK = 32;
    uint32_t addr[64];
    for (int w = 0; w < 4; ++w)
        for (int s = 0; s < BK / 16; ++s)
            for (int i = 0; i < 4; ++i) {
                for (int l = 0; l < 64; ++l)
                    addr[l] = 2u * (uint32_t)tn_frag4_offset<BK>(
                                       (w / 2) * 64 + i * 16, l, s);
                check_access(addr, 8, "f16acc fragment read", w, s, i, 0);
            }
    // element loader: thread t writes chunk t & 3 of row t >> 2
    for (int x = 0; x < 2; ++x)
        for (int w = 0; w < 4; ++w) {
            for (int l = 0; l < 64; ++l) {
                const int slot = w * 64 + l + 256 * x;
                const int row = slot >> 2;
                addr[l] = 2u * (uint32_t)(row * BK +
                                          swizzle_chunk<BK>(row, slot & 3) * 8);
            }
            check_access(addr, 16, "f16acc staged store", x, w, 0, 0);
        }
}

// ---- attention: K tile like a GEMM operand; V tile with transposing reads;
// O staged in the epilogue layout -------------------------------------------------
template <int ES>
static void attention()
{
    constexpr int D = 64, BN = 64, MI = 2;
    uint32_t addr[64];
    for (int s = 0; s < D / 32; ++s)
        for (int j = 0; j < BN / 16; ++j) {
            for (int l = 0; l < 64; ++l)
                addr[l] = 2u * (uint32_t)tn_frag_offset<D, 16>(j * 16, l, s);
            check_access(addr, 16, "attention K read", s, j, 0, 0);
        }
    for (int row = 0; row < BN; ++row)
        check_bijection(8, [&](int c) { return c ^ v_swizzle(row); },
                        "v_swizzle not a bijection", row);
    for (int dj = 0; dj < D / 16; ++dj)
        for (int t = 0; t < 4; ++t) {
            for (int l = 0; l < 64; ++l) {
                addr[l] = v_read_offset<D>(l, dj) + (uint32_t)(16 * t * D * 2);
                const int row = 4 * (l >> 4) + ((l & 15) >> 2) + 16 * t;
                const int col = dj * 16 + 4 * (l & 3);
                const uint32_t want = (uint32_t)(
                    (row * D + ((col >> 3) ^ v_swizzle(row)) * 8 + (col & 7)) *
                    2);
                ++g_checks;
                if (addr[l] != want)
                    fail("V read address != layout", dj, t, l, 0);
            }
            check_access(addr, 8, "attention V read", dj, t, 0, 0);
        }
    for (int i = 0; i < MI; ++i)
        for (int dj = 0; dj < D / 16; ++dj) {
            for (int l = 0; l < 64; ++l)
                addr[l] = (uint32_t)stage_offset<D * ES>(
                    i * 16 + (l & 15), (dj * 16 + 4 * (l >> 4)) * ES);
            check_access(addr, 4 * ES, "attention O staging write", ES, i, dj,
                         0);
        }
    constexpr int LPR = D * ES / 16, RPI = 64 / LPR;
    for (int it = 0; it < MI * 16 / RPI; ++it) {
        for (int l = 0; l < 64; ++l)
            addr[l] = (uint32_t)stage_offset<D * ES>(it * RPI + l / LPR,
                                                     (l % LPR) * 16);
        check_access(addr, 16, "attention O row read", ES, it, 0, 0);
    }
}

// ---- fp32 transpose, 64 x 64 words, 256 threads ---------------------------
static void transpose()
{
    constexpr int T = 64;
    uint32_t addr[64];
    for (int i = 0; i < T; ++i)
        check_bijection(T, [&](int j) { return transpose_word<T>(i, j) - i * T; },
                        "transpose row not a bijection", i);
    for (int w = 0; w < 4; ++w)
        for (int k = 0; k < 4; ++k)
            for (int e = 0; e < 4; ++e) {
                for (int l = 0; l < 64; ++l) {
                    const int t = w * 64 + l;
                    addr[l] = 4u * (uint32_t)transpose_word<T>(t / 16 + 16 * k,
                                                               4 * (t % 16) + e);
                }
                check_access(addr, 4, "transpose tile write", w, k, e, 0);
                for (int l = 0; l < 64; ++l) {
                    const int t = w * 64 + l;
                    addr[l] = 4u * (uint32_t)transpose_word<T>(4 * (t % 16) + e,
                                                               t / 16 + 16 * k);
                }
                check_access(addr, 4, "transpose tile read", w, k, e, 0);
            }
}

int main()
{
    // GEMM tiles as instantiated (16 x 16 MFMA blocks) and the 32 x 32
    // alternative the tiles can be built with.
    gemm_tile<256, 256, 64, 2, 4, 16>();
    gemm_tile<256, 256, 64, 2, 2, 16>();      // four waves, 128 x 128 each
    gemm_tile<128, 128, 64, 2, 2, 16>();
    gemm_tile<64, 64, 64, 2, 2, 16>();
    gemm_tile<256, 256, 64, 2, 4, 32>();
    gemm_tile<128, 128, 64, 2, 2, 32>();
    gemm_tile<64, 64, 64, 2, 2, 32>();
    gemm_tile<128, 128, 32, 2, 2, 16>();
    gemm_tile<64, 64, 128, 2, 2, 16>();       // 256-byte rows
    // Operands stored along M / N: A (W = BM, a wave's rows at wm * WTM,
    // MI fragments) and B (W = BN, columns at wn * WTN, NI fragments).
    for (int wm = 0; wm < 2; ++wm)
        mn_tile<256, 64>(wm * 128, 8);
    for (int wn = 0; wn < 4; ++wn)
        mn_tile<256, 64>(wn * 64, 4);
    for (int w = 0; w < 2; ++w) {
        mn_tile<128, 64>(w * 64, 4);
        mn_tile<64, 64>(w * 32, 2);
        mn_tile<64, 128>(w * 32, 2);          // 128 k-rows
    }
    // Epilogue staging: wave sub-tiles of the 256 tile on eight and on four
    // waves (128 x 64, 128 x 128), the 128 tile (64 x 64) and the 64 tile
    // (32 x 32), fp16, fp32 and split-K partials.
    epilogue<128, 64, 2, 16>();
    epilogue<128, 64, 4, 16>();
    epilogue<128, 128, 2, 16>();
    epilogue<128, 128, 4, 16>();
    epilogue<64, 64, 2, 16>();
    epilogue<64, 64, 4, 16>();
    epilogue<32, 32, 2, 16>();
    epilogue<32, 32, 4, 16>();
    f16acc_tile();
    attention<2>();
    attention<4>();
    transpose();
    printf("%ld checks, %ld failures\n", g_checks, g_fail);
    return g_fail == 0 ? 0 : 1;
}
