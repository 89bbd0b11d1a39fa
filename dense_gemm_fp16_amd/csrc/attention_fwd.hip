// Attention forward pass O = softmax(scale * Q K^T) V for gfx950 (declared
// in include/attention_fwd.h), head dimension 64.
//
// The score product is the TN product of page "为什么
// cutlass_cute_tutorial_zh.md 中要用 retile_D" (blog.qingsen.net, sections
// 1-3: score = Q @ K.T, Q the A operand and K the B operand, fp32
// accumulation, head dimension 64, 64-query blocks in a FlashAttention-style
// tutorial).  Here the score tile never leaves the registers: each
// workgroup keeps 128 queries of one head and walks the keys in blocks of
// 64, with a running (online) softmax.
//
//  * Work: one workgroup of 4 waves per 128 queries of a head; each wave
//    owns 32 query rows (two 16-row MFMA blocks).  Workgroup ids are
//    remapped so the query blocks of a head run on one XCD and share its
//    L2 copy of K and V.
//  * Q: each wave loads its fragments once, straight from HBM into
//    registers (16 bytes per lane per 32-wide d-step).
//  * K, V: per key block, a 64 x 64 K tile and V tile go into LDS through
//    direct 16-byte buffer loads, two stages each.  Keys past Lk read as
//    zero.  The loop is software-pipelined: while the softmax of block kb
//    runs on the vector ALU, the MFMAs form the scores of block kb + 1, so
//    the K tiles run one block ahead of the V tiles.
//  * S = Q K^T: v_mfma_f32_16x16x32_f16 with the K fragment as the first
//    operand, so a lane holds query row (lane % 16) and keys
//    16j + 4(lane / 16) + e of each 16-key block j.
//  * Softmax: per-row maximum over the block (in-lane, then across the four
//    lanes that share a row), exp2 of the score times |scale| log2(e) minus
//    the shifted row maximum.  The row sums come from the MFMA too: one
//    more product of the fp16 probabilities with a fragment of ones leaves
//    each row's sum in every lane of that row.  The row shift moves
//    only when a new maximum exceeds it by more than 2^8 in probability
//    (then the accumulators are rescaled once); probabilities up to 2^8 stay
//    well inside fp16.
//  * P V: the probabilities, rounded to fp16, are already in the layout of
//    the MFMA's second operand once the 32 keys of a k-step are numbered
//    k-slot 8(lane/16) + x <-> key 4(lane/16) + x (x < 4), 16 + 4(lane/16)
//    + x - 4 (x >= 4).  V's fragment must use the same key order: two
//    ds_read_b64_tr_b16 reads of the V tile (rows = keys) give a lane 4
//    consecutive keys of one column each, at key offsets 4(lane/16) and
//    16 + 4(lane/16).
//  * Epilogue: each row is divided by its sum, rounded once to fp16 or
//    fp32, staged through LDS and stored as whole rows with the
//    non-temporal policy (O is written once); lse = |scale| * shift +
//    ln(sum).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attention_fwd.h"
#include "gemm_tn_kernels.hpp"

namespace gtn {
namespace {

constexpr int kBM = 128;        // queries per workgroup
constexpr int kBN = 64;         // keys per block
constexpr int kD = 64;          // head dimension
constexpr int kWaves = 4;
constexpr float kLazy = 8.0f;   // log2 headroom before the row shift moves
constexpr int64_t kMaxLk = int64_t(1) << 23;

struct AttnArgs {
    const _Float16 *Q, *K, *V;
    void *O;
    float *lse;
    int64_t Lq, Lk;
    float c;            // |scale| * log2(e)
    float scale_abs;
    uint32_t qsign;     // 0x80008000: Q's signs flipped for a negative scale
    int q_blocks, batch;
};

// The V tile's swizzle and read addresses are v_swizzle and
// v_read_offset (lds_layout.hpp).

__device__ inline f32x4 mfma16(const half8 &a, const half8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <typename OutT>
__global__ void __launch_bounds__(kWaves * 64) attn_fwd_kernel(AttnArgs p)
{
    constexpr int MI = kBM / kWaves / 16;   // 16-row query blocks per wave
    constexpr int NJ = kBN / 16;            // 16-key blocks per key block
    constexpr int DJ = kD / 16;             // 16-column blocks of O
    constexpr int DS = kD / 32;             // d-steps of the score product
    constexpr int KS = kBN / 32;            // key steps of the P V product
    constexpr int TILE = kBN * kD;          // halves per K or V tile
    // After the key loop the same LDS stages each wave's block of O: 32 rows
    // of 128 (fp16) or 256 (fp32) bytes in the GEMM epilogue's layout
    // (stage_offset), so that the 16 rows a lane group writes at one column,
    // and the rows a lane group reads back, fall on distinct banks.
    constexpr int ES = OutTraits<OutT>::bytes;
    constexpr int OROW = kD * ES;                           // bytes per row
    constexpr int OWAVE = MI * 16 * OROW;                   // bytes per wave
    constexpr int LDS_HALVES = (4 * TILE > kWaves * OWAVE / 2)
                                   ? 4 * TILE : kWaves * OWAVE / 2;
    __shared__ __attribute__((aligned(1024))) _Float16 lds[LDS_HALVES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, g = lane >> 4;

    // Workgroup id -> (head, query block); XCD x (= id mod 8) receives a
    // contiguous range of logical ids, so a head's query blocks share an L2.
    const int total = p.q_blocks * p.batch;
    const int wg = blockIdx.x;
    const int qq = total >> 3, rr = total & 7, x8 = wg & 7;
    const int logical = x8 * qq + (x8 < rr ? x8 : rr) + (wg >> 3);
    const int b = logical / p.q_blocks;
    const int qb = logical - b * p.q_blocks;
    const int64_t Lq = p.Lq, Lk = p.Lk;
    const int64_t q0 = (int64_t)qb * kBM + wave * (MI * 16);

    // ---- Q fragments: row q0 + 16i + lane % 16, d = 32s + 8(lane/16) ..
    const __amdgpu_buffer_rsrc_t rQ =
        make_rsrc(p.Q + (b * Lq + q0) * kD, (Lq - q0) * kD * 2);
    half8 qf[MI][DS];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int s = 0; s < DS; ++s) {
            const uint32_t off =
                (uint32_t)(((i * 16 + r16) * kD + 32 * s + 8 * g) * 2);
            u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rQ, off, 0, 0);
            v ^= p.qsign;
            qf[i][s] = __builtin_bit_cast(half8, v);
        }

    // ---- K / V tiles into LDS --------------------------------------------
    // LDS holds two stages of K tiles, then two of V tiles.  The K tiles
    // run one key block ahead of the V tiles (the scores of block kb + 1 are
    // formed while block kb is multiplied with V).  One 1 KiB load of a wave
    // fills 8 tile rows; lane l lands in physical chunk l % 8 of row l / 8
    // and fetches the logical chunk the tile's swizzle maps there.
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(p.K + b * Lk * kD, Lk * kD * 2);
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(p.V + b * Lk * kD, Lk * kD * 2);
    auto issue_tile = [&](auto v_tag, int stage, int kb) {
        constexpr bool IS_V = decltype(v_tag)::value;
        GTN_LDS _Float16 *base = (GTN_LDS _Float16 *)lds +
                                 (IS_V ? 2 * TILE : 0) + stage * TILE;
#pragma unroll
        for (int h = 0; h < kBN / 8 / kWaves; ++h) {
            const int grp = wave + kWaves * h;
            const int row = grp * 8 + (lane >> 3);
            const uint32_t roff = (uint32_t)(kb * kBN + row) * (kD * 2);
            const int ch = IS_V ? (lane & 7) ^ v_swizzle(row)
                                : swizzle_chunk<kD>(row, lane & 7);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                IS_V ? rV : rK, (GTN_LDS void *)(base + grp * 8 * kD), 16,
                roff + (uint32_t)ch * 16, 0, 0, 0);
        }
    };

    f32x4 oacc[MI][DJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < DJ; ++j)
            oacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Row sums: lacc[i] = ones * P^T accumulates, in each of its four
    // registers, the sum of row (lane % 16) of block i.
    f32x4 lacc[MI];
    float mref[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        mref[i] = 0.f;
        lacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};

    const int nblk = (int)((Lk + kBN - 1) / kBN);
    const int tail_keys = (int)(Lk - (int64_t)(nblk - 1) * kBN);   // 1..64
    const float c = p.c;

    // Scores of the key block in K stage `ks`.
    auto score = [&](int ks, f32x4 (&sacc)[MI][NJ]) {
        const _Float16 *sK = lds + ks * TILE;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                sacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DS; ++s)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const half8 kf = *(const half8 *)(
                    sK + tn_frag_offset<kD, 16>(j * 16, lane, s));
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    sacc[i][j] = mfma16(kf, qf[i][s], sacc[i][j]);
            }
    };
    // Row maxima of a block; with MASK, keys past Lk (in the last block)
    // are set to -inf first.  A row's 64 scores sit in the four lanes
    // l, l ^ 16, l ^ 32, l ^ 48; v_permlane32_swap / v_permlane16_swap of a
    // value with itself bring the other half (row) of the wave alongside,
    // so two swaps and two maxima finish the reduction in registers.  The
    // maxima are NaN-propagating (v_maximum3_f32): fmaxf's IEEE semantics
    // would first quiet every MFMA-produced input with one more vector
    // instruction.
    auto vmax = [](float a, float b) {
        return __builtin_elementwise_maximum(a, b);
    };
    auto rowmax = [&](auto mask_tag, f32x4 (&sacc)[MI][NJ], float (&mx)[MI]) {
        constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            if (MASK) {
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (j * 16 + 4 * g + e >= tail_keys)
                            sacc[i][j][e] = -INFINITY;
            }
            float m = sacc[i][0][0];
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    m = vmax(m, sacc[i][j][e]);
            const uint32_t mu = __builtin_bit_cast(uint32_t, m);
            const auto h32 = __builtin_amdgcn_permlane32_swap(mu, mu, false,
                                                              false);
            m = vmax(__builtin_bit_cast(float, (uint32_t)h32[0]),
                     __builtin_bit_cast(float, (uint32_t)h32[1]));
            const uint32_t mv = __builtin_bit_cast(uint32_t, m);
            const auto h16 = __builtin_amdgcn_permlane16_swap(mv, mv, false,
                                                              false);
            mx[i] = vmax(__builtin_bit_cast(float, (uint32_t)h16[0]),
                         __builtin_bit_cast(float, (uint32_t)h16[1]));
        }
    };
    // The row shift: set by the first block, moved (with a rescale of the
    // accumulators) only when a block maximum exceeds it by more than
    // kLazy / c.
    auto update_shift = [&](bool first, const float (&mx)[MI]) {
        if (first) {
#pragma unroll
            for (int i = 0; i < MI; ++i)
                mref[i] = mx[i];
            return;
        }
        bool need = false;
#pragma unroll
        for (int i = 0; i < MI; ++i)
            need |= (mx[i] - mref[i]) * c > kLazy;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const float mn = fmaxf(mref[i], mx[i]);
                const float f = __builtin_amdgcn_exp2f((mref[i] - mn) * c);
                mref[i] = mn;
                lacc[i] *= f;
#pragma unroll
                for (int j = 0; j < DJ; ++j)
                    oacc[i][j] *= f;
            }
        }
    };
    // Probabilities of a block as the fp16 fragments of the P V product.
    auto probs = [&](auto tail_tag, const f32x4 (&sacc)[MI][NJ],
                     half8 (&pf)[MI][KS]) {
        constexpr bool TAIL = decltype(tail_tag)::value;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const float mc = mref[i] * c;
            float pr[NJ][4];
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float pe = __builtin_amdgcn_exp2f(
                        __builtin_fmaf(sacc[i][j][e], c, -mc));
                    if (TAIL && j * 16 + 4 * g + e >= tail_keys)
                        pe = 0.f;
                    pr[j][e] = pe;
                }
#pragma unroll
            for (int t = 0; t < KS; ++t)
                pf[i][t] = half8{
                    (_Float16)pr[2 * t][0], (_Float16)pr[2 * t][1],
                    (_Float16)pr[2 * t][2], (_Float16)pr[2 * t][3],
                    (_Float16)pr[2 * t + 1][0], (_Float16)pr[2 * t + 1][1],
                    (_Float16)pr[2 * t + 1][2], (_Float16)pr[2 * t + 1][3]};
        }
    };
    // V fragments of the V tile in V stage `vs`: for column block dj and
    // key step t, two transposing reads at key rows 32t + 16r + 4(lane/16)
    // + (lane % 16) / 4, r = 0, 1, column 16 dj + 4 (lane % 4).  The row
    // swizzle depends only on bits 1-2 of the row, which t and r do not
    // change, so one address per dj serves all four reads (constant
    // offsets of 32 and 16 rows).
    const uint32_t lds_base = (uint32_t)(uintptr_t)(const GTN_LDS void *)lds;
    uint32_t v_addr[DJ];
#pragma unroll
    for (int dj = 0; dj < DJ; ++dj)
        v_addr[dj] = lds_base + (uint32_t)(2 * TILE * 2) +
                     v_read_offset<kD>(lane, dj);
    auto read_v = [&](int vs, u32x2 (&vr)[KS * DJ * 2]) {
        const uint32_t so = (uint32_t)(vs * TILE * 2);
#pragma unroll
        for (int dj = 0; dj < DJ; ++dj) {
            const uint32_t a = v_addr[dj] + so;
            vr[0 * DJ * 2 + dj * 2 + 0] = ds_read_tr_asm<0>(a);
            vr[0 * DJ * 2 + dj * 2 + 1] = ds_read_tr_asm<16 * kD * 2>(a);
            vr[1 * DJ * 2 + dj * 2 + 0] = ds_read_tr_asm<32 * kD * 2>(a);
            vr[1 * DJ * 2 + dj * 2 + 1] = ds_read_tr_asm<48 * kD * 2>(a);
        }
    };
    static_assert(KS == 2, "two key steps per block");
    // O += P V and the row sums, with the V fragments read by read_v.
    auto pv = [&](u32x2 (&vr)[KS * DJ * 2], const half8 (&pf)[MI][KS]) {
        lds_fence(vr);
#pragma unroll
        for (int t = 0; t < KS; ++t)
#pragma unroll
            for (int dj = 0; dj < DJ; ++dj) {
                const half4 lo = __builtin_bit_cast(half4, vr[t * DJ * 2 + dj * 2]);
                const half4 hi =
                    __builtin_bit_cast(half4, vr[t * DJ * 2 + dj * 2 + 1]);
                const half8 vf = {lo[0], lo[1], lo[2], lo[3],
                                  hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    oacc[i][dj] = mfma16(vf, pf[i][t], oacc[i][dj]);
            }
#pragma unroll
        for (int t = 0; t < KS; ++t)
#pragma unroll
            for (int i = 0; i < MI; ++i)
                lacc[i] = mfma16(ones, pf[i][t], lacc[i]);
    };

    // One pipelined step for key block kb < nblk - 1: `cur` holds its
    // scores (shift already applied to mref), `nxt` receives the scores of
    // block kb + 1 and their row maxima move the shift.  Two interleaved
    // phases: the MFMAs of the next scores with the exponentials of this
    // block, then the P V MFMAs of this block with the next row maxima.
    // The K tile of block kb + 1 is in K stage (kb + 1) & 1 and the V tile
    // of block kb in V stage kb & 1; the barrier orders both their arrival
    // (each wave waited for its own loads) and the reuse of the stages read
    // in the previous step.
    auto step = [&](auto mask_next_tag, int kb, f32x4 (&cur)[MI][NJ],
                    f32x4 (&nxt)[MI][NJ]) {
        wait_vmcnt<0>();
        wait_lgkmcnt<0>();
        block_sync();
        if (kb + 2 < nblk)
            issue_tile(Bool<false>{}, kb & 1, kb + 2);
        issue_tile(Bool<true>{}, (kb + 1) & 1, kb + 1);
        u32x2 vr[KS * DJ * 2];
        read_v(kb & 1, vr);
        half8 pf[MI][KS];
        __builtin_amdgcn_sched_barrier(0);
        score((kb + 1) & 1, nxt);
        probs(Bool<false>{}, cur, pf);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * DS * NJ / 2, 0);
#pragma unroll
        for (int x = 0; x < MI * NJ * DS; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        pv(vr, pf);
        float mx[MI];
        rowmax(mask_next_tag, nxt, mx);
#pragma unroll
        for (int x = 0; x < MI * (DJ + 1) * KS; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        update_shift(false, mx);
    };
    // The last block: no next scores.
    auto last = [&](f32x4 (&cur)[MI][NJ]) {
        wait_vmcnt<0>();
        wait_lgkmcnt<0>();
        block_sync();
        u32x2 vr[KS * DJ * 2];
        read_v((nblk - 1) & 1, vr);
        half8 pf[MI][KS];
        if (tail_keys < kBN)
            probs(Bool<true>{}, cur, pf);
        else
            probs(Bool<false>{}, cur, pf);
        pv(vr, pf);
    };

    // Prologue: K and V of block 0, K of block 1; scores and shift of
    // block 0.  Only Q and K of block 0 are waited for here (loads retire
    // in issue order, so vmcnt counts the V and K tiles issued after them);
    // the first step's wait covers the rest.
    constexpr int TILE_LOADS = kBN / 8 / kWaves;
    issue_tile(Bool<false>{}, 0, 0);
    issue_tile(Bool<true>{}, 0, 0);
    if (nblk > 1) {
        issue_tile(Bool<false>{}, 1, 1);
        wait_vmcnt<2 * TILE_LOADS>();
    } else {
        wait_vmcnt<TILE_LOADS>();
    }
    block_sync();
    f32x4 sa[MI][NJ], sb[MI][NJ];
    score(0, sa);
    {
        float mx[MI];
        if (nblk == 1 && tail_keys < kBN)
            rowmax(Bool<true>{}, sa, mx);
        else
            rowmax(Bool<false>{}, sa, mx);
        update_shift(true, mx);
    }
    // Steps 0 .. nblk - 2, unrolled by two so that the score tiles swap
    // roles without copies; the step before the last block masks the
    // last block's scores.
    const bool tail = tail_keys < kBN;
    int kb = 0;
    for (; kb + 2 < nblk - 1; kb += 2) {
        step(Bool<false>{}, kb, sa, sb);
        step(Bool<false>{}, kb + 1, sb, sa);
    }
    if (kb + 1 < nblk - 1) {
        // two steps left: kb (plain) and kb + 1 (before the last block)
        step(Bool<false>{}, kb, sa, sb);
        if (tail)
            step(Bool<true>{}, kb + 1, sb, sa);
        else
            step(Bool<false>{}, kb + 1, sb, sa);
        last(sa);
    } else if (kb + 1 == nblk - 1) {
        if (tail)
            step(Bool<true>{}, kb, sa, sb);
        else
            step(Bool<false>{}, kb, sa, sb);
        last(sb);
    } else {
        last(sa);
    }

    // ---- epilogue ----------------------------------------------------------
    // O / row sum, rounded once, into this wave's LDS block (every wave is
    // done with the K and V tiles after the barrier), then read back as
    // whole rows: each store instruction writes 8 (fp16) or 4 (fp32)
    // complete 128- or 256-byte rows of O instead of 32-byte pieces of 16.
    wait_lgkmcnt<0>();
    block_sync();
    char *ob = (char *)lds + wave * OWAVE;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const float l = lacc[i][0];
        const float inv = 1.0f / l;
#pragma unroll
        for (int dj = 0; dj < DJ; ++dj) {
            const f32x4 o = oacc[i][dj] * inv;
            char *dst = ob + stage_offset<OROW>(i * 16 + r16,
                                                (dj * 16 + 4 * g) * ES);
            if constexpr (ES == 2) {
                const half4 h = {(_Float16)o[0], (_Float16)o[1],
                                 (_Float16)o[2], (_Float16)o[3]};
                *(u32x2 *)dst = __builtin_bit_cast(u32x2, h);
            } else {
                *(f32x4 *)dst = o;
            }
        }
        const int64_t row = q0 + i * 16 + r16;
        if (p.lse != nullptr && g == 0 && row < Lq)
            p.lse[b * Lq + row] = p.scale_abs * mref[i] + logf(l);
    }
    wait_lgkmcnt<0>();
    asm volatile("" ::: "memory");
    const __amdgpu_buffer_rsrc_t rO =
        make_rsrc((char *)p.O + (b * Lq + q0) * kD * ES, (Lq - q0) * kD * ES);
    constexpr int LPR = kD * ES / 16;               // lanes per row
    constexpr int RPI = 64 / LPR;                   // rows per instruction
#pragma unroll
    for (int it = 0; it < MI * 16 / RPI; ++it) {
        const int row = it * RPI + lane / LPR, ch = lane % LPR;
        const u32x4 v = *(const u32x4 *)(ob + stage_offset<OROW>(row, ch * 16));
        __builtin_amdgcn_raw_buffer_store_b128(
            v, rO, (uint32_t)(row * kD * ES + ch * 16), 0, GTN_STORE_CPOL);
    }
}

bool overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na > 0 && nb > 0 && x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

}  // namespace
}  // namespace gtn

extern "C" int attention_fwd(int64_t batch, int64_t Lq, int64_t Lk,
                             int64_t d, float scale, const void *Q,
                             const void *K, const void *V, void *O,
                             int o_dtype, void *lse, void *stream)
{
    using namespace gtn;
    if (batch < 0 || Lq < 0 || Lk < 0 || d < 0)
        return GEMM_TN_ERR_INVALID_ARG;
    if (o_dtype != GEMM_TN_F16 && o_dtype != GEMM_TN_F32)
        return GEMM_TN_ERR_INVALID_ARG;
    if (!isfinite(scale))
        return GEMM_TN_ERR_INVALID_ARG;
    if (batch == 0 || Lq == 0)
        return GEMM_TN_OK;
    if (Lk == 0)
        return GEMM_TN_ERR_INVALID_ARG;
    if (Q == nullptr || K == nullptr || V == nullptr || O == nullptr)
        return GEMM_TN_ERR_INVALID_ARG;
    const int64_t es = o_dtype == GEMM_TN_F16 ? 2 : 4;
    int64_t nq, nk, bq, bk, bo, bl;
    if (__builtin_mul_overflow(batch, Lq, &nq) ||
        __builtin_mul_overflow(nq, d, &bq) ||
        __builtin_mul_overflow(bq, es, &bo) ||
        __builtin_mul_overflow(bq, (int64_t)2, &bq) ||
        __builtin_mul_overflow(nq, (int64_t)4, &bl) ||
        __builtin_mul_overflow(batch, Lk, &nk) ||
        __builtin_mul_overflow(nk, d, &bk) ||
        __builtin_mul_overflow(bk, (int64_t)2, &bk))
        return GEMM_TN_ERR_INVALID_ARG;
    if (overlap(O, bo, Q, bq) || overlap(O, bo, K, bk) ||
        overlap(O, bo, V, bk))
        return GEMM_TN_ERR_INVALID_ARG;
    if (lse != nullptr &&
        (overlap(lse, bl, Q, bq) || overlap(lse, bl, K, bk) ||
         overlap(lse, bl, V, bk) || overlap(lse, bl, O, bo)))
        return GEMM_TN_ERR_INVALID_ARG;
    if (d != kD || Lk > kMaxLk)
        return GEMM_TN_ERR_UNSUPPORTED;
    if ((uintptr_t)Q % 16 || (uintptr_t)K % 16 || (uintptr_t)V % 16 ||
        (uintptr_t)O % 16 || (uintptr_t)lse % 4)
        return GEMM_TN_ERR_UNSUPPORTED;
    const int64_t q_blocks = (Lq + kBM - 1) / kBM;
    if (q_blocks > 0x7FFFFFFF / batch)
        return GEMM_TN_ERR_UNSUPPORTED;

    AttnArgs a;
    a.Q = (const _Float16 *)Q;
    a.K = (const _Float16 *)K;
    a.V = (const _Float16 *)V;
    a.O = O;
    a.lse = (float *)lse;
    a.Lq = Lq;
    a.Lk = Lk;
    a.scale_abs = fabsf(scale);
    a.c = (float)((double)a.scale_abs * 1.4426950408889634);
    a.qsign = scale < 0.f ? 0x80008000u : 0u;
    a.q_blocks = (int)q_blocks;
    a.batch = (int)batch;
    void *fn = o_dtype == GEMM_TN_F16 ? (void *)&attn_fwd_kernel<_Float16>
                                      : (void *)&attn_fwd_kernel<float>;
    void *args[] = {&a};
    const hipError_t e =
        hipLaunchKernel(fn, dim3((unsigned)(q_blocks * batch)),
                        dim3(kWaves * 64), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? GEMM_TN_OK : GEMM_TN_ERR_LAUNCH;
}
