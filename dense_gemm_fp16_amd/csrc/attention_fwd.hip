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
//    direct 16-byte buffer loads (two stages: block kb+1 loads while kb is
//    computed).  Keys past Lk read as zero.
//  * S = Q K^T: v_mfma_f32_16x16x32_f16 with the K fragment as the first
//    operand, so a lane holds query row (lane % 16) and keys
//    16j + 4(lane / 16) + e of each 16-key block j.
//  * Softmax: per-row maximum over the block (in-lane, then across the four
//    lanes that share a row), exp2 of the score times |scale| log2(e) minus
//    the shifted row maximum, fp32 row sums per lane.  The row shift moves
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
//  * Epilogue: each row is divided by its sum (the four lane partials
//    added), rounded once to fp16 or fp32, and stored; lse = |scale| *
//    shift + ln(sum).
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

// LDS swizzle of the V tile (64-element = 128-byte rows of keys), for its
// ds_read_b64_tr_b16 reads: a half wave reads 8 consecutive key rows at one
// pair of 16-byte chunks (c, c + 1), c even.  Rows of one parity share a
// 256-byte bank line; XORing the chunk with 2 * ((row / 2) % 4) puts the 4
// rows of each parity on distinct chunk pairs, so the 32 lanes hit 64
// distinct banks.
__device__ inline int v_swizzle(int row) { return 2 * ((row >> 1) & 3); }

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
    __shared__ __attribute__((aligned(1024))) _Float16 lds[2 * 2 * TILE];

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

    // ---- K / V tiles of key block kb into LDS stage `stage` -------------
    // One 1 KiB load of a wave fills 8 tile rows; lane l lands in physical
    // chunk l % 8 of row l / 8 and fetches the logical chunk mapped there.
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(p.K + b * Lk * kD, Lk * kD * 2);
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(p.V + b * Lk * kD, Lk * kD * 2);
    auto issue = [&](int stage, int kb) {
        GTN_LDS _Float16 *base = (GTN_LDS _Float16 *)lds + stage * 2 * TILE;
#pragma unroll
        for (int h = 0; h < kBN / 8 / kWaves; ++h) {
            const int grp = wave + kWaves * h;
            const int row = grp * 8 + (lane >> 3);
            const uint32_t roff = (uint32_t)(kb * kBN + row) * (kD * 2);
            const int kc = swizzle_chunk<kD>(row, lane & 7);
            const int vc = (lane & 7) ^ v_swizzle(row);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rK, (GTN_LDS void *)(base + grp * 8 * kD), 16,
                roff + (uint32_t)kc * 16, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rV, (GTN_LDS void *)(base + TILE + grp * 8 * kD), 16,
                roff + (uint32_t)vc * 16, 0, 0, 0);
        }
    };

    f32x4 oacc[MI][DJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < DJ; ++j)
            oacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mref[MI], lsum[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        mref[i] = 0.f;
        lsum[i] = 0.f;
    }

    const int nblk = (int)((Lk + kBN - 1) / kBN);
    const int tail_keys = (int)(Lk - (int64_t)(nblk - 1) * kBN);   // 1..64
    const float c = p.c;

    // Softmax of one key block, in place in sacc (scores -> probabilities),
    // then the fp16 probability fragments of the P V product.
    auto softmax = [&](auto tail_tag, int kb, f32x4 (&sacc)[MI][NJ],
                       half8 (&pf)[MI][KS]) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        float mx[MI];
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            if (TAIL) {
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
                    m = fmaxf(m, sacc[i][j][e]);
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            mx[i] = m;
        }
        if (kb == 0) {
#pragma unroll
            for (int i = 0; i < MI; ++i)
                mref[i] = mx[i];
        } else {
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
                    lsum[i] *= f;
#pragma unroll
                    for (int j = 0; j < DJ; ++j)
                        oacc[i][j] *= f;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const float mc = mref[i] * c;
            float ls = 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float pe = __builtin_amdgcn_exp2f(
                        __builtin_fmaf(sacc[i][j][e], c, -mc));
                    if (TAIL && j * 16 + 4 * g + e >= tail_keys)
                        pe = 0.f;
                    sacc[i][j][e] = pe;
                    ls += pe;
                }
            lsum[i] += ls;
#pragma unroll
            for (int t = 0; t < KS; ++t) {
                const f32x4 a = sacc[i][2 * t], bb = sacc[i][2 * t + 1];
                pf[i][t] = half8{(_Float16)a[0], (_Float16)a[1],
                                 (_Float16)a[2], (_Float16)a[3],
                                 (_Float16)bb[0], (_Float16)bb[1],
                                 (_Float16)bb[2], (_Float16)bb[3]};
            }
        }
    };

    issue(0, 0);
    for (int kb = 0; kb < nblk; ++kb) {
        const int cur = kb & 1;
        // Own loads of block kb landed; after the barrier every wave's have,
        // and every wave is done reading stage cur ^ 1 (block kb - 1).
        wait_vmcnt<0>();
        wait_lgkmcnt<0>();
        block_sync();
        if (kb + 1 < nblk)
            issue(cur ^ 1, kb + 1);
        const _Float16 *sK = lds + cur * 2 * TILE;
        const _Float16 *sV = sK + TILE;

        f32x4 sacc[MI][NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                sacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DS; ++s)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int row = j * 16 + r16;
                const half8 kf = *(const half8 *)(
                    sK + row * kD + swizzle_chunk<kD>(row, 4 * s + g) * 8);
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    sacc[i][j] = mfma16(kf, qf[i][s], sacc[i][j]);
            }

        half8 pf[MI][KS];
        if (kb == nblk - 1 && tail_keys < kBN)
            softmax(Bool<true>{}, kb, sacc, pf);
        else
            softmax(Bool<false>{}, kb, sacc, pf);

#pragma unroll
        for (int t = 0; t < KS; ++t)
#pragma unroll
            for (int dj = 0; dj < DJ; ++dj) {
                const int col = dj * 16 + 4 * (r16 & 3);
                auto rd = [&](int r) {
                    const int row = 32 * t + 16 * r + 4 * g + (r16 >> 2);
                    const int pc = (col >> 3) ^ v_swizzle(row);
                    const GTN_LDS _Float16 *a =
                        (const GTN_LDS _Float16 *)sV + row * kD + pc * 8 +
                        (col & 7);
                    return __builtin_bit_cast(
                        half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                   (GTN_LDS s16x4 *)a));
                };
                const half4 lo = rd(0), hi = rd(1);
                const half8 vf = {lo[0], lo[1], lo[2], lo[3],
                                  hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    oacc[i][dj] = mfma16(vf, pf[i][t], oacc[i][dj]);
            }
    }

    // ---- epilogue ----------------------------------------------------------
    constexpr int ES = OutTraits<OutT>::bytes;
    const __amdgpu_buffer_rsrc_t rO =
        make_rsrc((char *)p.O + (b * Lq + q0) * kD * ES, (Lq - q0) * kD * ES);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        float l = lsum[i];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const float inv = 1.0f / l;
#pragma unroll
        for (int dj = 0; dj < DJ; ++dj) {
            const uint32_t off =
                (uint32_t)(((i * 16 + r16) * kD + dj * 16 + 4 * g) * ES);
            store_out_vec4(rO, off, oacc[i][dj] * inv, (OutT *)nullptr);
        }
        const int64_t row = q0 + i * 16 + r16;
        if (p.lse != nullptr && g == 0 && row < Lq)
            p.lse[b * Lq + row] = p.scale_abs * mref[i] + logf(l);
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
