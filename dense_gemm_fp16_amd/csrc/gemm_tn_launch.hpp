// Launch helpers: pick the kernel instantiation for a plan and enqueue it.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_tn_kernels.hpp"

#include "gemm_tn_config.hpp"

namespace gtn {

// One launcher per tile shape (each defined in its own translation unit so
// the instantiations compile in parallel).
hipError_t launch_tile256(const GemmArgs &a, int loader, int layout,
                          bool out_f32, bool split, bool vec_out,
                          unsigned grid, hipStream_t s);
// The 256 tile of TN operands with direct loads and 16-byte output rows,
// on four waves.
hipError_t launch_tile256_w4(const GemmArgs &a, bool out_f32, bool split,
                             bool vec_out, unsigned grid, hipStream_t s);
hipError_t launch_tile128(const GemmArgs &a, int loader, int layout,
                          bool out_f32, bool split, bool vec_out,
                          unsigned grid, hipStream_t s);
hipError_t launch_tile64(const GemmArgs &a, int loader, int layout,
                         bool out_f32, bool split, bool vec_out,
                         unsigned grid, hipStream_t s);
hipError_t launch_splitk_reduce(const GemmArgs &a, bool out_f32,
                                bool vec_out, hipStream_t s);
// Persistent kernel for K <= 64 (gemm_tn_onek.hip): 128 x 128 tiles walked
// by `grid` workgroups, the next tile's operands loaded while the current
// tile's stores drain.
hipError_t launch_onek(const GemmArgs &a, bool out_f32, unsigned grid,
                       hipStream_t s);

// Kernels instantiated for a launcher: bit 0 = whole-K kernels, bit 1 =
// split-K slices (a tile may run the two with different ring depths).
enum { KERNELS_WHOLE = 1, KERNELS_SPLIT = 2, KERNELS_ALL = 3 };

template <int BM, int BN, int BK, int WM, int WN, int ST, int MINW, int SC,
          int MB, int LOADER, int LAY, int WHICH>
void *pick_kernel(bool out_f32, bool split, bool vec_out)
{
    if (split) {
        if constexpr ((WHICH & KERNELS_SPLIT) != 0)
            return (void *)&gemm_tn_kernel<BM, BN, BK, WM, WN, ST, LOADER,
                                           float, true, true, MINW, SC, MB,
                                           LAY>;
        else
            return nullptr;
    }
    if constexpr ((WHICH & KERNELS_WHOLE) == 0) {
        return nullptr;
    } else {
        if (out_f32)
            return vec_out ? (void *)&gemm_tn_kernel<BM, BN, BK, WM, WN, ST,
                                                     LOADER, float, false,
                                                     true, MINW, SC, MB, LAY>
                           : (void *)&gemm_tn_kernel<BM, BN, BK, WM, WN, ST,
                                                     LOADER, float, false,
                                                     false, MINW, SC, MB,
                                                     LAY>;
        return vec_out ? (void *)&gemm_tn_kernel<BM, BN, BK, WM, WN, ST,
                                                 LOADER, _Float16, false,
                                                 true, MINW, SC, MB, LAY>
                       : (void *)&gemm_tn_kernel<BM, BN, BK, WM, WN, ST,
                                                 LOADER, _Float16, false,
                                                 false, MINW, SC, MB, LAY>;
    }
}

template <int BM, int BN, int BK, int WM, int WN, int ST, int MINW, int SC,
          int MB, int LOADER, int WHICH>
void *pick_layout(int layout, bool out_f32, bool split, bool vec_out)
{
    switch (layout) {
    case 0:
        return pick_kernel<BM, BN, BK, WM, WN, ST, MINW, SC, MB, LOADER, 0,
                           WHICH>(
            out_f32, split, vec_out);
    case 1:
        return pick_kernel<BM, BN, BK, WM, WN, ST, MINW, SC, MB, LOADER, 1,
                           WHICH>(
            out_f32, split, vec_out);
    case 2:
        return pick_kernel<BM, BN, BK, WM, WN, ST, MINW, SC, MB, LOADER, 2,
                           WHICH>(
            out_f32, split, vec_out);
    default:
        return pick_kernel<BM, BN, BK, WM, WN, ST, MINW, SC, MB, LOADER, 3,
                           WHICH>(
            out_f32, split, vec_out);
    }
}

// Kernels of one tile shape for a (loader, layout) pair; nullptr where the
// tile has none: the direct loader takes the layouts in the bit set
// DIRECT_LAYS (operands stored along M / N need 16x16 MFMA tiles), the
// element loader every layout when ELEM_LAYS is set and TN otherwise, the
// register-staged vector loader TN only.  The planner asks only for pairs
// that exist (kTileLayouts).
template <int BM, int BN, int BK, int WM, int WN, int ST, int MINW, int SC,
          int MB, int DIRECT_LAYS, bool ELEM_LAYS, int WHICH = KERNELS_ALL>
hipError_t launch_tile(const GemmArgs &a, int loader, int layout, bool out_f32,
                       bool split, bool vec_out, unsigned grid, hipStream_t s)
{
    static_assert(MB == 16 || DIRECT_LAYS == 1, "layouts need 16x16 MFMA");
    void *fn = nullptr;
    auto direct = [&](auto lay_tag) {
        constexpr int L = decltype(lay_tag)::value;
        if constexpr (((DIRECT_LAYS >> L) & 1) != 0)
            fn = pick_kernel<BM, BN, BK, WM, WN, ST, MINW, SC, MB,
                             LOAD_DIRECT, L, WHICH>(out_f32, split, vec_out);
    };
    switch (loader) {
    case LOAD_DIRECT:
        switch (layout) {
        case 0: direct(Int<0>{}); break;
        case 1: direct(Int<1>{}); break;
        case 2: direct(Int<2>{}); break;
        default: direct(Int<3>{}); break;
        }
        break;
    case LOAD_VREG:
        if (layout == 0)
            fn = pick_kernel<BM, BN, BK, WM, WN, ST, MINW, SC, MB, LOAD_VREG,
                             0, WHICH>(out_f32, split, vec_out);
        break;
    default:
        if constexpr (ELEM_LAYS)
            fn = pick_layout<BM, BN, BK, WM, WN, ST, MINW, SC, MB, LOAD_ELEM,
                             WHICH>(layout, out_f32, split, vec_out);
        else if (layout == 0)
            fn = pick_kernel<BM, BN, BK, WM, WN, ST, MINW, SC, MB, LOAD_ELEM,
                             0, WHICH>(out_f32, split, vec_out);
        break;
    }
    if (fn == nullptr)
        return hipErrorInvalidValue;
    GemmArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(fn, dim3(grid), dim3(WM * WN * 64), args, 0, s);
}

}  // namespace gtn
