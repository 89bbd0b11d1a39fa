// Launch helpers: pick the kernel instantiation for a plan and enqueue it.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_tn_kernels.hpp"

#include "gemm_tn_config.hpp"

namespace gtn {

// One launcher per tile shape (each defined in its own translation unit so
// the instantiations compile in parallel).
hipError_t launch_tile256(const GemmArgs &a, int loader, bool out_f32,
                          bool split, bool vec_out, unsigned grid,
                          hipStream_t s);
hipError_t launch_tile128(const GemmArgs &a, int loader, bool out_f32,
                          bool split, bool vec_out, unsigned grid,
                          hipStream_t s);
hipError_t launch_tile64(const GemmArgs &a, int loader, bool out_f32,
                         bool split, bool vec_out, unsigned grid,
                         hipStream_t s);
hipError_t launch_splitk_reduce(const GemmArgs &a, bool out_f32,
                                bool vec_out, hipStream_t s);

template <int BM, int BN, int BK, int WM, int WN, int ST, int MINW, int SC,
          int MB, int LOADER>
void *pick_kernel(bool out_f32, bool split, bool vec_out)
{
    if (split)
        return (void *)&gemm_tn_kernel<BM, BN, BK, WM, WN, ST, LOADER, float,
                                       true, true, MINW, SC, MB>;
    if (out_f32)
        return vec_out ? (void *)&gemm_tn_kernel<BM, BN, BK, WM, WN, ST,
                                                 LOADER, float, false, true,
                                                 MINW, SC, MB>
                       : (void *)&gemm_tn_kernel<BM, BN, BK, WM, WN, ST,
                                                 LOADER, float, false, false,
                                                 MINW, SC, MB>;
    return vec_out ? (void *)&gemm_tn_kernel<BM, BN, BK, WM, WN, ST, LOADER,
                                             _Float16, false, true, MINW, SC,
                                             MB>
                   : (void *)&gemm_tn_kernel<BM, BN, BK, WM, WN, ST, LOADER,
                                             _Float16, false, false, MINW, SC,
                                             MB>;
}

template <int BM, int BN, int BK, int WM, int WN, int ST, int MINW, int SC,
          int MB>
hipError_t launch_tile(const GemmArgs &a, int loader, bool out_f32, bool split,
                       bool vec_out, unsigned grid, hipStream_t s)
{
    void *fn;
    switch (loader) {
    case LOAD_DIRECT:
        fn = pick_kernel<BM, BN, BK, WM, WN, ST, MINW, SC, MB, LOAD_DIRECT>(
            out_f32, split, vec_out);
        break;
    case LOAD_VREG:
        fn = pick_kernel<BM, BN, BK, WM, WN, ST, MINW, SC, MB, LOAD_VREG>(
            out_f32, split, vec_out);
        break;
    default:
        fn = pick_kernel<BM, BN, BK, WM, WN, ST, MINW, SC, MB, LOAD_ELEM>(
            out_f32, split, vec_out);
        break;
    }
    GemmArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(fn, dim3(grid), dim3(WM * WN * 64), args, 0, s);
}

}  // namespace gtn
