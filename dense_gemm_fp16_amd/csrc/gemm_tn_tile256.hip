// Instantiations of the 256x256 tile.
#include "gemm_tn_launch.hpp"

namespace gtn {

hipError_t launch_tile256(const GemmArgs &a, int loader, int layout,
                          bool out_f32, bool split, bool vec_out,
                          unsigned grid, hipStream_t s)
{
    return launch_tile<256, 256, GTN_T256_BK, GTN_T256_WM, GTN_T256_WN,
                       GTN_T256_STAGES, GTN_T256_MINW, GTN_T256_SCHED,
                       GTN_T256_MFMA, GTN_T256_DIRECT_LAYS,
                       GTN_T256_ELEM_LAYS>(
        a, loader, layout, out_f32, split, vec_out, grid, s);
}

// The 256 tile of TN operands with direct loads on four waves (one per
// SIMD, SCHED 3): whole-K kernels with 16-byte output rows and split-K
// slices only (the planner asks for nothing else).
hipError_t launch_tile256_w4(const GemmArgs &a, bool out_f32, bool split,
                             bool vec_out, unsigned grid, hipStream_t s)
{
    if (!vec_out && !split)
        return hipErrorInvalidValue;
    void *fn = split ? (void *)&gemm_tn_kernel<256, 256, 64, 2, 2, 2,
                                               LOAD_DIRECT, float, true, true,
                                               1, 3, 16, 0>
             : out_f32 ? (void *)&gemm_tn_kernel<256, 256, 64, 2, 2, 2,
                                                 LOAD_DIRECT, float, false,
                                                 true, 1, 3, 16, 0>
                       : (void *)&gemm_tn_kernel<256, 256, 64, 2, 2, 2,
                                                 LOAD_DIRECT, _Float16, false,
                                                 true, 1, 3, 16, 0>;
    GemmArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, s);
}

}  // namespace gtn
