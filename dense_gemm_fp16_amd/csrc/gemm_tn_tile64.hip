// Instantiations of the 64x64 tile (2 x 2 waves): whole-K kernels and
// split-K slices with their own ring depths.
#include "gemm_tn_launch.hpp"

namespace gtn {

hipError_t launch_tile64(const GemmArgs &a, int loader, int layout,
                         bool out_f32, bool split, bool vec_out,
                         unsigned grid, hipStream_t s)
{
    if (split)
        return launch_tile<64, 64, GTN_T64_SPLIT_BK, 2, 2, GTN_T64_SPLIT_STAGES, 2,
                           0, GTN_T64_MFMA, GTN_T64_DIRECT_LAYS,
                           GTN_T64_ELEM_LAYS, KERNELS_SPLIT>(
            a, loader, layout, out_f32, split, vec_out, grid, s);
    return launch_tile<64, 64, GTN_T64_BK, 2, 2, GTN_T64_STAGES, 2, 0,
                       GTN_T64_MFMA, GTN_T64_DIRECT_LAYS, GTN_T64_ELEM_LAYS,
                       KERNELS_WHOLE>(
        a, loader, layout, out_f32, split, vec_out, grid, s);
}

}  // namespace gtn
