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

}  // namespace gtn
