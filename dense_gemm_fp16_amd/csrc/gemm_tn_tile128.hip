// Instantiations of the 128x128 tile (2 x 2 waves).
#include "gemm_tn_launch.hpp"

namespace gtn {

hipError_t launch_tile128(const GemmArgs &a, int loader, int layout,
                          bool out_f32, bool split, bool vec_out,
                          unsigned grid, hipStream_t s)
{
    return launch_tile<128, 128, GTN_T128_BK, 2, 2, GTN_T128_STAGES, 2, 0,
                       GTN_T128_MFMA, GTN_T128_DIRECT_LAYS,
                       GTN_T128_ELEM_LAYS>(
        a, loader, layout, out_f32, split, vec_out, grid, s);
}

}  // namespace gtn
