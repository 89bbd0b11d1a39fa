// Instantiations of the 256x256x64 tile (2 x 2 waves).
#include "gemm_tn_launch.hpp"

namespace gtn {

hipError_t launch_tile256(const GemmArgs &a, int loader, bool out_f32,
                         bool split, bool vec_out, unsigned grid,
                         hipStream_t s)
{
    return launch_tile<256, 256, 2, 2, 1>(a, loader, out_f32, split, vec_out,
                                          grid, s);
}

}  // namespace gtn
