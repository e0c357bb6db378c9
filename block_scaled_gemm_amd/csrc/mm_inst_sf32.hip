// 32-element MX scale-factor instantiations of gemm_tile (both operands of one format).
#include "mm_launch.hpp"

namespace mmfp8 {
hipError_t launch_tile_sf32(int cfg, int f, const GemmArgs& p, int grid, hipStream_t s) {
    return tile_dispatch<MODE_SF32, 0>(cfg, f, f, p, grid, s);
}
}  // namespace mmfp8
