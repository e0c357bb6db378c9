// 32-element MX scale-factor instantiations of gemm_tile (both operands of one
// format), for fp32 factors and for the page-native E8M0 layout.
#include "mm_launch.hpp"

namespace mmfp8 {
hipError_t launch_tile_sf32(int cfg, int layout, int f, const GemmArgs& p, int grid, hipStream_t s) {
    if (layout == SF_ATOM_E8M0) return tile_dispatch<MODE_SF32, SF_ATOM_E8M0>(cfg, f, f, p, grid, s);
    return tile_dispatch<MODE_SF32, SF_F32>(cfg, f, f, p, grid, s);
}
}  // namespace mmfp8
