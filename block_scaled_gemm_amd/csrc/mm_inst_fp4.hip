// FP4 (E2M1) MX instantiations of gemm_tile: page-native E8M0 factors per 32
// or per 16 values, or E4M3 factors per 16 values.
#include "mm_launch.hpp"

namespace mmfp8 {
hipError_t launch_tile_fp4(int cfg, int layout, const GemmArgs& p, int grid, hipStream_t s) {
    if (layout == SF_ATOM_E8M0_16) return tile_launch<MODE_SF32, SF_ATOM_E8M0_16, T_E2M1, T_E2M1>(cfg, p, grid, s);
    if (layout == SF_ATOM_E4M3_16) return tile_launch<MODE_SF32, SF_ATOM_E4M3_16, T_E2M1, T_E2M1>(cfg, p, grid, s);
    return tile_launch<MODE_SF32, SF_ATOM_E8M0, T_E2M1, T_E2M1>(cfg, p, grid, s);
}
}  // namespace mmfp8
