// 1x128 / 128x128 block-scale instantiations of gemm_tile.
#include "mm_launch.hpp"

namespace mmfp8 {
hipError_t launch_tile_block(int cfg, int sbm, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s) {
    if (sbm == SB_128x128) return tile_dispatch<MODE_BLOCK, SB_128x128>(cfg, fa, fb, p, grid, s);
    return tile_dispatch<MODE_BLOCK, SB_1x128>(cfg, fa, fb, p, grid, s);
}
}  // namespace mmfp8
