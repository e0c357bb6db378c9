// Per-tensor-scale instantiations of gemm_tile: fast and slow accumulation.
#include "mm_launch.hpp"

namespace mmfp8 {
hipError_t launch_tile_fast(int cfg, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s) {
    return tile_dispatch<MODE_FAST, 0>(cfg, fa, fb, p, grid, s);
}
hipError_t launch_tile_slow(int cfg, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s) {
    return tile_dispatch<MODE_SLOW, 0>(cfg, fa, fb, p, grid, s);
}
}  // namespace mmfp8
