// mm_launch.hpp -- host-side launchers of the gfx950 kernels (internal to libmmfp8).
#pragma once

#include <hip/hip_runtime.h>

#include "mm_kernels.hpp"

namespace mmfp8 {

// Workgroup tiles of gemm_tile, largest first.
enum TileCfg : int { CFG_256x256 = 0, CFG_256x128 = 1, CFG_128x128 = 2, CFG_64x64 = 3, CFG_COUNT = 4 };
constexpr int kCfgBM[CFG_COUNT] = {256, 256, 128, 64};
constexpr int kCfgBN[CFG_COUNT] = {256, 128, 128, 64};

hipError_t launch_tile_fast(int cfg, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s);
hipError_t launch_tile_slow(int cfg, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s);
hipError_t launch_tile_block(int cfg, int sbm, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s);
hipError_t launch_tile_sf32(int cfg, int f, const GemmArgs& p, int grid, hipStream_t s);
hipError_t launch_skinny(int mt, int mode, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s);
hipError_t launch_amax_init(uint32_t* bits, unsigned long long* key, hipStream_t s);
hipError_t launch_amax_finalize(float* amax, unsigned long long* key, hipStream_t s);
hipError_t launch_debug_convert(const float* x, void* y, int t, int64_t n, hipStream_t s);

// Largest tile each mode is built for: the fast chain keeps 256 fp32
// accumulators per lane and nothing else, the promoted and MX-scaled modes also
// hold their partials or scale operands, so they stop at 256x128 (128x128 with
// a 1x128 scale_b, which needs four scale values per lane and tile).
constexpr int min_cfg(int mode, int sbm) {
    return mode == MODE_FAST ? CFG_256x256 : (mode == MODE_BLOCK && sbm == SB_1x128) ? CFG_128x128 : CFG_256x128;
}

// Launch gemm_tile<BM, BN, MODE, fa, fb, SBM> for a runtime cfg / format pair.
template <int MODE, int SBM>
hipError_t tile_dispatch(int cfg, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s) {
#define MMFP8_TILE(BM, BN, A, B) \
    hipLaunchKernelGGL((gemm_tile<BM, BN, MODE, A, B, SBM>), dim3(grid), dim3(256), 0, s, p)
#define MMFP8_FMTS(BM, BN)                                       \
    if (fa == 0 && fb == 0) MMFP8_TILE(BM, BN, 0, 0);            \
    else if (fa == 1 && fb == 1) MMFP8_TILE(BM, BN, 1, 1);       \
    else if (fa == 0 && fb == 1) MMFP8_TILE(BM, BN, 0, 1);       \
    else MMFP8_TILE(BM, BN, 1, 0);
    if (cfg < min_cfg(MODE, SBM)) cfg = min_cfg(MODE, SBM);
    switch (cfg) {
        case CFG_256x256:
            if constexpr (MODE == MODE_FAST) { MMFP8_FMTS(256, 256) }
            break;
        case CFG_256x128:
            if constexpr (!(MODE == MODE_BLOCK && SBM == SB_1x128)) { MMFP8_FMTS(256, 128) }
            break;
        case CFG_128x128: MMFP8_FMTS(128, 128) break;
        default: MMFP8_FMTS(64, 64) break;
    }
#undef MMFP8_FMTS
#undef MMFP8_TILE
    return hipGetLastError();
}

}  // namespace mmfp8
