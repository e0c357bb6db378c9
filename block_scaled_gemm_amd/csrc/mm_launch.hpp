// mm_launch.hpp -- host-side launchers of the gfx950 kernels (internal to libmmfp8).
#pragma once

#include <hip/hip_runtime.h>

#include "mm_kernels.hpp"

namespace mmfp8 {

// Workgroup tiles of gemm_tile, largest first: BM x BN and waves WM x WN.
// 256x256 gives each of its 8 waves a 64x128 tile (1.5 FP8->bf16 converts per
// MFMA); the others use 64x64 wave tiles (2 converts per MFMA).
enum TileCfg : int { CFG_256x256 = 0, CFG_128x256 = 1, CFG_128x128 = 2, CFG_64x64 = 3, CFG_COUNT = 4 };
constexpr int kCfgBM[CFG_COUNT] = {256, 128, 128, 64};
constexpr int kCfgBN[CFG_COUNT] = {256, 256, 128, 64};
constexpr int kCfgWM[CFG_COUNT] = {4, 2, 2, 2};
constexpr int kCfgWN[CFG_COUNT] = {2, 4, 2, 2};
// Whether the main loop runs its fragment reads a half-step ahead. Only the
// chained modes on the 4-wave 128x128 tile do: that workgroup has one wave per
// SIMD and runs alone on its CU (the second fragment set takes the registers a
// second workgroup would need). The promoted modes keep 64x64 partials as
// well, so there the 128x128 tile runs without it, two workgroups per CU whose
// waves share the SIMDs and cover each other's LDS latency.
// FP4 operands read their scale factors from the stage during the whole
// step, so they take the plain loop.
constexpr int cfg_pipe(int cfg, int mode, int fmt) {
    return cfg == CFG_128x128 && (mode == MODE_FAST || mode == MODE_SF32) && fmt != T_E2M1 ? 1 : 0;
}

// gemm_skinny: waves per workgroup and K steps in flight per wave, by MT
// (M <= 16 MT; MT = 1, 2). Sixteen waves with two steps each put a K = 4096 B
// tile in flight at once. M = 33 .. 64 (MT = 4) with K <= 4096 runs
// gemm_skinny_k, whose sixteen waves also keep two steps each in flight (with
// gemm_skinny at MT = 4 the A fragments need more registers than 16 waves per
// CU leave); a longer K runs gemm_skinny<4> with 8 waves of one step.
constexpr int skinny_waves(int mt) { return mt == 4 ? 8 : 16; }
constexpr int skinny_steps(int mt) { return mt == 4 ? 1 : 2; }

// gemm_ksplit variants for per-tensor M above the skinny range while the
// 128x128 tiles of gemm_tile are fewer than the CUs: a 64x64 tile, or 32x64
// when even the 64x64 tiles are fewer than the CUs; four waves split K, two K
// steps in flight for the smaller tile.
enum KsplitCfg : int { KS_64x64 = 0, KS_32x64 = 1 };
constexpr int kKsBM[2] = {64, 32};
constexpr int kKsBN[2] = {64, 64};

hipError_t launch_tile_fast(int cfg, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s);
hipError_t launch_tile_slow(int cfg, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s);
hipError_t launch_tile_block(int cfg, int sbm, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s);
hipError_t launch_tile_sf32(int cfg, int layout, int f, const GemmArgs& p, int grid, hipStream_t s);
hipError_t launch_tile_fp4(int cfg, int layout, const GemmArgs& p, int grid, hipStream_t s);
hipError_t launch_skinny(int mt, int mode, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s);
hipError_t launch_ksplit(int ks, int mode, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s);
hipError_t launch_amax_init(uint32_t* bits, unsigned long long* key, hipStream_t s);
hipError_t launch_amax_finalize(float* amax, unsigned long long* key, hipStream_t s);
hipError_t launch_debug_convert(const float* x, void* y, int t, int64_t n, hipStream_t s);
hipError_t launch_debug_mfma_gemm(int fmt, const uint8_t* a, const uint8_t* b, const uint8_t* sfa, const uint8_t* sfb,
                                  float* d, int M, int N, int K, hipStream_t s);
// Operand packing (mm_pack.hip).
hipError_t launch_group_starts(const int* sizes, int G, int64_t* start, hipStream_t s);
hipError_t launch_transpose(const uint8_t* src, int64_t L, int64_t R, int64_t C, int64_t ld_src, int64_t src_batch,
                            uint8_t* dst, int64_t ld_dst, int64_t dst_batch, hipStream_t s);
hipError_t launch_group_pack(bool trans, const uint8_t* src, int64_t R, int64_t C, int64_t ld_src, uint8_t* dst,
                             int64_t dst_cols, const int* sizes, const int* offsets, const int64_t* start, int G,
                             hipStream_t s);

// Largest tile each mode is built for. The chained modes (fast, MX) keep 128
// fp32 accumulators per lane and little else, so they take the 64x128 wave
// tile. The promoted modes (slow, block-scaled) also hold a 128-chunk partial
// per accumulator; their largest tile is 128x128 at two workgroups per CU,
// which measured faster than 128x256 at one (eight waves that all meet at
// every step's barrier, where the older wave of each SIMD pair finishes first
// and the younger then runs alone). Slow accumulation, and block scaling with
// a 128x128 scale_b, also have the 256x256 tile with its row-chunk loop (only
// the partials of one fragment row live), which the dense entry points price
// against the 128x128 tiles round by round (rc_columns in mm_api.cpp); it is
// not a starting point of the largest-tile search. FP4 operands on the 64x128
// wave tile spill over a hundred registers (their scale factors change within
// a step; on the scaled FP4 MFMA too: 242), so they start at 128x256.
constexpr int min_cfg(int mode, int sbm, int fmt = 0) {
    (void)sbm;
    if (fmt == T_E2M1) return CFG_128x256;
    return (mode == MODE_FAST || mode == MODE_SF32) ? CFG_256x256 : CFG_128x128;
}

// Compute units of the current device.
int device_cus();

// Launch gemm_tile<BM, BN, MODE, FA, FB, SBM> for a runtime cfg over `grid`
// tiles. 128x128 tiles that are no more than the CUs (one per CU) run with two
// K groups of four waves (eight waves per workgroup), FP8 operands in every
// mode: per-tensor slow it measured 5-7% faster there than four waves with one
// wave per SIMD (and slower as soon as two workgroups per CU are possible), MX
// 1.4x faster than the pipelined four-wave tile (L = 1, 2048 x 2048 x 8192).
template <int MODE, int SBM, int FA, int FB>
hipError_t tile_launch(int cfg, const GemmArgs& p, int grid, hipStream_t s) {
    constexpr int kKG = FA == T_E2M1 ? 1 : 2;
    const bool kgroups = kKG > 1 && cfg == CFG_128x128 && grid <= device_cus();
#define MMFP8_TILE(C)                                                                                              \
    do {                                                                                                           \
        bool done = false;                                                                                         \
        if constexpr (C == CFG_128x128 && kKG > 1) {                                                               \
            if (kgroups) {                                                                                         \
                hipLaunchKernelGGL((gemm_tile<kCfgBM[C], kCfgBN[C], kCfgWM[C], kCfgWN[C], 0, MODE, FA, FB, SBM, kKG>), \
                                   dim3(grid), dim3(kCfgWM[C] * kCfgWN[C] * kKG * 64), 0, s, p);                   \
                done = true;                                                                                       \
            }                                                                                                      \
        }                                                                                                          \
        if (!done)                                                                                                 \
            hipLaunchKernelGGL((gemm_tile<kCfgBM[C], kCfgBN[C], kCfgWM[C], kCfgWN[C], cfg_pipe(C, MODE, FA), MODE, FA, \
                                          FB, SBM>),                                                               \
                               dim3(grid), dim3(kCfgWM[C] * kCfgWN[C] * 64), 0, s, p);                             \
    } while (0)
    // (slow accumulation, and block scaling with a 128x128 scale_b, take the 256x256 tile only when the
    // caller picked it)
    const bool slow256 = (MODE == MODE_SLOW || (MODE == MODE_BLOCK && SBM == SB_128x128)) && cfg == CFG_256x256;
    if (cfg < min_cfg(MODE, SBM, FA) && !slow256) cfg = min_cfg(MODE, SBM, FA);
    switch (cfg) {
        case CFG_256x256:
            if constexpr ((MODE == MODE_FAST || MODE == MODE_SF32 || MODE == MODE_SLOW ||
                           (MODE == MODE_BLOCK && SBM == SB_128x128)) &&
                          FA != T_E2M1)
                MMFP8_TILE(CFG_256x256);
            break;
        case CFG_128x256:
            if constexpr (MODE == MODE_FAST || MODE == MODE_SF32) MMFP8_TILE(CFG_128x256);
            break;
        case CFG_128x128: MMFP8_TILE(CFG_128x128); break;
        default: MMFP8_TILE(CFG_64x64); break;
    }
#undef MMFP8_TILE
    return hipGetLastError();
}

// tile_launch for a runtime pair of FP8 formats.
template <int MODE, int SBM>
hipError_t tile_dispatch(int cfg, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s) {
    if (fa == 0 && fb == 0) return tile_launch<MODE, SBM, 0, 0>(cfg, p, grid, s);
    if (fa == 1 && fb == 1) return tile_launch<MODE, SBM, 1, 1>(cfg, p, grid, s);
    if (fa == 0 && fb == 1) return tile_launch<MODE, SBM, 0, 1>(cfg, p, grid, s);
    return tile_launch<MODE, SBM, 1, 0>(cfg, p, grid, s);
}

}  // namespace mmfp8
