// K-split tile kernel instantiations (per-tensor scales, mid-size M).
#include "mm_launch.hpp"

namespace mmfp8 {

// Slow accumulation on 64x64 tiles takes eight waves (two per SIMD) with its partials finished one B
// fragment at a time, which measured 15.2 against 15.9 us at M = 256 (N = K = 4096) for four waves.
template <int MODE>
static hipError_t ksplit_mode(int ks, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s) {
    constexpr int NW64 = MODE == MODE_SLOW ? 8 : 4;
#define MMFP8_KS(MT, NT, KU, A, B)                                                                              \
    do {                                                                                                        \
        constexpr int NW = MT == 4 ? NW64 : 4;                                                                  \
        hipLaunchKernelGGL((gemm_ksplit<MT, NT, MODE, A, B, NW, KU>), dim3(grid), dim3(NW * 64), 0, s, p);      \
    } while (0)
#define MMFP8_KSF(MT, NT, KU)                                   \
    if (fa == 0 && fb == 0) MMFP8_KS(MT, NT, KU, 0, 0);         \
    else if (fa == 1 && fb == 1) MMFP8_KS(MT, NT, KU, 1, 1);    \
    else if (fa == 0 && fb == 1) MMFP8_KS(MT, NT, KU, 0, 1);    \
    else MMFP8_KS(MT, NT, KU, 1, 0);
    if (ks == KS_64x64) { MMFP8_KSF(4, 4, 1) }
    else { MMFP8_KSF(2, 4, 2) }
#undef MMFP8_KSF
#undef MMFP8_KS
    return hipGetLastError();
}

hipError_t launch_ksplit(int ks, int mode, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s) {
    if (mode == MODE_FAST) return ksplit_mode<MODE_FAST>(ks, fa, fb, p, grid, s);
    return ksplit_mode<MODE_SLOW>(ks, fa, fb, p, grid, s);
}

}  // namespace mmfp8
