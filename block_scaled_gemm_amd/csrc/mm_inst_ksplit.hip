// K-split tile kernel instantiations (per-tensor scales, mid-size M).
#include "mm_launch.hpp"

namespace mmfp8 {

template <int MODE>
static hipError_t ksplit_mode(int ks, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s) {
#define MMFP8_KS(MT, NT, KU, A, B) \
    hipLaunchKernelGGL((gemm_ksplit<MT, NT, MODE, A, B, 4, KU>), dim3(grid), dim3(4 * 64), 0, s, p)
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
