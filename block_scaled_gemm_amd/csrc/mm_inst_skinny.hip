// Skinny-M instantiations (M <= 64, per-tensor scales) and the small helper kernels.
#include "mm_launch.hpp"
#include "mm_skinny_k.hpp"

namespace mmfp8 {

// ------------------------------------------------------------------ small kernels

// Clear the amax outputs on the stream (a kernel rather than a memset, so that
// a captured graph holds no memset node).
__global__ void amax_init(uint32_t* amax_bits, unsigned long long* key) {
    if (threadIdx.x == 0) {
        if (amax_bits) *amax_bits = 0u;
        if (key) *key = 0ull;
    }
}

// Unpack the (|x| bits, index) key into the caller's amax and amax_index; the
// key lives in the amax_index slot itself. Key 0 means no output (index -1).
__global__ void amax_finalize(float* amax, unsigned long long* key_in_index) {
    if (threadIdx.x == 0) {
        const unsigned long long k = *key_in_index;
        const uint32_t bits = (uint32_t)(k >> 33);
        const int64_t idx = k == 0 ? -1 : (int64_t)((1ull << 33) - 1ull - (k & ((1ull << 33) - 1ull)));
        if (amax) *amax = __uint_as_float(bits);
        *(int64_t*)key_in_index = idx;
    }
}

__global__ void debug_convert(const float* x, void* y, int t, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t v = convert(x[i], t);
    if (t == T_F32) ((uint32_t*)y)[i] = v;
    else if (t == T_BF16 || t == T_F16) ((uint16_t*)y)[i] = (uint16_t)v;
    else ((uint8_t*)y)[i] = (uint8_t)v;
}


template <int MODE>
static hipError_t skinny_mode(int mt, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s) {
#define MMFP8_SK(MT, A, B)                                                                                \
    hipLaunchKernelGGL((gemm_skinny<MT, MODE, A, B, skinny_waves(MT), skinny_steps(MT)>), dim3(grid),        \
                       dim3(skinny_waves(MT) * 64), 0, s, p)
#define MMFP8_SKF(MT)                                         \
    if (fa == 0 && fb == 0) MMFP8_SK(MT, 0, 0);               \
    else if (fa == 1 && fb == 1) MMFP8_SK(MT, 1, 1);          \
    else if (fa == 0 && fb == 1) MMFP8_SK(MT, 0, 1);          \
    else MMFP8_SK(MT, 1, 0);
#define MMFP8_SKK(A, B)                                                                                      \
    hipLaunchKernelGGL((gemm_skinny_k<4, 1, MODE, A, B, 16, 2>), dim3(grid), dim3(16 * 64), 0, s, p)
    if (mt == 1) { MMFP8_SKF(1) }
    else if (mt == 2) { MMFP8_SKF(2) }
    else if ((p.K + kBK - 1) / kBK > 32) { MMFP8_SKF(4) }
    else {
        // M = 33 .. 64, K <= 32 steps: sixteen waves with two steps each in flight (gemm_skinny_k)
        if (fa == 0 && fb == 0) MMFP8_SKK(0, 0);
        else if (fa == 1 && fb == 1) MMFP8_SKK(1, 1);
        else if (fa == 0 && fb == 1) MMFP8_SKK(0, 1);
        else MMFP8_SKK(1, 0);
    }
#undef MMFP8_SKK
#undef MMFP8_SKF
#undef MMFP8_SK
    return hipGetLastError();
}

hipError_t launch_skinny(int mt, int mode, int fa, int fb, const GemmArgs& p, int grid, hipStream_t s) {
    if (mode == MODE_FAST) return skinny_mode<MODE_FAST>(mt, fa, fb, p, grid, s);
    return skinny_mode<MODE_SLOW>(mt, fa, fb, p, grid, s);
}

hipError_t launch_amax_init(uint32_t* bits, unsigned long long* key, hipStream_t s) {
    hipLaunchKernelGGL(amax_init, dim3(1), dim3(64), 0, s, bits, key);
    return hipGetLastError();
}

hipError_t launch_amax_finalize(float* amax, unsigned long long* key, hipStream_t s) {
    hipLaunchKernelGGL(amax_finalize, dim3(1), dim3(64), 0, s, amax, key);
    return hipGetLastError();
}

hipError_t launch_debug_convert(const float* x, void* y, int t, int64_t n, hipStream_t s) {
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(debug_convert, dim3((unsigned)blocks), dim3(256), 0, s, x, y, t, n);
    return hipGetLastError();
}

}  // namespace mmfp8
