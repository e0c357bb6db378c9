// Test hook: a plain GEMM on the scaled FP8 / FP4 MFMA of gfx950
// (v_mfma_scale_f32_16x16x128_f8f6f4), to measure how exactly that instruction
// sums its products. Not used by any GEMM entry point: their contraction runs
// on the bf16 MFMA after exact conversion, because this one does not meet the
// 2^-20 sum|t| bound on FP8 data (the measurement this hook serves).
#include "mm_launch.hpp"

namespace mmfp8 {

// One wave per 16 x 16 output tile, every 128 K one scaled MFMA into a single
// fp32 chain: d[m][n] = sum_k A[m][k] B[n][k] 2^(sa[m][k/32] - 127) 2^(sb[n][k/32] - 127)
// (the E8M0 factors default to 127, i.e. 1). Lane (r, g) holds k = 32 g .. 32 g + 31
// of row r: 32 bytes of FP8, or 16 bytes of FP4 (two values per byte), and
// its block's factor byte. Rows are K (FP8) or K / 2 (FP4) bytes.
template <int FMT>  // MFMA format code: 0 E4M3, 1 E5M2, 4 E2M1
__global__ void __launch_bounds__(64) debug_mfma_gemm(const uint8_t* a, const uint8_t* b, const uint8_t* sfa,
                                                      const uint8_t* sfb, float* d, int M, int N, int K) {
    const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
    const int m = blockIdx.x * 16 + r, n = blockIdx.y * 16 + r;
    constexpr bool kFp4 = FMT == 4;
    const int64_t row_bytes = kFp4 ? K / 2 : K;
    const uint8_t* ap = a + (int64_t)m * row_bytes;
    const uint8_t* bp = b + (int64_t)n * row_bytes;
    const int groups = K / 32;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < K; k0 += 128) {
        const int kk = k0 + 32 * g;
        i32x8 va = {0, 0, 0, 0, 0, 0, 0, 0}, vb = {0, 0, 0, 0, 0, 0, 0, 0};
        if constexpr (kFp4) {
            const i32x4 x = *(const i32x4*)(ap + kk / 2), y = *(const i32x4*)(bp + kk / 2);
            va = cat(x, i32x4{0, 0, 0, 0});
            vb = cat(y, i32x4{0, 0, 0, 0});
        } else {
            va = cat(*(const i32x4*)(ap + kk), *(const i32x4*)(ap + kk + 16));
            vb = cat(*(const i32x4*)(bp + kk), *(const i32x4*)(bp + kk + 16));
        }
        const int sa = sfa ? (int)sfa[(int64_t)m * groups + kk / 32] : 127;
        const int sb = sfb ? (int)sfb[(int64_t)n * groups + kk / 32] : 127;
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, acc, FMT, FMT, 0, sa, 0, sb);
    }
    // D[i][j] (i from the first operand, j from the second) is in lane j + 16 (i / 4), register i % 4
#pragma unroll
    for (int q = 0; q < 4; ++q) d[(int64_t)(blockIdx.x * 16 + 4 * g + q) * N + blockIdx.y * 16 + r] = acc[q];
}

hipError_t launch_debug_mfma_gemm(int fmt, const uint8_t* a, const uint8_t* b, const uint8_t* sfa, const uint8_t* sfb,
                                  float* d, int M, int N, int K, hipStream_t s) {
    const dim3 grid(M / 16, N / 16);
    if (fmt == 0) hipLaunchKernelGGL(debug_mfma_gemm<0>, grid, dim3(64), 0, s, a, b, sfa, sfb, d, M, N, K);
    else if (fmt == 1) hipLaunchKernelGGL(debug_mfma_gemm<1>, grid, dim3(64), 0, s, a, b, sfa, sfb, d, M, N, K);
    else hipLaunchKernelGGL(debug_mfma_gemm<4>, grid, dim3(64), 0, s, a, b, sfa, sfb, d, M, N, K);
    return hipGetLastError();
}

}  // namespace mmfp8
