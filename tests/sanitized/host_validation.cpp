// Host-side checks of the C ABI's argument validation, built with AddressSanitizer
// and UndefinedBehaviorSanitizer (host code only) and run on the CPU. The kernel
// launchers are replaced by stubs that count calls: a call that validation
// rejects, or that has nothing to do, must return before any launch.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "mm.h"
#include "mm_launch.hpp"

static int g_launches = 0;

namespace mmfp8 {
#define STUB(...)            \
    {                        \
        ++g_launches;        \
        return hipErrorUnknown; \
    }
hipError_t launch_tile_fast(int, int, int, const GemmArgs&, int, hipStream_t) STUB()
hipError_t launch_tile_slow(int, int, int, const GemmArgs&, int, hipStream_t) STUB()
hipError_t launch_tile_block(int, int, int, int, const GemmArgs&, int, hipStream_t) STUB()
hipError_t launch_tile_sf32(int, int, int, const GemmArgs&, int, hipStream_t) STUB()
hipError_t launch_tile_fp4(int, int, const GemmArgs&, int, hipStream_t) STUB()
hipError_t launch_skinny(int, int, int, int, const GemmArgs&, int, hipStream_t) STUB()
hipError_t launch_ksplit(int, int, int, int, const GemmArgs&, int, hipStream_t) STUB()
hipError_t launch_amax_init(uint32_t*, unsigned long long*, hipStream_t) STUB()
hipError_t launch_amax_finalize(float*, unsigned long long*, hipStream_t) STUB()
hipError_t launch_debug_convert(const float*, void*, int, int64_t, hipStream_t) STUB()
hipError_t launch_debug_mfma_gemm(int, const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, float*, int,
                                  int, int, hipStream_t) STUB()
hipError_t launch_group_starts(const int*, int, int64_t*, hipStream_t) STUB()
hipError_t launch_transpose(const uint8_t*, int64_t, int64_t, int64_t, int64_t, int64_t, uint8_t*, int64_t, int64_t,
                            hipStream_t) STUB()
hipError_t launch_group_pack(bool, const uint8_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, const int*,
                             const int*, const int64_t*, int, hipStream_t) STUB()
#undef STUB
}  // namespace mmfp8

static int g_failures = 0, g_cases = 0;

// A rejected call: not MM_OK, no launch, a message.
static void rejected(const char* what, mm_status st) {
    ++g_cases;
    const char* msg = mm_last_error();
    if (st == MM_OK || g_launches != 0 || msg == nullptr || std::strlen(msg) == 0) {
        std::printf("FAIL %s: status %d, launches %d, message '%s'\n", what, (int)st, g_launches, msg ? msg : "(null)");
        ++g_failures;
    }
    g_launches = 0;
}

// A call with nothing to do: MM_OK and no launch.
static void nothing(const char* what, mm_status st) {
    ++g_cases;
    if (st != MM_OK || g_launches != 0) {
        std::printf("FAIL %s: status %d, launches %d\n", what, (int)st, g_launches);
        ++g_failures;
    }
    g_launches = 0;
}

int main() {
    // device pointers are never dereferenced on the host: aligned placeholders stand in for them
    void* const P = reinterpret_cast<void*>(uintptr_t(1) << 20);
    float* const S = reinterpret_cast<float*>(uintptr_t(1) << 21);
    int32_t* const G32 = reinterpret_cast<int32_t*>(uintptr_t(1) << 22);
    const int E4 = MM_F8_E4M3FN, BF = MM_BF16;
    const int64_t BIG = INT64_MAX;

    rejected("gemm M < 0", mm_scaled_gemm(-1, 64, 64, P, E4, 64, P, E4, 64, S, MM_SCALE_TENSOR, S, MM_SCALE_TENSOR,
                                          nullptr, P, BF, 64, 0, nullptr));
    rejected("gemm K huge", mm_scaled_gemm(64, 64, BIG, P, E4, BIG, P, E4, BIG, S, MM_SCALE_TENSOR, S,
                                           MM_SCALE_TENSOR, nullptr, P, BF, 64, 0, nullptr));
    rejected("gemm a null", mm_scaled_gemm(64, 64, 64, nullptr, E4, 64, P, E4, 64, S, MM_SCALE_TENSOR, S,
                                           MM_SCALE_TENSOR, nullptr, P, BF, 64, 0, nullptr));
    rejected("gemm bad a_type", mm_scaled_gemm(64, 64, 64, P, 99, 64, P, E4, 64, S, MM_SCALE_TENSOR, S,
                                               MM_SCALE_TENSOR, nullptr, P, BF, 64, 0, nullptr));
    rejected("gemm bad d_type", mm_scaled_gemm(64, 64, 64, P, E4, 64, P, E4, 64, S, MM_SCALE_TENSOR, S,
                                               MM_SCALE_TENSOR, nullptr, P, -7, 64, 0, nullptr));
    rejected("gemm lda < K", mm_scaled_gemm(64, 64, 128, P, E4, 64, P, E4, 128, S, MM_SCALE_TENSOR, S,
                                            MM_SCALE_TENSOR, nullptr, P, BF, 64, 0, nullptr));
    rejected("gemm ldd < N", mm_scaled_gemm(64, 128, 64, P, E4, 64, P, E4, 64, S, MM_SCALE_TENSOR, S,
                                            MM_SCALE_TENSOR, nullptr, P, BF, 64, 0, nullptr));
    rejected("gemm scale pair", mm_scaled_gemm(64, 64, 128, P, E4, 128, P, E4, 128, S, MM_SCALE_1x128, S,
                                               MM_SCALE_TENSOR, nullptr, P, BF, 64, 0, nullptr));
    rejected("gemm bad scale mode", mm_scaled_gemm(64, 64, 128, P, E4, 128, P, E4, 128, S, 42, S, MM_SCALE_TENSOR,
                                                   nullptr, P, BF, 64, 0, nullptr));
    rejected("gemm scale null", mm_scaled_gemm(64, 64, 64, P, E4, 64, P, E4, 64, nullptr, MM_SCALE_TENSOR, S,
                                               MM_SCALE_TENSOR, nullptr, P, BF, 64, 0, nullptr));
    rejected("gemm misaligned a", mm_scaled_gemm(64, 64, 64, static_cast<char*>(P) + 1, E4, 64, P, E4, 64, S,
                                                 MM_SCALE_TENSOR, S, MM_SCALE_TENSOR, nullptr, P, BF, 64, 0, nullptr));
    rejected("gemm misaligned lda", mm_scaled_gemm(64, 64, 64, P, E4, 65, P, E4, 64, S, MM_SCALE_TENSOR, S,
                                                   MM_SCALE_TENSOR, nullptr, P, BF, 64, 0, nullptr));
    nothing("gemm M = 0", mm_scaled_gemm(0, 64, 64, P, E4, 64, P, E4, 64, S, MM_SCALE_TENSOR, S, MM_SCALE_TENSOR,
                                         nullptr, P, BF, 64, 0, nullptr));
    rejected("bias with FP8 out", mm_scaled_gemm_bias(64, 64, 64, P, E4, 64, P, E4, 64, S, MM_SCALE_TENSOR, S,
                                                      MM_SCALE_TENSOR, P, P, MM_F8_E4M3FN, 64, 0, nullptr));
    rejected("bias misaligned", mm_scaled_gemm_bias(64, 64, 64, P, E4, 64, P, E4, 64, S, MM_SCALE_TENSOR, S,
                                                    MM_SCALE_TENSOR, static_cast<char*>(P) + 1, P, BF, 64, 0, nullptr));
    rejected("batched L < 0", mm_scaled_gemm_batched(-3, 64, 64, 64, P, E4, 64, 4096, P, E4, 64, 4096, S, S, nullptr,
                                                     P, BF, 64, 4096, 0, nullptr));
    rejected("batched stride < 0", mm_scaled_gemm_batched(2, 64, 64, 64, P, E4, 64, -4096, P, E4, 64, 4096, S, S,
                                                          nullptr, P, BF, 64, 4096, 0, nullptr));
    rejected("batched stride not 16-byte", mm_scaled_gemm_batched(2, 64, 64, 64, P, E4, 64, 4104, P, E4, 64, 4096, S,
                                                                  S, nullptr, P, BF, 64, 4096, 0, nullptr));
    nothing("batched L = 0", mm_scaled_gemm_batched(0, 64, 64, 64, P, E4, 64, 4096, P, E4, 64, 4096, S, S, nullptr, P,
                                                    BF, 64, 4096, 0, nullptr));
    rejected("grouped G < 0", mm_scaled_gemm_grouped(64, 64, 64, -1, P, E4, 64, P, E4, 64, 4096, G32, G32, S, S,
                                                     nullptr, P, BF, 64, 0, nullptr));
    rejected("grouped sizes null", mm_scaled_gemm_grouped(64, 64, 64, 2, P, E4, 64, P, E4, 64, 4096, nullptr, G32, S,
                                                          S, nullptr, P, BF, 64, 0, nullptr));
    rejected("transpose R < 0", mm_transpose_u8(1, -5, 64, P, 64, 4096, P, 64, 4096, nullptr));
    rejected("transpose ld_dst < R", mm_transpose_u8(1, 128, 64, P, 64, 8192, P, 64, 8192, nullptr));
    nothing("transpose C = 0", mm_transpose_u8(1, 64, 0, P, 64, 4096, P, 64, 4096, nullptr));
    uint64_t bytes = 1;
    rejected("workspace N < 0", mm_grouped_workspace_bytes(64, -1, 64, 2, 0, 0, &bytes));
    rejected("workspace bytes null", mm_grouped_workspace_bytes(64, 64, 64, 2, 0, 0, nullptr));
    const struct { int ta, tb; } lay[4] = {{0, 1}, {0, 0}, {1, 0}, {1, 1}};
    for (auto l : lay) {
        ++g_cases;
        const mm_status st = mm_grouped_workspace_bytes(1000, 96, 136, 5, l.ta, l.tb, &bytes);
        const bool nt = l.ta == 0 && l.tb == 1;
        if (st != MM_OK || (nt ? bytes != 0 : bytes == 0)) {
            std::printf("FAIL workspace layout (%d, %d): status %d, bytes %llu\n", l.ta, l.tb, (int)st,
                        (unsigned long long)bytes);
            ++g_failures;
        }
    }
    rejected("layout bad flag", mm_scaled_gemm_grouped_layout(64, 64, 64, 2, 2, 0, P, E4, 64, P, E4, 64, 4096, G32,
                                                              G32, S, S, nullptr, P, BF, 64, 4096, P, 1 << 20, 0,
                                                              nullptr));
    rejected("layout workspace short", mm_scaled_gemm_grouped_layout(64, 64, 64, 2, 0, 0, P, E4, 64, P, E4, 64, 4096,
                                                                     G32, G32, S, S, nullptr, P, BF, 64, 4096, P, 16,
                                                                     0, nullptr));
    rejected("noalloc bad flag", mm_scaled_gemm_grouped_layout_noalloc(64, 64, 64, 2, 0, 7, P, E4, 64, P, E4, 64,
                                                                       4096, G32, G32, S, S, nullptr, P, BF, 64, 4096,
                                                                       0, nullptr));
    rejected("noalloc beyond the scratch array",
             mm_scaled_gemm_grouped_layout_noalloc(1 << 20, 8192, 8192, 4, 1, 0, P, E4, 8192, P, E4, 8192, 0, G32,
                                                   G32, S, S, nullptr, P, BF, 8192, 8192LL * 8192, 0, nullptr));
    rejected("amax sf_vec", mm_blockscaled_gemm_amax(128, 128, 128, 1, P, P, E4, S, S, 7, P, MM_F32, S,
                                                     reinterpret_cast<int64_t*>(P), nullptr));
    rejected("amax FP8 C with FP8 operands", mm_blockscaled_gemm_amax(128, 128, 128, 1, P, P, E4, S, S, 32, P,
                                                                      MM_F8_E4M3FN, S, nullptr, nullptr));
    rejected("amax L < 0", mm_blockscaled_gemm_amax(128, 128, 128, -1, P, P, E4, S, S, 32, P, MM_F32, S, nullptr,
                                                    nullptr));
    rejected("atom sf_type", mm_blockscaled_gemm_amax_atom(128, 128, 128, 1, P, P, E4, P, P, 9, 32, P, MM_F32, S,
                                                           nullptr, nullptr));
    rejected("atom FP4 sf 16 E8M0 with K odd", mm_blockscaled_gemm_amax_atom(128, 128, 33, 1, P, P, MM_F4_E2M1, P, P,
                                                                             MM_SF_E8M0, 16, P, MM_F32, S, nullptr,
                                                                             nullptr));
    rejected("debug convert dtype", mm_debug_convert(S, P, 77, 64, nullptr));
    rejected("debug mfma M % 16", mm_debug_mfma_gemm(17, 16, 128, P, P, E4, nullptr, nullptr, S, nullptr));
    rejected("debug mfma type", mm_debug_mfma_gemm(16, 16, 128, P, P, MM_BF16, nullptr, nullptr, S, nullptr));
    ++g_cases;
    if (std::strlen(mm_version()) == 0) {
        std::printf("FAIL version\n");
        ++g_failures;
    }
    std::printf("%d cases, %d failures\n", g_cases, g_failures);
    return g_failures ? 1 : 0;
}
