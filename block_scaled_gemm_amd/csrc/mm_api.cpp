// mm_api.cpp -- the C ABI of libmmfp8 (declared in include/mm.h): argument
// validation (complete before any HIP call), kernel choice and launch.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <string>

#include "mm.h"
#include "mm_launch.hpp"

namespace {

thread_local std::string g_error;

mm_status fail(mm_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mm_status fail(mm_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool is_fp8(int t) { return t == MM_F8_E4M3FN || t == MM_F8_E5M2; }
bool is_dtype(int t) { return t >= MM_F8_E4M3FN && t <= MM_F16; }
int elem_size(int t) { return t == MM_F32 ? 4 : (t == MM_BF16 || t == MM_F16) ? 2 : 1; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kMaxDim = (int64_t)1 << 31;   // M, N, K, L < 2^31
constexpr int64_t kMaxPitch = (int64_t)1 << 22; // row pitch in bytes (buffer offsets stay below 2^31)

// Test hook: MM_TEST_FORCE_FAIL=launch makes a valid call return MM_ERR_DEVICE
// right after validation, before any HIP call, so the device-error path can be
// exercised without a GPU.
bool forced_launch_failure() {
    const char* e = std::getenv("MM_TEST_FORCE_FAIL");
    return e && std::strstr(e, "launch") != nullptr;
}

// Compute units of the current device (cached per device).
int cu_count() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// Largest workgroup tile (not larger than `first`) that still gives every
// compute unit a tile.
int choose_cfg(int64_t M, int64_t N, int64_t L, int cus, int first) {
    for (int c = first; c < mmfp8::CFG_COUNT - 1; ++c) {
        const int64_t tiles = cdiv(M, mmfp8::kCfgBM[c]) * cdiv(N, mmfp8::kCfgBN[c]) * L;
        if (tiles >= cus) return c;
    }
    return mmfp8::CFG_64x64;
}

// Columns of the product that the 256x256 row-chunk tiles take (slow accumulation, or block scaling with a
// 128x128 scale_b): 0 for none, N for all, or a multiple of 256 whose tiles fill whole rounds of the CUs, the
// other columns then going to the usual tiles in a second launch. Each plan is priced in rounds: one 256x256
// tile per CU counts 1000, two 128x128 tiles per CU 565 (their measured times per round; the row-chunk loop
// does about 13% more per clock, but one tile per CU leaves a partial last round half idle), a second launch
// 250.
int64_t rc_columns(int64_t M, int64_t N, int64_t L, int64_t cus) {
    const int64_t tm = cdiv(M, 256) * L;  // 256-row tiles over the batch
    const int64_t t256 = tm * cdiv(N, 256);
    if (t256 < cus) return 0;
    auto r128 = [&](int64_t cols) { return cdiv(cdiv(M, 128) * cdiv(cols, 128) * L, 2 * cus) * 565; };
    int64_t best = r128(N), cols = 0;
    if (cdiv(t256, cus) * 1000 < best) {
        best = cdiv(t256, cus) * 1000;
        cols = N;
    }
    const int64_t c = t256 / cus * cus / tm;  // 256-column blocks that whole rounds cover
    if (c > 0 && c * 256 < N && cdiv(tm * c, cus) * 1000 + 250 + r128(N - c * 256) < best) cols = c * 256;
    return cols;
}

mm_status device_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return MM_OK;
    return fail(MM_ERR_DEVICE, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

}  // namespace

int mmfp8::device_cus() { return cu_count(); }

extern "C" {

const char* mm_last_error(void) { return g_error.c_str(); }

const char* mm_version(void) { return "mmfp8 0.1.0 gfx950"; }

}  // extern "C"

namespace {

// The dense FP8 GEMM behind mm_scaled_gemm, mm_scaled_gemm_bias,
// mm_scaled_gemm_batched and mm_scaled_gemm_grouped: L items (L = 1 for the
// first two) at byte strides stride_a / stride_b and element stride stride_d,
// an optional bias [N]; or, grouped, G groups packed along M (L = 1), group
// g's b at g * stride_b bytes, rows and first rows in gsizes / goffsets.
mm_status scaled_gemm(const char* who, int64_t L, int64_t M, int64_t N, int64_t K, const void* a, int a_type,
                      int64_t lda, int64_t stride_a, const void* b, int b_type, int64_t ldb, int64_t stride_b,
                      const float* scale_a, int sa_mode, const float* scale_b, int sb_mode, const float* scale_result,
                      const void* bias, void* d, int d_type, int64_t ldd, int64_t stride_d, int use_fast_accum,
                      void* stream, bool grouped = false, int64_t G = 0, const int32_t* gsizes = nullptr,
                      const int32_t* goffsets = nullptr,
                      const std::function<hipError_t(hipStream_t)>& pre = {}) {
    g_error.clear();
    if (L < 0 || M < 0 || N < 0 || K < 0)
        return fail(MM_ERR_INVALID_ARGUMENT, "L, M, N and K must be >= 0 (got %lld, %lld, %lld, %lld)", (long long)L,
                    (long long)M, (long long)N, (long long)K);
    if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim || L >= kMaxDim)
        return fail(MM_ERR_UNSUPPORTED, "L, M, N and K must be below 2^31");
    if (!is_fp8(a_type) || !is_fp8(b_type))
        return fail(MM_ERR_INVALID_ARGUMENT, "a_type and b_type must be MM_F8_E4M3FN or MM_F8_E5M2 (got %d, %d)",
                    a_type, b_type);
    if (!is_dtype(d_type)) return fail(MM_ERR_INVALID_ARGUMENT, "unknown d_type %d", d_type);
    if (sa_mode < MM_SCALE_TENSOR || sa_mode > MM_SCALE_128x128 || sb_mode < MM_SCALE_TENSOR ||
        sb_mode > MM_SCALE_128x128)
        return fail(MM_ERR_INVALID_ARGUMENT, "unknown scale mode (%d, %d)", sa_mode, sb_mode);
    const bool per_tensor = sa_mode == MM_SCALE_TENSOR && sb_mode == MM_SCALE_TENSOR;
    const bool block = sa_mode == MM_SCALE_1x128 && (sb_mode == MM_SCALE_1x128 || sb_mode == MM_SCALE_128x128);
    if (!per_tensor && !block)
        return fail(MM_ERR_UNSUPPORTED,
                    "scale pair (%d, %d) not supported: use (TENSOR, TENSOR), (1x128, 1x128) or (1x128, 128x128)",
                    sa_mode, sb_mode);
    if (lda < K || ldb < K) return fail(MM_ERR_INVALID_ARGUMENT, "lda and ldb must be >= K");
    if (ldd < N) return fail(MM_ERR_INVALID_ARGUMENT, "ldd must be >= N");
    if (lda > kMaxPitch || ldb > kMaxPitch) return fail(MM_ERR_UNSUPPORTED, "lda and ldb must be at most 2^22 bytes");
    if (stride_a < 0 || stride_b < 0 || stride_d < 0)
        return fail(MM_ERR_INVALID_ARGUMENT, "batch strides must be >= 0");
    if (bias && is_fp8(d_type))
        return fail(MM_ERR_UNSUPPORTED, "a bias needs an f32, bf16 or f16 output (got d_type %d)", d_type);
    // (the workgroup count is checked against 2^31 below; 64x64 tiles are the smallest)
    if (L > 0 && cdiv(M, 64) * cdiv(N, 64) >= kMaxDim / L) return fail(MM_ERR_UNSUPPORTED, "too many output tiles");
    if (G < 0) return fail(MM_ERR_INVALID_ARGUMENT, "the group count must be >= 0");
    if (G >= kMaxDim || (cdiv(M, 64) + G) * cdiv(N, 64) >= kMaxDim)
        return fail(MM_ERR_UNSUPPORTED, "too many groups or output tiles");
    if (L == 0 || M == 0 || N == 0) return MM_OK;
    if (grouped && G > 0 && (!gsizes || !goffsets))
        return fail(MM_ERR_INVALID_ARGUMENT, "batch_sizes or batch_offsets is NULL");
    if (!aligned(gsizes, 4) || !aligned(goffsets, 4))
        return fail(MM_ERR_MISALIGNED, "batch_sizes and batch_offsets must be 4-byte aligned");
    if (!d) return fail(MM_ERR_INVALID_ARGUMENT, "d is NULL");
    if (K > 0 && (!a || !b)) return fail(MM_ERR_INVALID_ARGUMENT, "a or b is NULL");
    if ((per_tensor || K > 0) && (!scale_a || !scale_b)) return fail(MM_ERR_INVALID_ARGUMENT, "scale_a or scale_b is NULL");
    if (!aligned(a, 16) || !aligned(b, 16)) return fail(MM_ERR_MISALIGNED, "a and b must be 16-byte aligned");
    if (lda % 8 || ldb % 8) return fail(MM_ERR_MISALIGNED, "lda and ldb must be multiples of 8 bytes");
    if ((L > 1 || G > 1) && (stride_a % 16 || stride_b % 16))
        return fail(MM_ERR_MISALIGNED, "stride_a and stride_b must be multiples of 16 bytes");
    if (!aligned(d, elem_size(d_type))) return fail(MM_ERR_MISALIGNED, "d must be aligned to its element size");
    if (!aligned(bias, elem_size(d_type))) return fail(MM_ERR_MISALIGNED, "bias must be aligned to its element size");
    if (!aligned(scale_a, 4) || !aligned(scale_b, 4) || !aligned(scale_result, 4))
        return fail(MM_ERR_MISALIGNED, "scale pointers must be 4-byte aligned");
    if (grouped && G == 0) return MM_OK;  // no groups: no rows to compute
    if (forced_launch_failure()) return fail(MM_ERR_DEVICE, "launch failure forced by MM_TEST_FORCE_FAIL");

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (pre) {  // operand packing that the validated call needs first
        const hipError_t e = pre(s);
        if (e != hipSuccess) return device_status(e, who);
    }
    mmfp8::GemmArgs p{};
    p.a = static_cast<const uint8_t*>(a);
    p.b = static_cast<const uint8_t*>(b);
    p.lda = lda;
    p.ldb = ldb;
    p.a_batch = L > 1 ? stride_a : 0;
    p.b_batch = (L > 1 || G > 1) ? stride_b : 0;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.L = (int)L;
    p.sa = scale_a;
    p.sb = scale_b;
    const int64_t kb = cdiv(K, 128);
    p.sa_ld = kb;
    p.sb_ld = kb;
    p.scale_result = scale_result;
    p.bias = bias;
    p.d = d;
    p.ldd = ldd;
    p.d_batch = L > 1 ? stride_d : 0;
    p.d_type = d_type;
    const int es = elem_size(d_type);
    p.vec_store = (ldd % 4 == 0) && (p.d_batch % 4 == 0) && aligned(d, 4 * es);

    const int fa = a_type == MM_F8_E5M2 ? 1 : 0;
    const int fb = b_type == MM_F8_E5M2 ? 1 : 0;
    hipError_t e;
    if (grouped) {
        // groups: the tile kernel over ceil(M / BM) + G tile rows, each mapped to its group on the device
        // (partial tiles of each group; the rows past the groups' tiles leave at once)
        const int mode = use_fast_accum ? mmfp8::MODE_FAST : mmfp8::MODE_SLOW;
        const int cfg = choose_cfg(M, N, 1, cu_count(), mmfp8::min_cfg(mode, 0));
        p.groups = (int)G;
        p.grp_sizes = gsizes;
        p.grp_offsets = goffsets;
        p.tiles_m = (int)(cdiv(M, mmfp8::kCfgBM[cfg]) + G);
        p.tiles_n = (int)cdiv(N, mmfp8::kCfgBN[cfg]);
        const int64_t grid = (int64_t)p.tiles_m * p.tiles_n;
        e = use_fast_accum ? mmfp8::launch_tile_fast(cfg, fa, fb, p, (int)grid, s)
                           : mmfp8::launch_tile_slow(cfg, fa, fb, p, (int)grid, s);
        return device_status(e, who);
    }
    // the skinny and K-split kernels serve one item; batches go to the tiles
    if (per_tensor && L == 1 && M <= 64) {
        const int mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
        const int grid = (int)cdiv(N, 16);
        e = mmfp8::launch_skinny(mt, use_fast_accum ? mmfp8::MODE_FAST : mmfp8::MODE_SLOW, fa, fb, p, grid, s);
        return device_status(e, who);
    }
    const int mode = per_tensor ? (use_fast_accum ? mmfp8::MODE_FAST : mmfp8::MODE_SLOW) : mmfp8::MODE_BLOCK;
    const int sbm = sb_mode == MM_SCALE_128x128 ? mmfp8::SB_128x128 : mmfp8::SB_1x128;
    auto launch_tiles = [&](int c, mmfp8::GemmArgs& q, int64_t n) {
        q.tiles_m = (int)cdiv(M, mmfp8::kCfgBM[c]);
        q.tiles_n = (int)cdiv(n, mmfp8::kCfgBN[c]);
        const int grid = (int)((int64_t)q.tiles_m * q.tiles_n * L);
        if (!per_tensor) return mmfp8::launch_tile_block(c, sbm, fa, fb, q, grid, s);
        return use_fast_accum ? mmfp8::launch_tile_fast(c, fa, fb, q, grid, s)
                              : mmfp8::launch_tile_slow(c, fa, fb, q, grid, s);
    };
    int cfg = choose_cfg(M, N, L, cu_count(), mmfp8::min_cfg(mode, sbm));
    const bool rc = mode == mmfp8::MODE_SLOW || (mode == mmfp8::MODE_BLOCK && sbm == mmfp8::SB_128x128);
    if (rc && cfg == mmfp8::CFG_128x128) {
        const int64_t cols = rc_columns(M, N, L, cu_count());
        if (cols == N) {
            cfg = mmfp8::CFG_256x256;
        } else if (cols > 0) {
            // columns [0, cols) on 256x256 tiles, the rest on the tiles their own count gives
            mmfp8::GemmArgs q = p;
            q.N = (int)cols;
            e = launch_tiles(mmfp8::CFG_256x256, q, cols);
            if (e != hipSuccess) return device_status(e, who);
            p.b += cols * ldb;
            p.d = static_cast<uint8_t*>(d) + cols * es;
            if (bias) p.bias = static_cast<const uint8_t*>(bias) + cols * es;
            if (mode == mmfp8::MODE_BLOCK) p.sb += cols / 128 * p.sb_ld;
            N -= cols;
            p.N = (int)N;
            cfg = choose_cfg(M, N, L, cu_count(), mmfp8::min_cfg(mode, sbm));
        }
    }
    if (per_tensor && L == 1 && cfg == mmfp8::CFG_64x64) {
        // too few 128x128 tiles to fill the chip: K split over the waves of 64x64 / 32x64 tiles
        const int ks = cdiv(M, 64) * cdiv(N, 64) >= cu_count() ? mmfp8::KS_64x64 : mmfp8::KS_32x64;
        p.tiles_m = (int)cdiv(M, mmfp8::kKsBM[ks]);
        p.tiles_n = (int)cdiv(N, mmfp8::kKsBN[ks]);
        const int64_t grid = (int64_t)p.tiles_m * p.tiles_n;
        e = mmfp8::launch_ksplit(ks, mode, fa, fb, p, (int)grid, s);
        return device_status(e, who);
    }
    e = launch_tiles(cfg, p, N);
    return device_status(e, who);
}

}  // namespace

extern "C" {

mm_status mm_scaled_gemm(int64_t M, int64_t N, int64_t K, const void* a, int a_type, int64_t lda, const void* b,
                         int b_type, int64_t ldb, const float* scale_a, int sa_mode, const float* scale_b,
                         int sb_mode, const float* scale_result, void* d, int d_type, int64_t ldd,
                         int use_fast_accum, void* stream) {
    return scaled_gemm("mm_scaled_gemm launch", 1, M, N, K, a, a_type, lda, 0, b, b_type, ldb, 0, scale_a, sa_mode,
                       scale_b, sb_mode, scale_result, nullptr, d, d_type, ldd, 0, use_fast_accum, stream);
}

mm_status mm_scaled_gemm_bias(int64_t M, int64_t N, int64_t K, const void* a, int a_type, int64_t lda, const void* b,
                              int b_type, int64_t ldb, const float* scale_a, int sa_mode, const float* scale_b,
                              int sb_mode, const void* bias, void* d, int d_type, int64_t ldd, int use_fast_accum,
                              void* stream) {
    return scaled_gemm("mm_scaled_gemm_bias launch", 1, M, N, K, a, a_type, lda, 0, b, b_type, ldb, 0, scale_a,
                       sa_mode, scale_b, sb_mode, nullptr, bias, d, d_type, ldd, 0, use_fast_accum, stream);
}

mm_status mm_scaled_gemm_batched(int64_t L, int64_t M, int64_t N, int64_t K, const void* a, int a_type, int64_t lda,
                                 int64_t stride_a, const void* b, int b_type, int64_t ldb, int64_t stride_b,
                                 const float* scale_a, const float* scale_b, const float* scale_result, void* d,
                                 int d_type, int64_t ldd, int64_t stride_d, int use_fast_accum, void* stream) {
    return scaled_gemm("mm_scaled_gemm_batched launch", L, M, N, K, a, a_type, lda, stride_a, b, b_type, ldb,
                       stride_b, scale_a, MM_SCALE_TENSOR, scale_b, MM_SCALE_TENSOR, scale_result, nullptr, d, d_type,
                       ldd, stride_d, use_fast_accum, stream);
}

}  // extern "C"

namespace {

// The batched MX GEMM + amax behind both entry points; `atom` selects the
// page-native E8M0 bytes (FP8 or FP4 operands) over fp32 factors (FP8).
mm_status blockscaled_amax(const char* who, int64_t M, int64_t N, int64_t K, int64_t L, const void* a,
                           const void* b, int ab_type, const void* sfa, const void* sfb, bool atom, int sf_vec_size,
                           void* c, int c_type, float* amax, int64_t* amax_index, void* stream,
                           bool e4m3_factors = false) {
    if (M < 0 || N < 0 || K < 0 || L < 0)
        return fail(MM_ERR_INVALID_ARGUMENT, "M, N, K and L must be >= 0");
    if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim || L >= kMaxDim)
        return fail(MM_ERR_UNSUPPORTED, "M, N, K and L must be below 2^31");
    const int64_t lim = (int64_t)1 << 48;
    if ((K && L * M > lim / K) || (K && L * N > lim / K) || (N && L * M > lim / N))
        return fail(MM_ERR_UNSUPPORTED, "L*M*K, L*N*K and L*M*N must be below 2^48");
    const bool fp4 = ab_type == MM_F4_E2M1;
    if (fp4 && !atom)
        return fail(MM_ERR_UNSUPPORTED, "FP4 operands take E8M0 factors in the page's layout (the _atom entry)");
    if (!is_fp8(ab_type) && !fp4)
        return fail(MM_ERR_INVALID_ARGUMENT, "ab_type must be MM_F8_E4M3FN, MM_F8_E5M2%s", atom ? " or MM_F4_E2M1" : "");
    if (sf_vec_size == 16 && !fp4)
        return fail(MM_ERR_UNSUPPORTED, "sf_vec_size 16 is not supported with FP8 operands; use 32");
    if (sf_vec_size != 32 && sf_vec_size != 16)
        return fail(MM_ERR_INVALID_ARGUMENT, "sf_vec_size must be 32%s (got %d)", fp4 ? " or 16" : "", sf_vec_size);
    if (e4m3_factors && (!fp4 || sf_vec_size != 16))
        return fail(MM_ERR_UNSUPPORTED, "E4M3 scale factors need FP4 operands and sf_vec_size 16");
    if (is_fp8(c_type) && !fp4) return fail(MM_ERR_UNSUPPORTED, "FP8 C with FP8 operands is not supported");
    if (c_type == MM_F4_E2M1 && !fp4) return fail(MM_ERR_UNSUPPORTED, "FP4 C needs FP4 operands");
    if (!is_dtype(c_type) && c_type != MM_F4_E2M1) return fail(MM_ERR_INVALID_ARGUMENT, "unknown c_type %d", c_type);
    if (K > kMaxPitch) return fail(MM_ERR_UNSUPPORTED, "K must be at most 2^22");
    const int64_t outs = L * M * N;
    if (amax_index && outs >= ((int64_t)1 << 33))
        return fail(MM_ERR_UNSUPPORTED, "amax_index needs L*M*N < 2^33");
    if (outs > 0 && !c) return fail(MM_ERR_INVALID_ARGUMENT, "c is NULL");
    if (outs > 0 && K > 0 && (!a || !b || !sfa || !sfb))
        return fail(MM_ERR_INVALID_ARGUMENT, "a, b, sfa or sfb is NULL");
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 16))
        return fail(MM_ERR_MISALIGNED, "a, b and c must be 16-byte aligned");
    if (K % (fp4 ? 32 : 16))
        return fail(MM_ERR_MISALIGNED, "K must be a multiple of %d (16-byte aligned rows)", fp4 ? 32 : 16);
    if (!aligned(sfa, 4) || !aligned(sfb, 4) || !aligned(amax, 4))
        return fail(MM_ERR_MISALIGNED, "sfa, sfb and amax must be 4-byte aligned");
    if (!aligned(amax_index, 8)) return fail(MM_ERR_MISALIGNED, "amax_index must be 8-byte aligned");
    const int64_t groups = cdiv(K, sf_vec_size), kblocks = cdiv(groups, 4);
    if (atom && (cdiv(M, 128) * kblocks * 512 >= kMaxDim || cdiv(N, 128) * kblocks * 512 >= kMaxDim))
        return fail(MM_ERR_UNSUPPORTED, "each batch item's scale-factor tensor must be below 2^31 bytes");
    if (outs == 0 && !amax && !amax_index) return MM_OK;
    if (forced_launch_failure()) return fail(MM_ERR_DEVICE, "launch failure forced by MM_TEST_FORCE_FAIL");

    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t* amax_bits = amax_index ? nullptr : reinterpret_cast<uint32_t*>(amax);
    unsigned long long* key = reinterpret_cast<unsigned long long*>(amax_index);
    if (amax || amax_index) {
        mm_status st = device_status(mmfp8::launch_amax_init(amax_bits, key, s), "amax init launch");
        if (st != MM_OK) return st;
    }
    if (outs > 0) {
        const int64_t kbytes = fp4 ? K / 2 : K;  // operand row in bytes
        mmfp8::GemmArgs p{};
        p.a = static_cast<const uint8_t*>(a);
        p.b = static_cast<const uint8_t*>(b);
        p.lda = kbytes;
        p.ldb = kbytes;
        p.a_batch = M * kbytes;
        p.b_batch = N * kbytes;
        p.M = (int)M;
        p.N = (int)N;
        p.K = (int)kbytes;  // the kernels load K bytes per row
        p.L = (int)L;
        p.sa = static_cast<const float*>(sfa);
        p.sb = static_cast<const float*>(sfb);
        p.sa_ld = groups;
        p.sb_ld = groups;
        if (atom) {  // 4-byte units: 128 per 128 rows and 4 groups
            p.sa_batch = cdiv(M, 128) * kblocks * 128;
            p.sb_batch = cdiv(N, 128) * kblocks * 128;
        } else {
            p.sa_batch = M * groups;
            p.sb_batch = N * groups;
        }
        p.d = c;
        // FP4 C: rows of ceil(N/2) bytes, so the pitch in elements is N rounded up to even
        p.ldd = c_type == MM_F4_E2M1 ? N + (N & 1) : N;
        p.d_batch = M * p.ldd;
        p.d_type = c_type;
        p.vec_store = (p.ldd % 4 == 0);
        p.amax_bits = amax_bits;
        p.amax_key = key;
        const int layout = !atom                ? mmfp8::SF_F32
                           : e4m3_factors       ? mmfp8::SF_ATOM_E4M3_16
                           : sf_vec_size == 16  ? mmfp8::SF_ATOM_E8M0_16
                                                : mmfp8::SF_ATOM_E8M0;
        const int cfg = choose_cfg(M, N, L, cu_count(), mmfp8::min_cfg(mmfp8::MODE_SF32, layout, ab_type));
        p.tiles_m = (int)cdiv(M, mmfp8::kCfgBM[cfg]);
        p.tiles_n = (int)cdiv(N, mmfp8::kCfgBN[cfg]);
        const int64_t grid = (int64_t)p.tiles_m * p.tiles_n * L;
        if (grid >= kMaxDim) return fail(MM_ERR_UNSUPPORTED, "too many output tiles");
        const hipError_t e = fp4 ? mmfp8::launch_tile_fp4(cfg, layout, p, (int)grid, s)
                                 : mmfp8::launch_tile_sf32(cfg, layout, ab_type == MM_F8_E5M2 ? 1 : 0, p, (int)grid, s);
        mm_status st = device_status(e, who);
        if (st != MM_OK) return st;
    }
    if (amax_index) return device_status(mmfp8::launch_amax_finalize(amax, key, s), "amax finalize launch");
    return MM_OK;
}

}  // namespace

extern "C" {

mm_status mm_scaled_gemm_grouped(int64_t batch_sum, int64_t N, int64_t K, int64_t G, const void* a, int a_type,
                                 int64_t lda, const void* b, int b_type, int64_t ldb, int64_t stride_b,
                                 const int32_t* batch_sizes, const int32_t* batch_offsets, const float* scale_a,
                                 const float* scale_b, const float* scale_result, void* d, int d_type, int64_t ldd,
                                 int use_fast_accum, void* stream) {
    return scaled_gemm("mm_scaled_gemm_grouped launch", 1, batch_sum, N, K, a, a_type, lda, 0, b, b_type, ldb,
                       stride_b, scale_a, MM_SCALE_TENSOR, scale_b, MM_SCALE_TENSOR, scale_result, nullptr, d, d_type,
                       ldd, 0, use_fast_accum, stream, true, G, batch_sizes, batch_offsets);
}

mm_status mm_blockscaled_gemm_amax(int64_t M, int64_t N, int64_t K, int64_t L, const void* a, const void* b,
                                   int ab_type, const float* sfa, const float* sfb, int sf_vec_size, void* c,
                                   int c_type, float* amax, int64_t* amax_index, void* stream) {
    g_error.clear();
    return blockscaled_amax("mm_blockscaled_gemm_amax launch", M, N, K, L, a, b, ab_type, sfa, sfb, false,
                            sf_vec_size, c, c_type, amax, amax_index, stream);
}

mm_status mm_blockscaled_gemm_amax_atom(int64_t M, int64_t N, int64_t K, int64_t L, const void* a, const void* b,
                                        int ab_type, const void* sfa, const void* sfb, int sf_type,
                                        int sf_vec_size, void* c, int c_type, float* amax, int64_t* amax_index,
                                        void* stream) {
    g_error.clear();
    if (sf_type != MM_SF_E8M0 && sf_type != MM_SF_E4M3FN)
        return fail(MM_ERR_INVALID_ARGUMENT, "unknown sf_type %d", sf_type);
    return blockscaled_amax("mm_blockscaled_gemm_amax_atom launch", M, N, K, L, a, b, ab_type, sfa, sfb, true,
                            sf_vec_size, c, c_type, amax, amax_index, stream, sf_type == MM_SF_E4M3FN);
}

mm_status mm_debug_convert(const float* x, void* y, int dtype, int64_t n, void* stream) {
    g_error.clear();
    if (n < 0) return fail(MM_ERR_INVALID_ARGUMENT, "n must be >= 0");
    if (!is_dtype(dtype)) return fail(MM_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    if (n >= ((int64_t)1 << 40)) return fail(MM_ERR_UNSUPPORTED, "n too large");
    if (n == 0) return MM_OK;
    if (!x || !y) return fail(MM_ERR_INVALID_ARGUMENT, "x or y is NULL");
    if (!aligned(x, 4) || !aligned(y, elem_size(dtype))) return fail(MM_ERR_MISALIGNED, "x or y misaligned");
    if (forced_launch_failure()) return fail(MM_ERR_DEVICE, "launch failure forced by MM_TEST_FORCE_FAIL");
    return device_status(mmfp8::launch_debug_convert(x, y, dtype, n, static_cast<hipStream_t>(stream)),
                         "mm_debug_convert launch");
}

mm_status mm_debug_mfma_gemm(int64_t M, int64_t N, int64_t K, const void* a, const void* b, int ab_type,
                             const void* sfa, const void* sfb, float* d, void* stream) {
    g_error.clear();
    if (M < 0 || N < 0 || K < 0) return fail(MM_ERR_INVALID_ARGUMENT, "M, N and K must be >= 0");
    if (!is_fp8(ab_type) && ab_type != MM_F4_E2M1) return fail(MM_ERR_INVALID_ARGUMENT, "unknown ab_type %d", ab_type);
    if (M % 16 || N % 16 || K % 128) return fail(MM_ERR_UNSUPPORTED, "M and N must be multiples of 16, K of 128");
    if (M >= (1 << 20) || N >= (1 << 20) || K >= (1 << 22)) return fail(MM_ERR_UNSUPPORTED, "M, N or K too large");
    if (M == 0 || N == 0) return MM_OK;
    if (!d || (K > 0 && (!a || !b))) return fail(MM_ERR_INVALID_ARGUMENT, "a, b or d is NULL");
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 4)) return fail(MM_ERR_MISALIGNED, "a and b must be 16-byte aligned");
    if (forced_launch_failure()) return fail(MM_ERR_DEVICE, "launch failure forced by MM_TEST_FORCE_FAIL");
    const int fmt = ab_type == MM_F8_E4M3FN ? 0 : (ab_type == MM_F8_E5M2 ? 1 : 4);
    return device_status(mmfp8::launch_debug_mfma_gemm(fmt, static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(b),
                                                       static_cast<const uint8_t*>(sfa), static_cast<const uint8_t*>(sfb),
                                                       d, (int)M, (int)N, (int)K, static_cast<hipStream_t>(stream)),
                         "mm_debug_mfma_gemm launch");
}

}  // extern "C"

// ------------------------------------------------------------------ layouts with packing
//
// "TileOPs: Linear Algebra Operators": BmmFP8FwdOp accepts b as [B, K, N] and
// GroupedGemmFwdOp has the NN, TN and TT layouts besides NT. The kernels read
// the contraction innermost; other operands are packed first (mm_pack.hip).

namespace {

int64_t round16(int64_t x) { return (x + 15) & ~(int64_t)15; }

// The packing grid: ceil(R/64) x ceil(C/64) x L workgroups of 256 lanes.
bool pack_fits(int64_t L, int64_t R, int64_t C) {
    return L < 65536 && cdiv(C, 64) < 65536 && R < ((int64_t)1 << 30);
}

// Pitch of the packed operands when groups split the contraction: every
// group's start rounded up to 16 bytes fits in it whatever the sizes.
int64_t kgroup_pitch(int64_t batch_sum, int64_t G) { return round16(batch_sum) + 16 * G; }

struct KGroupWs {
    size_t start, a, b, total;
};

KGroupWs kgroup_ws(int64_t batch_sum, int64_t N, int64_t K, int64_t G) {
    const auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t P = (size_t)kgroup_pitch(batch_sum, G);
    KGroupWs w{};
    w.start = 0;
    w.a = up(8 * (size_t)G);
    w.b = w.a + up((size_t)N * P);
    w.total = w.b + (size_t)K * P;
    return w;
}

}  // namespace

extern "C" {

mm_status mm_transpose_u8(int64_t L, int64_t R, int64_t C, const void* src, int64_t ld_src, int64_t stride_src,
                          void* dst, int64_t ld_dst, int64_t stride_dst, void* stream) {
    g_error.clear();
    if (L < 0 || R < 0 || C < 0) return fail(MM_ERR_INVALID_ARGUMENT, "L, R and C must be >= 0");
    if (ld_src < C || ld_dst < R) return fail(MM_ERR_INVALID_ARGUMENT, "ld_src must be >= C and ld_dst >= R");
    if (stride_src < 0 || stride_dst < 0) return fail(MM_ERR_INVALID_ARGUMENT, "batch strides must be >= 0");
    if (!pack_fits(L, R, C))
        return fail(MM_ERR_UNSUPPORTED, "L must be below 2^16, C below 2^22 and R below 2^30");
    if (L == 0 || R == 0 || C == 0) return MM_OK;
    if (!src || !dst) return fail(MM_ERR_INVALID_ARGUMENT, "src or dst is NULL");
    if (forced_launch_failure()) return fail(MM_ERR_DEVICE, "launch failure forced by MM_TEST_FORCE_FAIL");
    return device_status(mmfp8::launch_transpose(static_cast<const uint8_t*>(src), L, R, C, ld_src, stride_src,
                                                 static_cast<uint8_t*>(dst), ld_dst, stride_dst,
                                                 static_cast<hipStream_t>(stream)),
                         "mm_transpose_u8 launch");
}

mm_status mm_grouped_workspace_bytes(int64_t batch_sum, int64_t N, int64_t K, int64_t G, int transpose_a,
                                     int transpose_b, uint64_t* bytes) {
    g_error.clear();
    if (!bytes) return fail(MM_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (batch_sum < 0 || N < 0 || K < 0 || G < 0)
        return fail(MM_ERR_INVALID_ARGUMENT, "batch_sum, N, K and G must be >= 0");
    if (batch_sum >= kMaxDim || N >= kMaxDim || K >= kMaxDim || G >= kMaxDim)
        return fail(MM_ERR_UNSUPPORTED, "batch_sum, N, K and G must be below 2^31");
    if (transpose_a) *bytes = (G == 0 || N == 0 || K == 0) ? 0 : kgroup_ws(batch_sum, N, K, G).total;
    else *bytes = transpose_b ? 0 : (uint64_t)G * (uint64_t)N * (uint64_t)round16(K);
    return MM_OK;
}

mm_status mm_scaled_gemm_grouped_layout(int64_t batch_sum, int64_t N, int64_t K, int64_t G, int transpose_a,
                                        int transpose_b, const void* a, int a_type, int64_t lda, const void* b,
                                        int b_type, int64_t ldb, int64_t stride_b, const int32_t* batch_sizes,
                                        const int32_t* batch_offsets, const float* scale_a, const float* scale_b,
                                        const float* scale_result, void* d, int d_type, int64_t ldd,
                                        int64_t stride_d, void* workspace, uint64_t workspace_bytes,
                                        int use_fast_accum, void* stream) {
    g_error.clear();
    if ((transpose_a != 0 && transpose_a != 1) || (transpose_b != 0 && transpose_b != 1))
        return fail(MM_ERR_INVALID_ARGUMENT, "transpose_a and transpose_b must be 0 or 1");
    if (!transpose_a && transpose_b)  // NT: the operands are already contraction-innermost
        return mm_scaled_gemm_grouped(batch_sum, N, K, G, a, a_type, lda, b, b_type, ldb, stride_b, batch_sizes,
                                      batch_offsets, scale_a, scale_b, scale_result, d, d_type, ldd,
                                      use_fast_accum, stream);
    uint64_t need = 0;
    if (const mm_status st = mm_grouped_workspace_bytes(batch_sum, N, K, G, transpose_a, transpose_b, &need))
        return st;
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(MM_ERR_INVALID_ARGUMENT, "the workspace needs %llu bytes (got %llu%s)", (unsigned long long)need,
                    (unsigned long long)workspace_bytes, workspace ? "" : ", NULL");
    if (!aligned(workspace, 16)) return fail(MM_ERR_MISALIGNED, "the workspace must be 16-byte aligned");
    uint8_t* ws = static_cast<uint8_t*>(workspace);

    if (!transpose_a) {
        // NN: b [G][K][ldb] (N used) packed to [G][N][round16(K)], then the NT grouped GEMM
        if (ldb < N) return fail(MM_ERR_INVALID_ARGUMENT, "ldb must be >= N (b is [G][K][ldb] under NN)");
        if (stride_b < 0) return fail(MM_ERR_INVALID_ARGUMENT, "stride_b must be >= 0");
        if (!pack_fits(G, K, N))
            return fail(MM_ERR_UNSUPPORTED, "NN packing: G must be below 2^16, N below 2^22 and K below 2^30");
        const int64_t kp = round16(K);
        if (kp > kMaxPitch) return fail(MM_ERR_UNSUPPORTED, "NN packing: K must be at most 2^22 bytes");
        if (G > 0 && N > 0 && K > 0 && !b) return fail(MM_ERR_INVALID_ARGUMENT, "b is NULL");
        const auto pack = [=](hipStream_t s) {
            return mmfp8::launch_transpose(static_cast<const uint8_t*>(b), G, K, N, ldb, stride_b, ws, kp, N * kp, s);
        };
        return scaled_gemm("mm_scaled_gemm_grouped_layout launch", 1, batch_sum, N, K, a, a_type, lda, 0,
                           (G > 0 && N > 0 && K > 0) ? ws : b, b_type, kp, N * kp, scale_a, MM_SCALE_TENSOR,
                           scale_b, MM_SCALE_TENSOR, scale_result, nullptr, d, d_type, ldd, 0, use_fast_accum,
                           stream, true, G, batch_sizes, batch_offsets,
                           (G > 0 && N > 0 && K > 0) ? std::function<hipError_t(hipStream_t)>(pack)
                                                     : std::function<hipError_t(hipStream_t)>());
    }

    // TN / TT: the groups split the contraction; group g's [N][K] block is A_g^T B_g over its rows
    if (!is_fp8(a_type) || !is_fp8(b_type))
        return fail(MM_ERR_INVALID_ARGUMENT, "a_type and b_type must be MM_F8_E4M3FN or MM_F8_E5M2 (got %d, %d)",
                    a_type, b_type);
    if (!is_dtype(d_type)) return fail(MM_ERR_INVALID_ARGUMENT, "unknown d_type %d", d_type);
    if (lda < N) return fail(MM_ERR_INVALID_ARGUMENT, "lda must be >= N (a is [batch_sum][lda] with transpose_a)");
    if (transpose_b ? ldb < batch_sum : ldb < K)
        return fail(MM_ERR_INVALID_ARGUMENT, "ldb must be >= %s (b is %s)", transpose_b ? "batch_sum" : "K",
                    transpose_b ? "[K][ldb] under TT" : "[batch_sum][ldb] under TN");
    if (ldd < K) return fail(MM_ERR_INVALID_ARGUMENT, "ldd must be >= K (each group's block is [N][ldd])");
    if (stride_d < 0) return fail(MM_ERR_INVALID_ARGUMENT, "stride_d must be >= 0");
    const int64_t P = kgroup_pitch(batch_sum, G);
    if (P > kMaxPitch) return fail(MM_ERR_UNSUPPORTED, "batch_sum + 16 G must stay below 2^22");
    if (!pack_fits(1, batch_sum, N) || !pack_fits(1, batch_sum, K))
        return fail(MM_ERR_UNSUPPORTED, "N and K must be below 2^22");
    if (G > 0 && cdiv(N, 64) * cdiv(K, 64) >= kMaxDim / G) return fail(MM_ERR_UNSUPPORTED, "too many output tiles");
    if (G == 0 || N == 0 || K == 0) return MM_OK;
    if (!batch_sizes || !batch_offsets) return fail(MM_ERR_INVALID_ARGUMENT, "batch_sizes or batch_offsets is NULL");
    if (!aligned(batch_sizes, 4) || !aligned(batch_offsets, 4))
        return fail(MM_ERR_MISALIGNED, "batch_sizes and batch_offsets must be 4-byte aligned");
    if (!d) return fail(MM_ERR_INVALID_ARGUMENT, "d is NULL");
    if (batch_sum > 0 && (!a || !b)) return fail(MM_ERR_INVALID_ARGUMENT, "a or b is NULL");
    if (!scale_a || !scale_b) return fail(MM_ERR_INVALID_ARGUMENT, "scale_a or scale_b is NULL");
    if (!aligned(d, elem_size(d_type))) return fail(MM_ERR_MISALIGNED, "d must be aligned to its element size");
    if (!aligned(scale_a, 4) || !aligned(scale_b, 4) || !aligned(scale_result, 4))
        return fail(MM_ERR_MISALIGNED, "scale pointers must be 4-byte aligned");
    if (forced_launch_failure()) return fail(MM_ERR_DEVICE, "launch failure forced by MM_TEST_FORCE_FAIL");

    const char* who = "mm_scaled_gemm_grouped_layout launch";
    hipStream_t s = static_cast<hipStream_t>(stream);
    const KGroupWs w = kgroup_ws(batch_sum, N, K, G);
    int64_t* start = reinterpret_cast<int64_t*>(ws + w.start);
    uint8_t* at = ws + w.a;
    uint8_t* bt = ws + w.b;
    hipError_t e = mmfp8::launch_group_starts(batch_sizes, (int)G, start, s);
    if (e != hipSuccess) return device_status(e, who);
    if (batch_sum > 0) {
        e = mmfp8::launch_group_pack(true, static_cast<const uint8_t*>(a), batch_sum, N, lda, at, P, batch_sizes,
                                     batch_offsets, start, (int)G, s);
        if (e != hipSuccess) return device_status(e, who);
        e = mmfp8::launch_group_pack(!transpose_b, static_cast<const uint8_t*>(b), batch_sum, K, ldb, bt, P,
                                     batch_sizes, batch_offsets, start, (int)G, s);
        if (e != hipSuccess) return device_status(e, who);
    }
    mmfp8::GemmArgs p{};
    p.a = at;
    p.b = bt;
    p.lda = P;
    p.ldb = P;
    p.M = (int)N;
    p.N = (int)K;
    p.K = 0;  // per group, from batch_sizes
    p.L = (int)G;
    p.sa = scale_a;
    p.sb = scale_b;
    p.scale_result = scale_result;
    p.d = d;
    p.ldd = ldd;
    p.d_batch = stride_d;
    p.d_type = d_type;
    p.vec_store = (ldd % 4 == 0) && (stride_d % 4 == 0) && aligned(d, 4 * elem_size(d_type));
    p.grp_sizes = batch_sizes;
    p.kgrp_start = start;
    const int mode = use_fast_accum ? mmfp8::MODE_FAST : mmfp8::MODE_SLOW;
    int cfg = choose_cfg(N, K, G, cu_count(), mmfp8::min_cfg(mode, 0));
    // slow: the 256x256 row-chunk tiles where they cost less for every block (no split plan here)
    if (mode == mmfp8::MODE_SLOW && cfg == mmfp8::CFG_128x128 && rc_columns(N, K, G, cu_count()) == K)
        cfg = mmfp8::CFG_256x256;
    p.tiles_m = (int)cdiv(N, mmfp8::kCfgBM[cfg]);
    p.tiles_n = (int)cdiv(K, mmfp8::kCfgBN[cfg]);
    const int64_t grid = (int64_t)p.tiles_m * p.tiles_n * G;
    const int fa = a_type == MM_F8_E5M2 ? 1 : 0;
    const int fb = b_type == MM_F8_E5M2 ? 1 : 0;
    e = use_fast_accum ? mmfp8::launch_tile_fast(cfg, fa, fb, p, (int)grid, s)
                       : mmfp8::launch_tile_slow(cfg, fa, fb, p, (int)grid, s);
    return device_status(e, who);
}

}  // extern "C"

// ------------------------------------------------------------------ no-allocation variant
//
// mm_scaled_gemm_grouped_layout_noalloc: the same call with the library's own
// device scratch array in place of the caller's workspace. The array is a
// file-scope __device__ object, so every GPU the library runs on holds one copy
// of it from the code object's load until the process ends, and nothing is
// allocated per call. In host code its name is a host-side stand-in: the
// device address comes from hipGetSymbolAddress, once per device with that
// device current, and only that address reaches kernels.

static __device__ __attribute__((aligned(256))) uint8_t scratch[MM_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[64] = {};

mm_status scratch_address(uint8_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_status(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(MM_ERR_UNSUPPORTED, "device index %d is beyond 63", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return device_status(e, "hipGetSymbolAddress of the scratch array");
        g_scratch_ptr[dev] = static_cast<uint8_t*>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return MM_OK;
}

}  // namespace

extern "C" {

mm_status mm_scaled_gemm_grouped_layout_noalloc(int64_t batch_sum, int64_t N, int64_t K, int64_t G, int transpose_a,
                                                int transpose_b, const void* a, int a_type, int64_t lda,
                                                const void* b, int b_type, int64_t ldb, int64_t stride_b,
                                                const int32_t* batch_sizes, const int32_t* batch_offsets,
                                                const float* scale_a, const float* scale_b,
                                                const float* scale_result, void* d, int d_type, int64_t ldd,
                                                int64_t stride_d, int use_fast_accum, void* stream) {
    g_error.clear();
    if ((transpose_a != 0 && transpose_a != 1) || (transpose_b != 0 && transpose_b != 1))
        return fail(MM_ERR_INVALID_ARGUMENT, "transpose_a and transpose_b must be 0 or 1");
    uint64_t need = 0;
    if (const mm_status st = mm_grouped_workspace_bytes(batch_sum, N, K, G, transpose_a, transpose_b, &need))
        return st;
    if (need > (uint64_t)MM_NOALLOC_SCRATCH_BYTES)
        return fail(MM_ERR_UNSUPPORTED,
                    "this layout and size need %llu bytes of workspace, more than the library's %llu-byte scratch "
                    "array; use mm_scaled_gemm_grouped_layout with a workspace",
                    (unsigned long long)need, (unsigned long long)MM_NOALLOC_SCRATCH_BYTES);
    uint8_t* ws = nullptr;
    if (need > 0) {
        if (const mm_status st = scratch_address(&ws)) return st;
    }
    return mm_scaled_gemm_grouped_layout(batch_sum, N, K, G, transpose_a, transpose_b, a, a_type, lda, b, b_type, ldb,
                                         stride_b, batch_sizes, batch_offsets, scale_a, scale_b, scale_result, d,
                                         d_type, ldd, stride_d, ws, need > 0 ? (uint64_t)MM_NOALLOC_SCRATCH_BYTES : 0,
                                         use_fast_accum, stream);
}

}  // extern "C"
