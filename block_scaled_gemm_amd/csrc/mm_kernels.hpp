// mm_kernels.hpp -- gfx950 kernels of libmmfp8: FP8 scaled GEMM (per-tensor,
// 1x128 / 128x128 block scales, 32-element MX scale factors), fused epilogue
// cast and amax.
//
// The computation is the FP8 NT GEMM d = (a * s_a) @ (b * s_b)^T of "TileOPs:
// Linear Algebra Operators" (tileops.gemm.GemmFP8FwdOp), with the fast / slow
// accumulation and scale_result of "mmaemu API reference (v0.1)"
// (mmaemu.scaled_mm) and the batched block-scaled GEMM + amax of "cuDNN
// frontend: GEMM + Amax (SM100)" (Equations).
//
// Hardware facts this file relies on (measured on MI355X with in-bounds
// probes; tests/mfma_precision.py reproduces the first):
//  * The FP8 MFMAs of gfx950 (v_mfma_scale_f32_16x16x128_f8f6f4 and the older
//    fp8 ones) do not sum their products exactly: small products that share an
//    adder group with large ones lose low bits, up to ~2^-16.5 * sum|t| per
//    128 products on Gaussian data, which is outside the 2^-20 * sum|t| bound
//    this library guarantees. v_mfma_f32_16x16x32_bf16 forms exact products and
//    accumulates to ~2^-26 * sum|t|. Every FP8 value (E4M3 and E5M2) is exactly
//    a bf16 value, so the kernels convert FP8 to bf16 in registers
//    (v_cvt_scalef32_pk_bf16_fp8 / _bf8, with a power-of-two scale that is
//    exact) and contract with the bf16 MFMA. On FP4 (E2M1) operands the scaled
//    MFMA stays within 2^-22 * sum|t| (E8M0 factors 2^-8 .. 2^4, also 2^24
//    apart in one instruction), so FP4 with E8M0 factors per 32 runs on it.
//  * Issue: every VALU instruction, the MFMA included, holds the SIMD's VALU
//    issue for 4 cycles and a 16x16x32 bf16 MFMA runs 16; independent VALU
//    work issued between a wave's MFMAs overlaps them (2 conversions and 1 add
//    per MFMA: 22.5 cycles per MFMA at two waves per SIMD, 27 at one).
//  * 16x16 MFMA results: D[i][j] (i from the first operand, j from the
//    second) is in lane j + 16 (i / 4), register i % 4. Both operands use the
//    same lane layout, so any assignment of k to (lane group, element) that is
//    the same for A and B gives the same sum.
//  * The MFMA adds C to the product sum with one round-to-nearest-even; fp32
//    subnormal results are kept.
//  * Buffer loads check the range per dword: a dword past num_records reads 0.
//  * buffer_load ... lds writes lane l's 16 bytes to LDS base + 16 l.
//  * v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 round to nearest even but do not
//    saturate; v_cvt_pk_bf16_f32 and v_cvt_f16_f32 are IEEE RNE. NaN payloads
//    are not canonical, so the epilogue rewrites NaN itself.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmfp8 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

// Element types (the values of mm_dtype). T_E2M1: FP4, two per byte.
enum : int { T_E4M3 = 0, T_E5M2 = 1, T_F32 = 2, T_BF16 = 3, T_F16 = 4, T_E2M1 = 5 };
// Accumulation / scaling modes of the main loop.
enum : int { MODE_FAST = 0, MODE_SLOW = 1, MODE_BLOCK = 2, MODE_SF32 = 3 };
// Granularity of scale_b in MODE_BLOCK.
enum : int { SB_1x128 = 0, SB_128x128 = 1 };
// Scale-factor storage in MODE_SF32 (the same template slot): fp32 factors
// [L][MN][groups] of 32 K, or the cuDNN page's native layout of E8M0 bytes
// with groups of 32 or 16 K, where for every 128 rows and 4 groups the 512
// bytes hold row r's 4 groups as one dword at byte 16 (r % 32) + 4 (r / 32),
// blocks ordered [L][MN/128][ceil(groups/4)].
// SF_ATOM_E4M3_16: the same layout holding E4M3 factors, one per 16 values
// (FP4 operands only).
enum : int { SF_F32 = 0, SF_ATOM_E8M0 = 1, SF_ATOM_E8M0_16 = 2, SF_ATOM_E4M3_16 = 3 };

constexpr int kBK = 128;                 // K per main-loop step = one MFMA = one 128-element chunk
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9 buffer descriptor dword 3 (raw, 32-bit format)
constexpr uint32_t kOOB = 0x80000000u;   // a voffset beyond any extent: loads return 0

struct GemmArgs {
    const uint8_t* a;   // [L][M] rows of lda bytes
    const uint8_t* b;   // [L][N] rows of ldb bytes
    int64_t lda, ldb;   // bytes
    int64_t a_batch, b_batch;  // bytes between batch items
    int M, N, K, L;
    const float* sa;    // TENSOR: [1]; BLOCK: [M][sa_ld]; SF32: [L][M][sa_ld]; atom: E8M0 bytes
    const float* sb;    // TENSOR: [1]; BLOCK: [N or ceil(N/128)][sb_ld]; SF32: [L][N][sb_ld]; atom: E8M0 bytes
    int64_t sa_ld, sb_ld;         // SF32 (both layouts): ceil(K/32) groups
    int64_t sa_batch, sb_batch;   // 4-byte elements between batch items (SF32, both layouts)
    const float* scale_result;    // FP8 outputs only; may be null
    void* d;            // [L][M] rows of ldd elements
    int64_t ldd, d_batch;         // elements
    int d_type;
    int vec_store;      // 4-element vector stores are aligned
    uint32_t* amax_bits;          // amax without index (atomic max of |x| bits) or null
    unsigned long long* amax_key; // (|x| bits << 33) | (2^33 - 1 - index), or null
    int tiles_m, tiles_n;
    const void* bias;   // [N] of d_type (f32, bf16 or f16), added after the scales; or null
    // Grouped GEMM (groups > 0): a and d hold the groups' rows packed along M
    // (M = the packed row count), b one [N][ldb] operand per group, b_batch
    // bytes apart; grid tile row t is tile t - (tiles of the groups before) of
    // its group. grp_sizes / grp_offsets: rows and first row of each group.
    const int* grp_sizes;
    const int* grp_offsets;
    int groups;
    // Groups that split the contraction (kgrp_start non-null, tile kernel):
    // batch item l is group l, whose operands are columns kgrp_start[l] ..
    // + grp_sizes[l] - 1 of a and b (both [rows][lda] with lda == ldb), so its
    // K is grp_sizes[l] (0 gives a zero block).
    const int64_t* kgrp_start;
};

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, (int)kRsrcWord3);
}

// Extent in bytes of `rows` rows of pitch ld of which the last has K valid
// bytes, rounded up to a dword: the per-dword range check then never drops a
// valid byte, and bytes past it read as zero.
__device__ __forceinline__ uint32_t operand_extent(int rows, int64_t ld, int K) {
    if (rows <= 0) return 0;
    const int64_t e = (int64_t)(rows - 1) * ld + K;
    return (uint32_t)((e + 3) & ~(int64_t)3);
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& first, const bf16x8& second, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(first, second, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(const f16x8& first, const f16x8& second, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(first, second, c, 0, 0, 0);
}

// Two FP8 codes (bytes 2 hi, 2 hi + 1 of w) to two bf16 values times `scale`.
// F = 0: E4M3, F = 1: E5M2. Exact: every FP8 value is a bf16 value and the
// scales used here are powers of two.
template <int F, bool HI>
__device__ __forceinline__ bf16x2 cvt2(uint32_t w, float scale) {
    if constexpr (F == 0) return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI);
    else return __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, scale, HI);
}

// Dword q (q = 0..3) of a 16-byte FP4 chunk, i.e. 8 E2M1 values, as one bf16
// MFMA operand times `scale`: each byte's two values, low nibble first. Exact:
// every E2M1 value times a power of two in range is a bf16 value.
__device__ __forceinline__ bf16x8 fp4_to_bf16x8(const i32x4& f, int q, float scale) {
    const uint32_t w = (uint32_t)f[q];
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
    const auto lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
    const auto hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Bytes 8 s .. 8 s + 7 of a lane's 32-byte FP8 fragment as one bf16 MFMA operand.
template <int F>
__device__ __forceinline__ bf16x8 to_bf16x8(const i32x8& f, int s, float scale) {
    const uint32_t w0 = (uint32_t)f[2 * s], w1 = (uint32_t)f[2 * s + 1];
    const bf16x2 p0 = cvt2<F, false>(w0, scale), p1 = cvt2<F, true>(w0, scale);
    const bf16x2 p2 = cvt2<F, false>(w1, scale), p3 = cvt2<F, true>(w1, scale);
    const auto lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
    const auto hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Bytes 8 q .. 8 q + 7 (q = 0, 1) of a 16-byte FP8 chunk as one bf16 MFMA operand.
template <int F>
__device__ __forceinline__ bf16x8 to_bf16x8(const i32x4& f, int q, float scale) {
    const uint32_t w0 = (uint32_t)f[2 * q], w1 = (uint32_t)f[2 * q + 1];
    const bf16x2 p0 = cvt2<F, false>(w0, scale), p1 = cvt2<F, true>(w0, scale);
    const bf16x2 p2 = cvt2<F, false>(w1, scale), p3 = cvt2<F, true>(w1, scale);
    const auto lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
    const auto hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Dword q of a 16-byte FP4 chunk as one f16 MFMA operand, each value times the
// E4M3 factor s (a packed f16 multiply). Exact: an E2M1 value times an E4M3
// value has at most 6 significant bits and lies in [2^-10, 2688], inside f16's
// normal range. (The scaled conversions take only a power of two.)
__device__ __forceinline__ f16x8 fp4_to_f16x8(const i32x4& f, int q, _Float16 s) {
    const uint32_t w = (uint32_t)f[q];
    const f16x2 ss = {s, s};
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
    const auto lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
    const auto hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ i32x8 cat(i32x4 lo, i32x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Scale operands of the scaled conversions. The gfx950 conversions
// (v_cvt_scalef32_pk_bf16_fp8 / _bf8 / _fp4) read only the exponent field of
// their fp32 scale, as an E8M0 code: field e multiplies by 2^(e - 127), field 0
// by 2^-127, field 255 gives NaN; sign and mantissa are ignored (measured on
// MI355X for every field class, FP8, BF8 and FP4 sources). So an E8M0 code is
// passed as the float whose exponent field it is, and an fp32 factor is passed
// as it is.
__device__ __forceinline__ float e8m0_code_scale(uint32_t e) { return __uint_as_float(e << 23); }
__device__ __forceinline__ float e8m0_scale(float s) { return s; }

// ------------------------------------------------------------------ output conversions

__device__ __forceinline__ uint32_t cvt_f32(float v) {
    return __builtin_isnan(v) ? 0x7FFFFFFFu : __float_as_uint(v);
}
__device__ __forceinline__ uint32_t cvt_bf16(float v) {
    __bf16 h = (__bf16)v;  // v_cvt_pk_bf16_f32: RNE, overflow to Inf
    return __builtin_isnan(v) ? 0x7FFFu : (uint32_t)__builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t cvt_f16(float v) {
    _Float16 h = (_Float16)v;  // v_cvt_f16_f32: RNE, overflow to Inf
    return __builtin_isnan(v) ? 0x7FFFu : (uint32_t)__builtin_bit_cast(uint16_t, h);
}
// FP8 outputs saturate: clamp to +-max first (the converter itself would give
// NaN / Inf), then round; NaN becomes the canonical 0x7F.
__device__ __forceinline__ uint32_t cvt_e4m3(float v) {
    const float c = __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
    const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
    return __builtin_isnan(v) ? 0x7Fu : code;
}
__device__ __forceinline__ uint32_t cvt_e5m2(float v) {
    const float c = __builtin_fminf(__builtin_fmaxf(v, -57344.0f), 57344.0f);
    const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, c, 0, false) & 0xFFu;
    return __builtin_isnan(v) ? 0x7Fu : code;
}

// E2M1 (FP4) outputs: round to nearest even over 0, 0.5, 1, 1.5, 2, 3, 4, 6
// and saturate; each midpoint (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) goes to the
// neighbour with the even code, so the count of thresholds passed is the code.
// E2M1 has no NaN: NaN gives the largest value's code 0x7.
__device__ __forceinline__ uint32_t cvt_e2m1(float v) {
    const float a = __builtin_fabsf(v);
    const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
    return __builtin_isnan(v) ? 0x7u : (c | ((__float_as_uint(v) >> 28) & 8u));
}

template <int T>
__device__ __forceinline__ uint32_t convert_t(float v) {
    if constexpr (T == T_F32) return cvt_f32(v);
    else if constexpr (T == T_BF16) return cvt_bf16(v);
    else if constexpr (T == T_F16) return cvt_f16(v);
    else if constexpr (T == T_E4M3) return cvt_e4m3(v);
    else if constexpr (T == T_E2M1) return cvt_e2m1(v);
    else return cvt_e5m2(v);
}
__device__ __forceinline__ uint32_t convert(float v, int t) {
    switch (t) {
        case T_F32: return convert_t<T_F32>(v);
        case T_BF16: return convert_t<T_BF16>(v);
        case T_F16: return convert_t<T_F16>(v);
        case T_E4M3: return convert_t<T_E4M3>(v);
        default: return convert_t<T_E5M2>(v);
    }
}

// Element n of a bias vector of output type T, as fp32 (exact).
template <int T>
__device__ __forceinline__ float load_bias(const void* bias, int n) {
    if constexpr (T == T_F32) return ((const float*)bias)[n];
    else if constexpr (T == T_BF16) return __uint_as_float((uint32_t)((const uint16_t*)bias)[n] << 16);
    else return (float)((const _Float16*)bias)[n];
}

// A compile-time int, to hand a runtime choice to a generic lambda.
template <int V>
struct IC {
    static constexpr int value = V;
};
// Call f(IC<t>{}) for the output type t, so that the epilogue is compiled once
// per type instead of branching on the type at every element.
template <class F>
__device__ __forceinline__ void with_out_type(int t, F&& f) {
    switch (t) {
        case T_F32: f(IC<T_F32>{}); break;
        case T_BF16: f(IC<T_BF16>{}); break;
        case T_F16: f(IC<T_F16>{}); break;
        case T_E4M3: f(IC<T_E4M3>{}); break;
        default: f(IC<T_E5M2>{}); break;
    }
}

__device__ __forceinline__ int elem_bytes(int t) { return t == T_F32 ? 4 : (t == T_E4M3 || t == T_E5M2) ? 1 : 2; }

// Store 4 consecutive converted outputs starting at element e (row-major
// index); `valid` of them (0..4) exist. Vector store when aligned and whole.
template <int T>
__device__ __forceinline__ void store4(void* d, int64_t e, const uint32_t v[4], int valid, bool vec) {
    if constexpr (T == T_F32) {
        uint32_t* p = (uint32_t*)d + e;
        if (vec && valid == 4) { *(i32x4*)p = i32x4{(int)v[0], (int)v[1], (int)v[2], (int)v[3]}; return; }
        for (int r = 0; r < valid; ++r) p[r] = v[r];
    } else if constexpr (T == T_BF16 || T == T_F16) {
        uint16_t* p = (uint16_t*)d + e;
        if (vec && valid == 4) {
            *(i32x2*)p = i32x2{(int)(v[0] | (v[1] << 16)), (int)(v[2] | (v[3] << 16))};
            return;
        }
        for (int r = 0; r < valid; ++r) p[r] = (uint16_t)v[r];
    } else if constexpr (T == T_E2M1) {
        // packed two per byte, low nibble first; e (in elements) is even: rows
        // of an even number of elements, 4 consecutive ones per lane. A lone
        // last element leaves its byte's high nibble 0.
        uint8_t* p = (uint8_t*)d + (e >> 1);
        const uint32_t lo = v[0] | ((valid > 1 ? v[1] : 0u) << 4);
        const uint32_t hi = (valid > 2 ? v[2] : 0u) | ((valid > 3 ? v[3] : 0u) << 4);
        if (vec && valid == 4) { *(uint16_t*)p = (uint16_t)(lo | (hi << 8)); return; }
        if (valid > 0) p[0] = (uint8_t)lo;
        if (valid > 2) p[1] = (uint8_t)hi;
    } else {
        uint8_t* p = (uint8_t*)d + e;
        if (vec && valid == 4) { *(uint32_t*)p = v[0] | (v[1] << 8) | (v[2] << 16) | (v[3] << 24); return; }
        for (int r = 0; r < valid; ++r) p[r] = (uint8_t)v[r];
    }
}

// Amax keys. |x| as fp32 bits orders like |x|; canonical NaN (0x7FFFFFFF)
// beats +Inf. With an index the key also prefers the smallest index on ties.
__device__ __forceinline__ uint32_t abs_bits(float v) {
    return __builtin_isnan(v) ? 0x7FFFFFFFu : (__float_as_uint(v) & 0x7FFFFFFFu);
}
__device__ __forceinline__ unsigned long long amax_key(float v, int64_t idx) {
    return ((unsigned long long)abs_bits(v) << 33) | ((1ull << 33) - 1ull - (unsigned long long)idx);
}

template <class T>
__device__ __forceinline__ T wave_max(T x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const T y = __shfl_xor(x, off, 64);
        x = y > x ? y : x;
    }
    return x;
}

// Block-wide max of per-thread keys, then one atomic per workgroup.
template <int NT>
__device__ __forceinline__ void amax_commit(const GemmArgs& p, uint32_t kb, unsigned long long kk) {
    __shared__ unsigned long long red[NT / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (p.amax_key) {
        kk = wave_max(kk);
        if (lane == 0) red[wave] = kk;
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned long long m = red[0];
            for (int w = 1; w < NT / 64; ++w) m = red[w] > m ? red[w] : m;
            if (m) atomicMax(p.amax_key, m);
        }
    } else if (p.amax_bits) {
        kb = wave_max(kb);
        if (lane == 0) red[wave] = kb;
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned long long m = red[0];
            for (int w = 1; w < NT / 64; ++w) m = red[w] > m ? red[w] : m;
            atomicMax(p.amax_bits, (uint32_t)m);
        }
    }
}

// Map the linear workgroup id to a tile. Workgroups are dispatched round-robin
// over the 8 XCDs (each with its own L2); this gives every XCD a contiguous run
// of tiles, walked in groups of `group_m` tile rows so that the tiles live on
// one XCD at the same time share A rows and B columns. With l_fastest = L
// the batch index varies fastest along the run instead, so that every XCD
// gets an equal share of every item (items of unequal work: groups that split
// the contraction).
__device__ __forceinline__ void tile_of(int bid, int nblocks, int tiles_m, int tiles_n, int group_m, int& l,
                                        int& tm, int& tn, int l_fastest = 0) {
    const int per = nblocks / 8, rem = nblocks % 8;
    const int x = bid % 8, i = bid / 8;
    const int t = (x < rem) ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
    const int tiles = tiles_m * tiles_n;
    int u;
    if (l_fastest > 0) {
        l = t % l_fastest;
        u = t / l_fastest;
    } else {
        l = t / tiles;
        u = t - l * tiles;
    }
    const int width = group_m * tiles_n;
    const int grp = u / width;
    const int first = grp * group_m;
    const int gsz = min(tiles_m - first, group_m);
    const int v = u - grp * width;
    tm = first + v % gsz;
    tn = v / gsz;
}

// Grouped GEMM: grid tile row tm -> its group g (groups take ceil(rows / BM)
// tile rows each, in order) and the tile row within it. Moves a and d to the
// tile's first packed row and b to the group's operand, sets M to the tile's
// valid rows and tm to 0. Rows are clamped to the packed buffer, so group
// sizes and offsets that do not add up never read or write outside it. Every
// wave computes this (a wave-wide prefix over 64 groups at a time); false
// when the tile has no rows.
template <int BM>
__device__ __forceinline__ bool group_tile(GemmArgs& p, int& tm) {
    const int lane = threadIdx.x & 63;
    int64_t before = 0;  // tile rows of the groups before the current 64
    for (int g0 = 0; g0 < p.groups; g0 += 64) {
        const int g = g0 + lane;
        const int64_t rows = g < p.groups ? min(max((int64_t)p.grp_sizes[g], (int64_t)0), (int64_t)p.M) : 0;
        const int64_t own = (rows + BM - 1) / BM;
        int64_t incl = own;  // inclusive prefix of the tile rows over the wave
        for (int d = 1; d < 64; d <<= 1) {
            const int64_t v = __shfl_up(incl, d);
            if (lane >= d) incl += v;
        }
        const unsigned long long hit = __ballot(before + incl > tm);
        if (hit) {
            const int gl = __ffsll((long long)hit) - 1;
            const int gsel = __builtin_amdgcn_readfirstlane(g0 + gl);
            const int t = __builtin_amdgcn_readfirstlane((int)(tm - before - __shfl(incl - own, gl)));  // within the group
            const int64_t row0 = (int64_t)p.grp_offsets[gsel] + (int64_t)t * BM;
            const int64_t valid = min(min((int64_t)BM, (int64_t)p.grp_sizes[gsel] - (int64_t)t * BM), (int64_t)p.M - row0);
            if (row0 < 0 || valid <= 0) return false;
            const int es = p.d_type == T_F32 ? 4 : ((p.d_type == T_BF16 || p.d_type == T_F16) ? 2 : 1);
            p.a += row0 * p.lda;
            p.d = (uint8_t*)p.d + row0 * p.ldd * es;
            p.b += (int64_t)gsel * p.b_batch;
            p.M = (int)valid;
            tm = 0;
            return true;
        }
        before += __shfl(incl, 63);
    }
    return false;
}

// Scheduling pattern of one row of MFMAs: NMF times (one MFMA, then an even
// share of VALU VGPR instructions, then one LDS read while READS last).
template <int VALU, int READS, int NMF, int M = 0>
__device__ __forceinline__ void sched_row() {
    if constexpr (M < NMF) {
        constexpr int v = VALU / NMF + (M < VALU % NMF ? 1 : 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x002, v, 0);
        if constexpr (M < READS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        sched_row<VALU, READS, NMF, M + 1>();
    }
}

// One 128-K step of a wave's 16 NF x 16 NF tile whose fragments lie in LDS
// (A rows at As, B rows at Bs, 128-byte rows with the XOR swizzle; lane (r, g)
// reads its row's chunk 2 g + h at fo_h). The step is four sub-steps of K = 32
// (u = 2 h + q), each a row-by-row pass over the fragments (row j: the MFMAs of
// B fragment j with every A fragment). Next to row j's MFMAs of sub-step u go
// the conversions of B and A fragment j for sub-step u + 1 and, in sub-step 0,
// the reads of the second half's fragment j (into the registers the first
// half's fragment j just left), so that one wave keeps the matrix core and the
// vector ALU busy at once. CHAIN: the MFMAs accumulate into acc. Otherwise each
// step's 128-chunk sums into a fresh fp32 partial that is then added to acc
// (slow accumulation), row j's addition going between row j + 1's MFMAs of the
// last sub-step; with SCALED the partial is folded in as acc = fma(part,
// s_a * s_b, acc) (block scaling: s_a of A fragment i's row, read from LDS at
// sa_col[16 i] just before the last sub-step, and the step's one s_b). c_a /
// c_b scale the conversions of A / B fragment j.
template <int FA, int FB, int NF, bool CHAIN, bool SCALED = false>
__device__ __forceinline__ void ilv_step(const uint8_t* As, const uint8_t* Bs, int fo0, int fo1, const float* c_a,
                                         const float* c_b, f32x4 (&acc)[NF][NF], f32x4 (&part)[NF][NF],
                                         const float* sa_col = nullptr, float sb = 1.0f) {
    float sab[NF];
    auto row = [&](int j, const bf16x8 (&xa)[NF], const bf16x8& xbj) {
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            if constexpr (CHAIN) acc[j][i] = mfma_bf16(xbj, xa[i], acc[j][i]);
            else part[j][i] = mfma_bf16(xbj, xa[i], part[j][i]);
        }
    };
    auto promote_row = [&](int j) {
        if constexpr (!CHAIN) {
#pragma unroll
            for (int i = 0; i < NF; ++i) {
                if constexpr (SCALED) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[j][i][r] = __builtin_fmaf(part[j][i][r], sab[i], acc[j][i][r]);
                } else {
                    acc[j][i] += part[j][i];
                }
            }
        }
    };
    if constexpr (!CHAIN) {
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
            for (int i = 0; i < NF; ++i) part[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    i32x4 ra[NF], rb[NF];  // raw fragments: the first half, then the second
#pragma unroll
    for (int j = 0; j < NF; ++j) {
        ra[j] = *(const i32x4*)(As + j * 16 * kBK + fo0);
        rb[j] = *(const i32x4*)(Bs + j * 16 * kBK + fo0);
    }
    bf16x8 xa0[NF], xa1[NF], xb[NF];
#pragma unroll
    for (int j = 0; j < NF; ++j) {
        xa0[j] = to_bf16x8<FA>(ra[j], 0, c_a[j]);
        xb[j] = to_bf16x8<FB>(rb[j], 0, c_b[j]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 0: MFMAs of (xa0, xb); sub-step 1's operands from the first half; second-half reads
#pragma unroll
    for (int j = 0; j < NF; ++j) {
        row(j, xa0, xb[j]);
        xb[j] = to_bf16x8<FB>(rb[j], 1, c_b[j]);
        xa1[j] = to_bf16x8<FA>(ra[j], 1, c_a[j]);
        ra[j] = *(const i32x4*)(As + j * 16 * kBK + fo1);
        rb[j] = *(const i32x4*)(Bs + j * 16 * kBK + fo1);
        sched_row<8, 2, NF>();
        __builtin_amdgcn_sched_barrier(0);
    }
    // sub-step 1: MFMAs of (xa1, xb); sub-step 2's operands from the second half
#pragma unroll
    for (int j = 0; j < NF; ++j) {
        row(j, xa1, xb[j]);
        xb[j] = to_bf16x8<FB>(rb[j], 0, c_b[j]);
        xa0[j] = to_bf16x8<FA>(ra[j], 0, c_a[j]);
        sched_row<8, 0, NF>();
        __builtin_amdgcn_sched_barrier(0);
    }
    // sub-step 2: MFMAs of (xa0, xb); sub-step 3's operands
#pragma unroll
    for (int j = 0; j < NF; ++j) {
        row(j, xa0, xb[j]);
        xb[j] = to_bf16x8<FB>(rb[j], 1, c_b[j]);
        xa1[j] = to_bf16x8<FA>(ra[j], 1, c_a[j]);
        sched_row<8, 0, NF>();
        __builtin_amdgcn_sched_barrier(0);
    }
    // sub-step 3: MFMAs of (xa1, xb), each row with the promotion of the row before
    if constexpr (SCALED) {
#pragma unroll
        for (int i = 0; i < NF; ++i) sab[i] = sa_col[16 * i] * sb;
    }
#pragma unroll
    for (int j = 0; j < NF; ++j) {
        row(j, xa1, xb[j]);
        if (j > 0) promote_row(j - 1);
        if constexpr (!CHAIN) {
            if (j > 0) sched_row<4 * NF, 0, NF>();
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    promote_row(NF - 1);
}

// ------------------------------------------------------------------ tiled kernel
//
// Workgroup tile BM x BN computed by WM x WN waves, each wave a
// (BM/WM) x (BN/WN) block of 16 x 16 MFMA tiles. The MFMA's first operand is b
// (rows n) and its second is a (rows m), so every lane's results share one m
// and hold 4 consecutive n: one scale_a value per lane, vector stores along N.
//
// K is walked in steps of 128 (= one "slow" chunk = one 1x128 scale block =
// four 32-element MX groups). Each step's A and B tiles go from memory straight
// to LDS with buffer_load ... lds through two alternating buffers; rows are 128
// bytes with the 16-byte chunk c of row r stored at chunk c ^ swz(r),
// swz(r) = (r & 7) ^ ((r >> 3) & 1): any 8 consecutive rows, and any 16
// consecutive rows split by row parity, then hit distinct banks at one
// logical chunk, so the fragment reads are free of bank conflicts. Lane (r, g) of a fragment holds
// k = 32g .. 32g+31 of row r (one MX group), converted to bf16 8 values at a
// time for the four v_mfma_f32_16x16x32_bf16 of the step.
//
// The main loop is one of four. FP8 operands on 64x128 wave tiles (the 256x256
// tile: slow, fast, MX with fp32 factors, block scaling with a 128x128
// scale_b) run the row-chunk loop (kRc), which converts the step's A fragments
// once and walks the B fragment rows, so that the promoted modes keep only one
// row's 128-chunk partials live. FP8 operands on square wave tiles (every
// per-tensor and MX 128x128 / 64x64 tile, and block scaling with a 128x128
// scale_b) run ilv_step, which interleaves the next K = 32 sub-step's
// conversions and the second half's fragment reads with the current MFMAs.
// Otherwise PIPE runs the fragment reads a half-step ahead of the MFMAs (the
// way to hide LDS latency with one wave per SIMD, at the cost of a second set
// of fragment registers), and the plain loop reads each half-step's fragments
// and then multiplies, a second wave on the SIMD hiding the latency.
//
// KG = 2 splits the K steps of a tile between two groups of WM x WN waves (even
// steps to group 0, odd steps to group 1), each with its own pair of stages;
// at the end the groups add their partial tiles, group 0's first, and each
// group stores half of the rows. It gives a tile two waves per SIMD when the
// tiles are too few for two workgroups per CU.
template <int BM, int BN, int WM, int WN, int PIPE, int MODE, int FA, int FB, int SBM, int KG = 1>
__global__ void __launch_bounds__(WM * WN * KG * 64, (WM * WN * KG == 4 && !PIPE) ? 2 : 1) gemm_tile(GemmArgs p) {
    static_assert(KG == 1 || (KG == 2 && !PIPE), "K groups use the plain main loop");
    constexpr int NW = WM * WN;       // waves per K group
    constexpr int NT = NW * KG * 64;  // threads of the workgroup
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    // FP8 operands on 64x128 wave tiles run the row-chunk main loop below: slow accumulation, block scaling
    // with a 128x128 scale_b (one s_b per wave and step), and the chained modes (fast, and MX with fp32
    // factors; with the page-native factor bytes it spilled 32 VGPRs). A ragged K's last step is loaded like
    // the others (every offset is per lane there, so the range check covers it) and the chunks at or past K
    // are zeroed in LDS: the tail load path would not fit its registers.
    constexpr bool kRc = (MODE == MODE_SLOW || MODE == MODE_FAST || (MODE == MODE_SF32 && SBM == SF_F32) ||
                          (MODE == MODE_BLOCK && SBM == SB_128x128 && 128 % WTN == 0)) &&
                         !PIPE && KG == 1 && FA != T_E2M1 && FM == 4 && FN == 8;
    constexpr int A_INS = BM / 8 / NW, B_INS = BN / 8 / NW;  // 1 KB LDS-DMA writes per wave per step
    constexpr int INS = A_INS + B_INS;
    static_assert(A_INS * 8 * NW == BM && B_INS * 8 * NW == BN, "tile rows must split evenly over the waves");
    // Per-row scales travel with the tiles, into the end of each stage: MX, the
    // step's four 32-groups of every A and B row; block-scaled, the step's
    // scale_a of every A row (and scale_b of every B row when it is 1x128; a
    // 128x128 scale_b is one value per 128 columns, read from memory directly).
    // One 4-byte-per-lane load fills one scale column of 64 rows.
    // FP4 operands (MX only): a step's 128 bytes of a row hold 256 values;
    // each 16-byte fragment chunk feeds four MFMA k-slices instead of two.
    constexpr bool kFp4 = FA == T_E2M1;
    static_assert(FA == FB || !kFp4, "FP4 operands come in pairs");
    static_assert(!kFp4 || (MODE == MODE_SF32 && SBM != SF_F32 && !PIPE), "FP4: page-native factors, plain loop");
    constexpr int NQ = kFp4 ? 4 : 2;
    // The page-native E8M0 layout keeps a row's 4 groups in one dword per 4
    // groups: NKB dwords per row and step (1 for FP8, 2 / 4 for FP4 with 32 /
    // 16 values per group), one gathering load per 64 rows and dword, into
    // LDS [dword][row].
    // The FP8 256x256 tile issues each of these loads four times (the same
    // bytes into the same LDS slots, as many loads as the fp32 factors take):
    // its main loop then fits in 256 VGPRs, where with one issue the compiler
    // spills 38 of them, which measured 17% slower.
    constexpr bool kAtom = MODE == MODE_SF32 && SBM != SF_F32;
    constexpr bool kE4M3 = kAtom && SBM == SF_ATOM_E4M3_16;  // E4M3 factors (FP4 only): f16 operands
    // FP4 with E8M0 factors per 32 values: the scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4) takes the
    // E2M1 codes and the factors as they are; it sums E2M1 products exactly enough (measured against the
    // exact sums: at most 2^-22.6 sum|t| for factors 2^-8 .. 2^4 at K = 8192, with factors 2^24 apart inside
    // one instruction as well), where on FP8 data it does not.
    constexpr bool kFp4Mfma = kFp4 && SBM == SF_ATOM_E8M0;
    static_assert(!kE4M3 || kFp4, "E4M3 factors go with FP4 operands");
    constexpr int SFV = (SBM == SF_ATOM_E8M0_16 || SBM == SF_ATOM_E4M3_16) ? 16 : 32;  // values per scale group
    constexpr int GPS = (kFp4 ? 2 * kBK : kBK) / SFV;      // scale groups per step
    constexpr int NKB = kAtom ? GPS / 4 : 1;
    constexpr int kAtomRep = kAtom && !kFp4 && BM == 256 && BN == 256 ? 4 : 1;
    constexpr int SA_W = MODE == MODE_SF32 ? (kAtom ? kAtomRep * NKB : 4) : (MODE == MODE_BLOCK ? 1 : 0);
    constexpr int SB_W = MODE == MODE_SF32 ? (kAtom ? kAtomRep * NKB : 4)
                                           : ((MODE == MODE_BLOCK && SBM == SB_1x128) ? 1 : 0);
    constexpr int SC_A_INS = BM / 64 * SA_W, SC_INS = SC_A_INS + BN / 64 * SB_W;
    static_assert(BM % 64 == 0 && BN % 64 == 0, "scale columns are loaded 64 rows at a time");
    constexpr int STAGE = (BM + BN) * kBK + SC_INS * 256;
    // Distinct LDS objects (not one array indexed by stage) so that the compiler
    // can tell a fragment read of one stage from the in-flight LDS-DMA writes
    // into another and does not wait for those loads.
    __shared__ __attribute__((aligned(1024))) uint8_t smem0[KG * STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t smem1[KG * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps the LDS addressing scalar
    const int kg = KG > 1 ? wave / NW : 0;                       // K group
    const int gw = KG > 1 ? wave % NW : wave;                    // wave within its group
    const int wm = gw / WN, wn = gw % WN;
    int l, tm, tn;
    tile_of(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, 8, l, tm, tn, p.kgrp_start ? p.L : 0);
    if (p.groups > 0) {
        if (!group_tile<BM>(p, tm)) return;  // the whole workgroup leaves: a tile past the groups' rows
        l = 0;
    }
    if (p.kgrp_start) {
        // clamped so that a slice never leaves the rows, whatever the metadata
        const int64_t c0 = min(max(p.kgrp_start[l], (int64_t)0), p.lda);
        const int64_t kk = min(max((int64_t)p.grp_sizes[l], (int64_t)0), p.lda - c0);
        p.a += c0;
        p.b += c0;
        p.K = __builtin_amdgcn_readfirstlane((int)kk);
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = p.K;
    const int KT = (K + kBK - 1) / kBK;

    const uint8_t* abase = p.a + (int64_t)l * p.a_batch + (int64_t)m0 * p.lda;
    const uint8_t* bbase = p.b + (int64_t)l * p.b_batch + (int64_t)n0 * p.ldb;
    const rsrc_t ra = make_rsrc(abase, operand_extent(min(BM, p.M - m0), p.lda, K));
    const rsrc_t rb = make_rsrc(bbase, operand_extent(min(BN, p.N - n0), p.ldb, K));

    // Loader: wave-instruction q of a tile writes LDS bytes [1024 q, 1024 q + 1024),
    // i.e. rows 8q .. 8q+7; lane l fills row 8q + l/8, stored chunk l%8, which
    // holds logical chunk (l%8) ^ (row & 7) = (l%8) ^ (l/8).
    // The row of wave-instruction q is 8 q + ld_row, so swz(row) = ld_row ^ (q & 1).
    const int ld_row = lane >> 3;
    auto ld_chunk = [&](int ins) { return (lane & 7) ^ ld_row ^ (ins & 1); };
    const bool k_tail = !kRc && (K % kBK) != 0;
    uint32_t aoff[A_INS], boff[B_INS];
    // (the chunks are recomputed where the tail step needs them: kept from here,
    // they would hold registers across the whole main loop)
    auto achunk = [&](int q) { return ld_chunk(gw * A_INS + q); };
    auto bchunk = [&](int q) { return ld_chunk(gw * B_INS + q); };
#pragma unroll
    for (int q = 0; q < A_INS; ++q) {
        aoff[q] = (uint32_t)(((gw * A_INS + q) * 8 + ld_row) * p.lda + achunk(q) * 16);
    }
#pragma unroll
    for (int q = 0; q < B_INS; ++q) {
        boff[q] = (uint32_t)(((gw * B_INS + q) * 8 + ld_row) * p.ldb + bchunk(q) * 16);
    }
    // Slow 64x128 wave tiles keep only the two per-lane parts (the chunk depends on the instruction's
    // parity) and add the instruction's row block at issue: registers
    constexpr bool kRcOff = kRc && A_INS % 2 == 0 && B_INS % 2 == 0;
    static_assert(kRcOff == kRc, "the row-chunk loop's ragged K relies on per-lane step offsets");
    const uint32_t alane[2] = {(uint32_t)(ld_row * p.lda + ld_chunk(gw * A_INS) * 16),
                               (uint32_t)(ld_row * p.lda + ld_chunk(gw * A_INS + 1) * 16)};
    const uint32_t blane[2] = {(uint32_t)(ld_row * p.ldb + ld_chunk(gw * B_INS) * 16),
                               (uint32_t)(ld_row * p.ldb + ld_chunk(gw * B_INS + 1) * 16)};
    auto aoffq = [&](int q) -> uint32_t {
        return kRcOff ? alane[q & 1] + (uint32_t)((gw * A_INS + q) * 8 * p.lda) : aoff[q];
    };
    auto boffq = [&](int q) -> uint32_t {
        return kRcOff ? blane[q & 1] + (uint32_t)((gw * B_INS + q) * 8 * p.ldb) : boff[q];
    };

    const float* sa_l = p.sa + (int64_t)l * p.sa_batch;
    const float* sb_l = p.sb + (int64_t)l * p.sb_batch;
    // the tile's scale rows (rows past the matrix read zero, or the atom
    // layout's padding; their results are discarded)
    const int KB4 = (int)((p.sa_ld + 3) >> 2);  // atom layout: 4-group blocks per 128 rows
    const void* sa_t = kAtom ? (const void*)((const uint8_t*)sa_l + (int64_t)(m0 >> 7) * KB4 * 512)
                             : (const void*)(sa_l + (int64_t)m0 * p.sa_ld);
    const void* sb_t = kAtom ? (const void*)((const uint8_t*)sb_l + (int64_t)(n0 >> 7) * KB4 * 512)
                             : (const void*)(sb_l + (int64_t)n0 * p.sb_ld);
    const uint32_t sa_ext = kAtom ? (uint32_t)(((p.M + 127) / 128 - (m0 >> 7)) * KB4 * 512)
                                  : (SA_W ? (uint32_t)(min(BM, p.M - m0) * p.sa_ld * 4) : 0u);
    const uint32_t sb_ext = kAtom ? (uint32_t)(((p.N + 127) / 128 - (n0 >> 7)) * KB4 * 512)
                                  : (SB_W ? (uint32_t)(min(BN, p.N - n0) * p.sb_ld * 4) : 0u);
    const rsrc_t rsa = make_rsrc(sa_t, sa_ext);
    const rsrc_t rsb = make_rsrc(sb_t, sb_ext);
    // Atom layout: a load of 64 rows starting at row r0 (a multiple of 64)
    // of the 128-row blocks gathers, in lane order, row r0 + lane's dword of
    // the step's 512 bytes: byte (lane % 32) * 16 + 4 * ((r0 / 32) % 4 + lane / 32)
    // of its block, i.e. a per-lane part common to every load plus a uniform part.
    const uint32_t atom_lane = (uint32_t)((lane & 31) * 16 + (lane >> 5) * 4);
    auto atom_uni = [&](int r0) { return (r0 >> 7) * KB4 * 512 + ((r0 >> 5) & 3) * 4; };

    auto issue = [&](int kt, uint8_t* sbase) {
        if (kt >= KT) return;  // past the end: nothing to load
        const uint32_t kb = (uint32_t)(kt * kBK);
        // Where every chunk of the step lies inside its row, the step's K offset
        // rides in the scalar offset and the per-lane offsets stay loop-invariant
        // (rows past the matrix still read zero: their per-lane offset alone is
        // past the buffer's extent). In the last step of a ragged K the whole
        // offset goes in the per-lane part, which the range check covers (the
        // scalar part is not checked), so a chunk straddling the end of the last
        // row reads zeros past it; chunks starting at or past K get an
        // out-of-range offset.
        // The common path has loop-invariant per-lane offsets and no per-lane
        // arithmetic; the tail path is taken (a uniform branch) once per tile.
        auto load_ab = [&](auto tail) {
            constexpr bool TAIL = decltype(tail)::value;
            // (kRcOff: the step offset joins the per-lane sum at issue, which keeps the compiler from holding
            // every instruction's offset in a register across the loop)
            const int soff = (TAIL || kRcOff) ? 0 : (int)kb;
#pragma unroll
            for (int q = 0; q < A_INS; ++q) {
                uint32_t off = kRcOff ? alane[q & 1] + (uint32_t)((gw * A_INS + q) * 8 * p.lda + (int)kb) : aoffq(q);
                if constexpr (TAIL) {
                    if ((int)kb + achunk(q) * 16 >= K) off = kOOB;
                    else if (!kRcOff) off += kb;
                }
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(sbase + (gw * A_INS + q) * 1024), 16, off,
                                                         soff, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < B_INS; ++q) {
                uint32_t off = kRcOff ? blane[q & 1] + (uint32_t)((gw * B_INS + q) * 8 * p.ldb + (int)kb) : boffq(q);
                if constexpr (TAIL) {
                    if ((int)kb + bchunk(q) * 16 >= K) off = kOOB;
                    else if (!kRcOff) off += kb;
                }
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(sbase + BM * kBK + (gw * B_INS + q) * 1024),
                                                         16, off, soff, 0, 0);
            }
        };
        if (k_tail && kt == KT - 1) load_ab(IC<1>{});
        else load_ab(IC<0>{});
        // Scale columns: load t fills column j of rows 64 rg .. 64 rg + 63, at
        // LDS [j][row] after the tiles. MX groups past ceil(K/32) read whatever
        // follows (the next row, or zero past the last): their data is zero and
        // their conversion scale is replaced by 1 at use.
        if constexpr (kAtom) {
            // Load t brings dword u / RA (of the step's NKB) of rows
            // 64 (u % RA) .. + 63 of the tile, u = t % (RA NKB) (repeats when
            // kAtomRep > 1). The block part rides in the range-checked per-lane
            // offset, so blocks past the tensor's last (rows past M / N only)
            // read zero. FP8 steps are exactly the tensor's 4-group blocks, so
            // the step's 512 bytes ride in the scalar offset; an FP4 step's last
            // blocks can lie past a row block's end (groups past ceil(K/sf),
            // ignored at use), so its block index goes in the per-lane part too.
            constexpr int RA = BM < 128 ? 1 : BM / 64, RB = BN < 128 ? 1 : BN / 64;
            for (int t = gw; t < SC_A_INS; t += NW) {
                const int u = t % (RA * NKB), ta = u % RA, kb = u / RA;
                const uint32_t vo = atom_lane + atom_uni((BM < 128 ? (m0 & 127) : 0) + ta * 64);
                const uint32_t voff = kFp4 ? vo + (uint32_t)((kt * NKB + kb) * 512) : vo;
                const int soff = kFp4 ? 0 : kt * 512;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(sbase + (BM + BN) * kBK + u * 256), 4, voff,
                                                         soff, 0, 0);
            }
            for (int t = gw; t < SC_INS - SC_A_INS; t += NW) {
                const int u = t % (RB * NKB), tb = u % RB, kb = u / RB;
                const uint32_t vo = atom_lane + atom_uni((BN < 128 ? (n0 & 127) : 0) + tb * 64);
                const uint32_t voff = kFp4 ? vo + (uint32_t)((kt * NKB + kb) * 512) : vo;
                const int soff = kFp4 ? 0 : kt * 512;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsb, (lds_void*)(sbase + (BM + BN) * kBK + (SC_A_INS + u) * 256), 4, voff, soff, 0, 0);
            }
        } else if constexpr (SC_A_INS > 0) {
            for (int t = gw; t < SC_A_INS; t += NW) {
                const int j = t % SA_W, rg = t / SA_W;
                const uint32_t off = (uint32_t)(((rg * 64 + lane) * p.sa_ld + kt * SA_W + j) * 4);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsa, (lds_void*)(sbase + (BM + BN) * kBK + (j * BM + rg * 64) * 4), 4, off, 0, 0, 0);
            }
        }
        if constexpr (!kAtom && SC_INS > SC_A_INS) {
            for (int t = gw; t < SC_INS - SC_A_INS; t += NW) {
                const int j = t % SB_W, rg = t / SB_W;
                const uint32_t off = (uint32_t)(((rg * 64 + lane) * p.sb_ld + kt * SB_W + j) * 4);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsb, (lds_void*)(sbase + (BM + BN) * kBK + (BM * SA_W + j * BN + rg * 64) * 4), 4, off, 0, 0, 0);
            }
        }
    };
    // In the last step of a K that is not a multiple of 16, a chunk straddling K
    // holds bytes of the next row (or padding): zero them in this lane's own
    // LDS slots once its loads have landed. The row-chunk loop loads its ragged
    // last step like the others, so there every chunk at or past K is zeroed too.
    auto mask_straddle = [&](int kt, uint8_t* sbase) {
        // (the step's K offset is made opaque to the compiler: known to be the last step's, it let the masks be
        // computed before the main loop, where they held eight registers across it)
        int kbase = kt * kBK;
        asm volatile("" : "+s"(kbase));
        auto fix = [&](uint8_t* slot, int chunk) {
            const int k0 = kbase + chunk * 16;
            if (kRc ? K >= k0 + 16 : !(k0 < K && K < k0 + 16)) return;
            const int valid = K - k0;
            i32x4 v = *(i32x4*)slot;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int nb = valid - 4 * d;  // valid bytes in dword d
                const uint32_t m = nb >= 4 ? 0xFFFFFFFFu : (nb <= 0 ? 0u : ((1u << (8 * nb)) - 1u));
                v[d] = (int)((uint32_t)v[d] & m);
            }
            *(i32x4*)slot = v;
        };
#pragma unroll
        for (int q = 0; q < A_INS; ++q) fix(sbase + (gw * A_INS + q) * 1024 + lane * 16, achunk(q));
#pragma unroll
        for (int q = 0; q < B_INS; ++q) fix(sbase + BM * kBK + (gw * B_INS + q) * 1024 + lane * 16, bchunk(q));
    };

    // Fragment reads: lane (r, g) takes chunks 2g and 2g + 1 of row r, i.e.
    // k = 32g .. 32g + 31 of the step: one 32-element scale group per lane.
    const int fr = lane & 15, fg = lane >> 4;
    const int fsw = (fr & 7) ^ (fr >> 3);  // swz of the fragment's row (fragments start at multiples of 16)
    // With the scaled FP4 MFMA, half h of a step is one instruction's K = 128 values: lane (r, g) takes chunk
    // 4 h + g of row r, the 32 values of scale group 4 h + g.
    const int foff0 = fr * kBK + (((kFp4Mfma ? fg : 2 * fg) ^ fsw) << 4);
    const int foff1 = fr * kBK + (((kFp4Mfma ? 4 + fg : 2 * fg + 1) ^ fsw) << 4);

    f32x4 acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // 128x128 scale_b: one value per 128 columns, the same for the whole
    // fragment (clamped to the matrix: results of clamped columns are discarded).
    int srow_b[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) srow_b[j] = min((n0 + wn * WTN + j * 16) / 128, (p.N - 1) / 128);
    // epilogue scales, read now so that their latency hides behind the main loop
    float alpha = 1.0f;
    if (MODE == MODE_FAST || MODE == MODE_SLOW) alpha = p.sa[0] * p.sb[0];
    const bool fp8_out = p.d_type == T_E4M3 || p.d_type == T_E5M2;
    const float sr = (fp8_out && p.scale_result) ? p.scale_result[0] : 1.0f;

    // 128x128 scale_b of one step, loaded one step ahead of its use (the other
    // scales come through LDS with the tiles).
    constexpr bool kSbMem = MODE == MODE_BLOCK && SBM == SB_128x128;
    // the wave's columns lie in one 128-column block of scale_b (WTN divides 128)
    constexpr bool kSbOne = kSbMem && 128 % WTN == 0;
    struct StepScales {
        float b[FN];
    };
    auto load_scales = [&](int kt) {
        StepScales sc;
        if (KT == 0) return sc;  // K = 0: no step reads them (and the tables may be empty)
        kt = min(kt, KT - 1);    // the prefetch past the last step reads a valid entry
        if constexpr (kSbOne) {
            sc.b[0] = sb_l[(int64_t)srow_b[0] * p.sb_ld + kt];  // every fragment of the wave is in this block
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j) sc.b[j] = sb_l[(int64_t)srow_b[j] * p.sb_ld + kt];
        }
        return sc;
    };
    StepScales sc_cur;
    if (kSbMem) sc_cur = load_scales(kg);

    // Main loop, two LDS stages, software-pipelined by half-steps: the lane's
    // 32 bytes of a step are read as two 16-byte halves (sub-steps 0-1, 2-3),
    // and each half's fragment reads are issued before the MFMAs of the half
    // before it, so the LDS latency hides behind MFMA work. The stage barrier
    // sits in the middle of a step, once that step's second-half fragments are
    // read: past it the stage just read is free for the loads two steps ahead,
    // and the next step's first-half fragments can be read.
    struct Frag {
        i32x4 a[FM];
        i32x4 b[FN];
    };
    auto read_frag = [&](const uint8_t* stage, int h, Frag& f) {
        const int fo = h ? foff1 : foff0;
        const uint8_t* As = stage + wm * WTM * kBK;
        const uint8_t* Bs = stage + BM * kBK + wn * WTN * kBK;
#pragma unroll
        for (int i = 0; i < FM; ++i) f.a[i] = *(const i32x4*)(As + i * 16 * kBK + fo);
#pragma unroll
        for (int j = 0; j < FN; ++j) f.b[j] = *(const i32x4*)(Bs + j * 16 * kBK + fo);
    };
    // Fast / MX: one chain over K straight into the accumulators. Slow / block:
    // a fresh fp32 partial per 128-chunk, promoted into the accumulator after.
    constexpr bool chain = MODE == MODE_FAST || MODE == MODE_SF32;
    f32x4 part[chain ? 1 : FN][chain ? 1 : FM];
    auto mma_half = [&](const Frag& f, const float* c_a, const float* c_b) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            bf16x8 ab[FM];
#pragma unroll
            for (int i = 0; i < FM; ++i) ab[i] = to_bf16x8<FA>(f.a[i], q, c_a[i]);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const bf16x8 bb = to_bf16x8<FB>(f.b[j], q, c_b[j]);
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    if constexpr (chain) acc[j][i] = mfma_bf16(bb, ab[i], acc[j][i]);
                    else part[j][i] = mfma_bf16(bb, ab[i], part[j][i]);
                }
            }
        }
    };
    // FP4: the scale group of a lane's values changes within a step. Chunk
    // 2 fg + h holds values [32 (2 fg + h), + 32) of the step: group 2 fg + h
    // with 32 values per group, or 4 fg + 2 h + qp (k-slices 2 qp, 2 qp + 1)
    // with 16. Byte g % 4 of LDS dword [g / 4][row] holds the factor.
    auto fp4_scales = [&](int kt, const uint8_t* stage, int h, int qp, float* c_a, float* c_b) {
        const int g = SFV == 32 ? 2 * fg + h : 4 * fg + 2 * h + qp;
        const bool gv = kt * GPS + g < p.sa_ld;  // groups past ceil(K/sf) hold zero data
        const uint8_t* eA = stage + (BM + BN) * kBK + (g >> 2) * BM * 4 + (g & 3);
        const uint8_t* eB = stage + (BM + BN) * kBK + SC_A_INS * 256 + (g >> 2) * BN * 4 + (g & 3);
        auto factor = [&](uint32_t code) {
            if constexpr (kE4M3) return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);  // exact, NaN for 0x7F / 0xFF
            else return e8m0_code_scale(code);
        };
#pragma unroll
        for (int i = 0; i < FM; ++i) c_a[i] = gv ? factor(eA[(wm * WTM + i * 16 + fr) * 4]) : 1.0f;
#pragma unroll
        for (int j = 0; j < FN; ++j) c_b[j] = gv ? factor(eB[(wn * WTN + j * 16 + fr) * 4]) : 1.0f;
    };
    auto mma_half4 = [&](const Frag& f, int kt, const uint8_t* stage, int h) {
        constexpr int QPS = SFV == 32 ? 4 : 2;  // k-slices per scale group
#pragma unroll
        for (int qp = 0; qp < 4 / QPS; ++qp) {
            float c_a[FM], c_b[FN];
            fp4_scales(kt, stage, h, qp, c_a, c_b);
#pragma unroll
            for (int qq = 0; qq < QPS; ++qq) {
                const int q = qp * QPS + qq;
                if constexpr (kE4M3) {
                    f16x8 ab[FM];
#pragma unroll
                    for (int i = 0; i < FM; ++i) ab[i] = fp4_to_f16x8(f.a[i], q, (_Float16)c_a[i]);
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const f16x8 bb = fp4_to_f16x8(f.b[j], q, (_Float16)c_b[j]);
#pragma unroll
                        for (int i = 0; i < FM; ++i) acc[j][i] = mfma_f16(bb, ab[i], acc[j][i]);
                    }
                } else {
                    bf16x8 ab[FM];
#pragma unroll
                    for (int i = 0; i < FM; ++i) ab[i] = fp4_to_bf16x8(f.a[i], q, c_a[i]);
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const bf16x8 bb = fp4_to_bf16x8(f.b[j], q, c_b[j]);
#pragma unroll
                        for (int i = 0; i < FM; ++i) acc[j][i] = mfma_bf16(bb, ab[i], acc[j][i]);
                    }
                }
            }
        }
    };
    // FP4 on the scaled MFMA: half h of the step is one K = 128 instruction per 16 x 16 block; lane (r, g)
    // passes its group's E8M0 code (byte g of LDS dword [h][row], the step's groups 4 h .. 4 h + 3), 127 (a
    // factor of 1) for groups past ceil(K/32), whose data is zero.
    auto mma_fp4_scaled = [&](const Frag& f, int kt, const uint8_t* stage, int h) {
        if constexpr (kFp4Mfma) {
            const bool gv = kt * GPS + 4 * h + fg < p.sa_ld;
            const uint32_t* wA = (const uint32_t*)(stage + (BM + BN) * kBK) + h * BM;
            const uint32_t* wB = (const uint32_t*)(stage + (BM + BN) * kBK + SC_A_INS * 256) + h * BN;
            int sa[FM], sb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) sa[i] = gv ? (int)((wA[wm * WTM + i * 16 + fr] >> (8 * fg)) & 0xFFu) : 127;
#pragma unroll
            for (int j = 0; j < FN; ++j) sb[j] = gv ? (int)((wB[wn * WTN + j * 16 + fr] >> (8 * fg)) & 0xFFu) : 127;
            const i32x4 z = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cat(f.b[j], z), cat(f.a[i], z),
                                                                                 acc[j][i], 4, 4, 0, sb[j], 0, sa[i]);
        }
    };
    // The scales of step kt: s_a / s_b fold a block-scaled partial into the
    // accumulator, c_a / c_b ride in the FP8 -> bf16 conversion (MX groups).
    // They are read from the step's stage before the barrier that frees it.
    auto step_scales = [&](int kt, const uint8_t* stage, float* s_a, float (*s_b)[4], float* c_a, float* c_b) {
        const float* scA = (const float*)(stage + (BM + BN) * kBK);
        const float* scB = scA + BM * SA_W;
        if (MODE == MODE_BLOCK) {
#pragma unroll
            for (int i = 0; i < FM; ++i) s_a[i] = scA[wm * WTM + i * 16 + fr];
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s_b[j][r] = kSbMem ? sc_cur.b[kSbOne ? 0 : j] : scB[wn * WTN + j * 16 + 4 * fg + r];
        }
        if (MODE == MODE_SF32 && kAtom) {
            // the row's dword holds the step's 4 groups; byte fg is this lane's
            const bool gv = kt * 4 + fg < p.sa_ld;  // groups past ceil(K/32) hold zero data
            const uint32_t* wA = (const uint32_t*)scA;
            const uint32_t* wB = wA + SC_A_INS * 64;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                c_a[i] = gv ? e8m0_code_scale((wA[wm * WTM + i * 16 + fr] >> (8 * fg)) & 0xFFu) : 1.0f;
#pragma unroll
            for (int j = 0; j < FN; ++j)
                c_b[j] = gv ? e8m0_code_scale((wB[wn * WTN + j * 16 + fr] >> (8 * fg)) & 0xFFu) : 1.0f;
        } else if (MODE == MODE_SF32) {
            const bool gv = kt * 4 + fg < p.sa_ld;  // groups past ceil(K/32) hold zero data
#pragma unroll
            for (int i = 0; i < FM; ++i) c_a[i] = gv ? e8m0_scale(scA[fg * BM + wm * WTM + i * 16 + fr]) : 1.0f;
#pragma unroll
            for (int j = 0; j < FN; ++j) c_b[j] = gv ? e8m0_scale(scB[fg * BN + wn * WTN + j * 16 + fr]) : 1.0f;
        } else {
#pragma unroll
            for (int i = 0; i < FM; ++i) c_a[i] = 1.0f;
#pragma unroll
            for (int j = 0; j < FN; ++j) c_b[j] = 1.0f;
        }
    };
    auto promote = [&](const float* s_a, const float (*s_b)[4]) {
        if constexpr (!chain) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    if (MODE == MODE_SLOW) {
                        acc[j][i] += part[j][i];
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[j][i][r] = __builtin_fmaf(part[j][i][r], s_a[i] * s_b[j][r], acc[j][i][r]);
                    }
                }
        }
    };
    auto zero_part = [&]() {
        if constexpr (!chain) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int i = 0; i < FM; ++i) part[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    // The stage of step kt has landed in every wave: wait for this wave's loads,
    // mask a chunk straddling a ragged K, then the workgroup barrier (its
    // workgroup fence also makes the compiler drain every outstanding load;
    // issuing the loads untracked with a fence-free barrier measured no faster).
    auto stage_ready = [&](int kt, uint8_t* stage) {
        __builtin_amdgcn_s_waitcnt(0);
        if (kRc ? (kt == KT - 1 && (K % kBK) != 0) : (k_tail && kt == KT - 1 && (K & 15))) mask_straddle(kt, stage);
        __syncthreads();
    };

    // FP8 operands on square wave tiles take the interleaved loop below, block
    // scaling only with a 128x128 scale_b whose 128-column blocks hold whole wave
    // tiles (one s_b per wave and step): with a scale_b per column its step
    // scales on top of the second operand set push that loop past the register
    // file
    constexpr bool kIlv = !PIPE && !kFp4 && FM == FN && (MODE != MODE_BLOCK || kSbOne);

    if constexpr (kRc) {
        // Each step converts the wave's A fragments for all four K = 32 sub-steps once (the first sub-step's
        // before the first MFMA, the others between the first row's MFMAs) and then walks the B fragment rows.
        // Row j's four accumulation chains (one per A fragment) take their four MFMAs back to back,
        // interleaved over the A fragments, while the next row's B fragment is read and converted; B is thus
        // converted once per wave for four A fragments and A once for eight B fragments (1.5 conversions per
        // MFMA against 2 on 64x64 wave tiles).
        //  * Promoted modes: each row's 128-chunk partials start from zero and are folded into the
        //    accumulators just before the next row's first MFMAs overwrite them (acc += part; block scaling
        //    acc = fma(part, s_a * s_b, acc) with s_a of the A fragment's row from the stage's scale column and
        //    the step's one s_b). Only FM partials are live, which lets the promoted modes use the 64x128 tile.
        //  * Chained modes (fast, MX): each MFMA accumulates straight into acc, the MX factors of the step
        //    riding in the conversions.
        // Every accumulator sees its K values in the order of the other loops, so the results are the same bit
        // for bit.
        constexpr bool rc_chain = MODE == MODE_FAST || MODE == MODE_SF32;
        auto step = [&](int kt, uint8_t* cur, uint8_t* nxt) {
            stage_ready(kt, cur);
            float c_a[FM], c_b[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) c_a[i] = 1.0f;
#pragma unroll
            for (int j = 0; j < FN; ++j) c_b[j] = 1.0f;
            if constexpr (MODE == MODE_SF32) {
                float s_a[FM], s_b[FN][4];
                step_scales(kt, cur, s_a, s_b, c_a, c_b);
            }
            float sab[FM];
            if constexpr (MODE == MODE_BLOCK) {
                const float sb = sc_cur.b[0];
                sc_cur = load_scales(kt + 1);
                const float* sa_col = (const float*)(cur + (BM + BN) * kBK) + wm * WTM + fr;
#pragma unroll
                for (int i = 0; i < FM; ++i) sab[i] = sa_col[16 * i] * sb;
            }
            // (one vector fma per fragment: written per element, the fold pushed this loop past the register file)
            auto fold = [&](f32x4& a, const f32x4& part, int i) {
                if constexpr (MODE == MODE_BLOCK) a = __builtin_elementwise_fma(part, f32x4{sab[i], sab[i], sab[i], sab[i]}, a);
                else a += part;
            };
            issue(kt + 1, nxt);
            const uint8_t* As = cur + wm * WTM * kBK;
            const uint8_t* Bs = cur + BM * kBK + wn * WTN * kBK;
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            i32x4 ra[2][FM];
            bf16x8 xa[4][FM];
#pragma unroll
            for (int i = 0; i < FM; ++i) ra[0][i] = *(const i32x4*)(As + i * 16 * kBK + foff0);
            i32x4 rb0 = *(const i32x4*)(Bs + foff0), rb1 = *(const i32x4*)(Bs + foff1);
#pragma unroll
            for (int i = 0; i < FM; ++i) ra[1][i] = *(const i32x4*)(As + i * 16 * kBK + foff1);
#pragma unroll
            for (int i = 0; i < FM; ++i) xa[0][i] = to_bf16x8<FA>(ra[0][i], 0, c_a[i]);
            bf16x8 xb = to_bf16x8<FB>(rb0, 0, c_b[0]);
            f32x4 pt[FM];
            i32x4 nb0 = rb0, nb1 = rb1;
            __builtin_amdgcn_sched_barrier(0);
            // sub-step u of B fragment row j (compile-time j and u: the scheduling pattern depends on them)
            auto sub = [&](auto jc, auto uc) {
                constexpr int j = decltype(jc)::value, u = decltype(uc)::value;
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    if constexpr (rc_chain) {
                        acc[j][i] = mfma_bf16(xb, xa[u][i], acc[j][i]);
                    } else {
                        if constexpr (u == 0 && j > 0) fold(acc[j - 1][i], pt[i], i);
                        pt[i] = mfma_bf16(xb, xa[u][i], u == 0 ? z : pt[i]);
                    }
                }
                if constexpr (j == 0 && u < 3) {  // the A operands of the next sub-step
#pragma unroll
                    for (int i = 0; i < FM; ++i) xa[u + 1][i] = to_bf16x8<FA>(ra[(u + 1) / 2][i], (u + 1) & 1, c_a[i]);
                }
                // (the next row's halves are read once this row's have been converted for the last time, so
                // that one half of each is live at a time)
                if constexpr (u == 1 && j + 1 < FN) nb0 = *(const i32x4*)(Bs + (j + 1) * 16 * kBK + foff0);
                if constexpr (u < 3) xb = to_bf16x8<FB>(u + 1 < 2 ? rb0 : rb1, (u + 1) & 1, c_b[j]);
                else if constexpr (j + 1 < FN) xb = to_bf16x8<FB>(nb0, 0, c_b[j + 1]);
                if constexpr (u == 2 && j + 1 < FN) nb1 = *(const i32x4*)(Bs + (j + 1) * 16 * kBK + foff1);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (u == 3) {
                    rb0 = nb0;
                    rb1 = nb1;
                }
            };
            auto row = [&](auto jc) {
                sub(jc, IC<0>{});
                sub(jc, IC<1>{});
                sub(jc, IC<2>{});
                sub(jc, IC<3>{});
            };
            static_assert(FN == 8, "eight B fragment rows");
            row(IC<0>{}); row(IC<1>{}); row(IC<2>{}); row(IC<3>{});
            row(IC<4>{}); row(IC<5>{}); row(IC<6>{}); row(IC<7>{});
            if constexpr (!rc_chain) {
#pragma unroll
                for (int i = 0; i < FM; ++i) fold(acc[FN - 1][i], pt[i], i);
            }
        };
        issue(0, smem0);
        for (int kt = 0; kt < KT; kt += 2) {
            step(kt, smem0, smem1);
            if (kt + 1 < KT) step(kt + 1, smem1, smem0);
        }
    } else if constexpr (PIPE) {
        Frag f0, f1;
        auto step = [&](int kt, uint8_t* cur, uint8_t* nxt) {
            float s_a[FM], s_b[FN][4], c_a[FM], c_b[FN];
            step_scales(kt, cur, s_a, s_b, c_a, c_b);
            if (kSbMem) sc_cur = load_scales(kt + 1);
            zero_part();
            read_frag(cur, 1, f1);  // second half of this step, under the first half's MFMAs
            mma_half(f0, c_a, c_b);
            stage_ready(kt + 1, nxt);
            issue(kt + 2, cur);  // the stage just read, for the step after next
            if (kt + 1 < KT) read_frag(nxt, 0, f0);  // next step's first half, under this half's MFMAs
            mma_half(f1, c_a, c_b);
            promote(s_a, s_b);
        };
        if (KT > 0) {
            issue(0, smem0);
            stage_ready(0, smem0);
            issue(1, smem1);
            read_frag(smem0, 0, f0);
            for (int kt = 0; kt < KT; kt += 2) {
                step(kt, smem0, smem1);
                if (kt + 1 < KT) step(kt + 1, smem1, smem0);
            }
        }
    } else if constexpr (kIlv) {
        // the interleaved step of ilv_step (slow mode promotes per step, block
        // scaling folds the partial in with s_a of the row times the step's s_b)
        auto step = [&](int s, uint8_t* cur, uint8_t* nxt) {
            const int kt = s * KG + kg;
            uint8_t* cs = cur + kg * STAGE;
            stage_ready(kt, cs);
            float c_a[FM], c_b[FN];
            float sb = 1.0f;
            if (kt < KT) {
                if constexpr (MODE == MODE_BLOCK) {
#pragma unroll
                    for (int i = 0; i < FM; ++i) c_a[i] = 1.0f;
#pragma unroll
                    for (int j = 0; j < FN; ++j) c_b[j] = 1.0f;
                    sb = sc_cur.b[0];
                    sc_cur = load_scales(kt + KG);
                } else {
                    float s_a[FM], s_b[FN][4];
                    step_scales(kt, cs, s_a, s_b, c_a, c_b);
                }
            }
            issue(kt + KG, nxt + kg * STAGE);
            if (kt < KT) {
                const uint8_t* As = cs + wm * WTM * kBK;
                const uint8_t* Bs = cs + BM * kBK + wn * WTN * kBK;
                if constexpr (chain) ilv_step<FA, FB, FM, true>(As, Bs, foff0, foff1, c_a, c_b, acc, acc);
                else if constexpr (MODE == MODE_BLOCK)
                    ilv_step<FA, FB, FM, false, true>(As, Bs, foff0, foff1, c_a, c_b, acc, part,
                                                      (const float*)(cs + (BM + BN) * kBK) + wm * WTM + fr, sb);
                else ilv_step<FA, FB, FM, false>(As, Bs, foff0, foff1, c_a, c_b, acc, part);
            }
        };
        issue(kg, smem0 + kg * STAGE);
        const int KS = (KT + KG - 1) / KG;
        for (int s = 0; s < KS; s += 2) {
            step(s, smem0, smem1);
            if (s + 1 < KS) step(s + 1, smem1, smem0);
        }
    } else {
        // Each half-step reads its fragments and then multiplies; a second wave
        // on the SIMD covers the read latency.
        // One step of each K group (super-step s: K step s * KG + kg of group kg,
        // in that group's part of the stage); every wave takes the barrier.
        auto step = [&](int s, uint8_t* cur, uint8_t* nxt) {
            const int kt = s * KG + kg;
            uint8_t* cs = cur + kg * STAGE;
            stage_ready(kt, cs);
            float s_a[FM], s_b[FN][4], c_a[FM], c_b[FN];
            if (kt < KT) {
                if constexpr (!kFp4) step_scales(kt, cs, s_a, s_b, c_a, c_b);
                if (kSbMem) sc_cur = load_scales(kt + KG);
            }
            issue(kt + KG, nxt + kg * STAGE);
            if (kt < KT) {
                zero_part();
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    // keep the scheduler from hoisting the second half's reads and
                    // converts above the first half's MFMAs (that costs registers, not time)
                    if (h) __builtin_amdgcn_sched_barrier(0);
                    Frag f;
                    read_frag(cs, h, f);
                    if constexpr (kFp4Mfma) mma_fp4_scaled(f, kt, cs, h);
                    else if constexpr (kFp4) mma_half4(f, kt, cs, h);
                    else mma_half(f, c_a, c_b);
                }
                promote(s_a, s_b);
            }
        };
        issue(kg, smem0 + kg * STAGE);
        const int KS = (KT + KG - 1) / KG;
        for (int s = 0; s < KS; s += 2) {
            step(s, smem0, smem1);
            if (s + 1 < KS) step(s + 1, smem1, smem0);
        }
    }
    // the loads issued for steps past the end (they fetch nothing) must land
    // before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(0);

    // K groups: group g keeps fragment rows [g FM / 2, (g + 1) FM / 2) of its
    // wave tile and receives the other group's partial for them through LDS.
    // The two partials are added in one fp32 addition, the same either way round.
    constexpr int FMG = FM / KG;  // fragment rows each group stores
    if constexpr (KG > 1) {
        static_assert(KG == 2 && FM % 2 == 0, "two K groups, even fragment rows");
        static_assert(2 * NW * FN * FMG * 64 * 16 <= KG * STAGE, "the exchange fits in one stage pair");
        f32x4* xch = (f32x4*)smem0;  // [to group][wave][j][ii][lane]
        // (the group is a template argument here: indexing acc by a runtime
        // group would put the accumulators in scratch memory)
        auto exchange = [&](auto grp) {
            constexpr int G = decltype(grp)::value, O = 1 - G;
            __syncthreads();  // every wave is done with the stages
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int ii = 0; ii < FMG; ++ii)
                    xch[(((O * NW + gw) * FN + j) * FMG + ii) * 64 + lane] = acc[j][O * FMG + ii];
            __syncthreads();
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int ii = 0; ii < FMG; ++ii)
                    acc[j][G * FMG + ii] += xch[(((G * NW + gw) * FN + j) * FMG + ii) * 64 + lane];
        };
        if (kg) exchange(IC<1>{});
        else exchange(IC<0>{});
    }

    // ---------------------------------------------------------- epilogue
    // Compiled once per output type and amax kind (AM: 0 none, 1 |x| bits,
    // 2 key with index); amax is only asked of the MX entry.
    const int64_t dbase = (int64_t)l * p.d_batch;
    const bool want_amax = p.amax_bits || p.amax_key;
    const bool vec = p.vec_store != 0;
    uint32_t kb = 0;
    unsigned long long kk = 0;
    // 2-byte outputs of a whole tile go out through LDS: each wave writes its
    // converted results into its own region of the (now idle) stages, row-major
    // with 16-byte chunk c of row r at chunk c ^ (r mod chunks-per-row), and
    // reads them back as 16 bytes per lane along rows, so that every store
    // instruction writes whole 128-byte row segments. (Written straight from
    // the MFMA layout, each store covers 16 rows with 32 bytes each.)
    const bool full_tile = m0 + BM <= p.M && n0 + BN <= p.N;
    const bool st16 = ((uintptr_t)p.d & 15) == 0 && (p.ldd & 7) == 0 && (p.d_batch & 7) == 0;
    constexpr int RB = WTN * 2;  // bytes per row of a wave's region
    constexpr int CH = RB / 16;  // 16-byte chunks per row
    constexpr int RROWS = WTM / KG;  // rows of a wave's region
    static_assert((NW * KG / 2) * RROWS * RB <= KG * STAGE, "the output regions of half the waves fit in one stage");
    auto epilogue = [&](auto ot, auto am, auto grp, auto bi) {
        constexpr int OT = decltype(ot)::value, AM = decltype(am)::value, G = decltype(grp)::value;
        constexpr bool BI = decltype(bi)::value != 0;
        // the bias of this lane's columns (the same for every row)
        float bv[FN][4];
        if constexpr (BI) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = n0 + wn * WTN + j * 16 + 4 * fg + e;
                    bv[j][e] = n < p.N ? load_bias<OT>(p.bias, n) : 0.0f;
                }
        }
        if constexpr (OT == T_BF16 || OT == T_F16) {
            if (full_tile && st16) {
                uint8_t* region = (wave < NW * KG / 2 ? smem0 : smem1) + (wave % (NW * KG / 2)) * (RROWS * RB);
                __syncthreads();  // every wave is done with the stages
                const int mr = m0 + wm * WTM + G * RROWS;  // first row of the region
#pragma unroll
                for (int ii = 0; ii < FMG; ++ii) {
                    const int i = G * FMG + ii, r = ii * 16 + fr;
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        uint32_t out[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float v = (acc[j][i][e] + 0.0f) * alpha;
                            if constexpr (BI) v += bv[j][e];
                            if constexpr (AM == 2) {
                                const unsigned long long key = amax_key(
                                    v, (int64_t)l * p.M * p.N + (int64_t)(mr + r) * p.N + n0 + wn * WTN + j * 16 +
                                           4 * fg + e);
                                kk = key > kk ? key : kk;
                            } else if constexpr (AM == 1) {
                                const uint32_t a = abs_bits(v);
                                kb = a > kb ? a : kb;
                            }
                            out[e] = convert_t<OT>(v);
                        }
                        const int c = 2 * j + (fg >> 1);
                        *(i32x2*)(region + r * RB + ((c ^ (r & (CH - 1))) << 4) + ((fg & 1) << 3)) =
                            i32x2{(int)(out[0] | (out[1] << 16)), (int)(out[2] | (out[3] << 16))};
                    }
                }
                // each wave reads back only its own region
                constexpr int RPI = 64 / CH;  // rows per instruction
#pragma unroll
                for (int it = 0; it < RROWS / RPI; ++it) {
                    const int r = it * RPI + lane / CH, c = lane % CH;
                    const i32x4 v = *(const i32x4*)(region + r * RB + ((c ^ (r & (CH - 1))) << 4));
                    uint16_t* d = (uint16_t*)p.d + dbase + (int64_t)(mr + r) * p.ldd + n0 + wn * WTN + c * 8;
                    *(i32x4*)d = v;
                }
                return;
            }
        }
#pragma unroll
        for (int ii = 0; ii < FMG; ++ii) {
            const int i = G * FMG + ii;
            const int m = m0 + wm * WTM + i * 16 + fr;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * WTN + j * 16 + 4 * fg;
                const int valid = (m < p.M) ? max(0, min(4, p.N - n)) : 0;
                uint32_t out[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // +0.0f turns a -0 sum into +0: a sum of products starts from +0
                    float v = (acc[j][i][r] + 0.0f) * alpha;
                    if constexpr (BI) v += bv[j][r];
                    if constexpr (AM == 2) {
                        const unsigned long long key = amax_key(v, (int64_t)l * p.M * p.N + (int64_t)m * p.N + n + r);
                        if (r < valid) kk = key > kk ? key : kk;
                    } else if constexpr (AM == 1) {
                        const uint32_t a = abs_bits(v);
                        if (r < valid) kb = a > kb ? a : kb;
                    }
                    if constexpr (OT == T_E4M3 || OT == T_E5M2) v *= sr;
                    out[r] = convert_t<OT>(v);
                }
                if (valid > 0) store4<OT>(p.d, dbase + (int64_t)m * p.ldd + n, out, valid, vec);
            }
        }
    };
    // the group's half of the rows (K groups), with compile-time fragment indices
    auto epilogue_g = [&](auto ot, auto am, auto bi) {
        if (KG > 1 && kg) epilogue(ot, am, IC<KG - 1>{}, bi);
        else epilogue(ot, am, IC<0>{}, bi);
    };
    if constexpr (MODE == MODE_SF32) {
        // the MX entries write f32, bf16 or f16, and FP8 or FP4 (E2M1) with FP4 operands
        auto with_amax = [&](auto ot) {
            if (p.amax_key) epilogue_g(ot, IC<2>{}, IC<0>{});
            else if (p.amax_bits) epilogue_g(ot, IC<1>{}, IC<0>{});
            else epilogue_g(ot, IC<0>{}, IC<0>{});
        };
        if (p.d_type == T_BF16) with_amax(IC<T_BF16>{});
        else if (p.d_type == T_F16) with_amax(IC<T_F16>{});
        else if (p.d_type == T_F32 || !kFp4) with_amax(IC<T_F32>{});
        else if constexpr (kFp4) {
            if (p.d_type == T_E4M3) with_amax(IC<T_E4M3>{});
            else if (p.d_type == T_E5M2) with_amax(IC<T_E5M2>{});
            else with_amax(IC<T_E2M1>{});
        }
    } else {
        // a bias (f32, bf16 and f16 outputs) is another compile-time variant
        with_out_type(p.d_type, [&](auto ot) {
            constexpr int OT = decltype(ot)::value;
            if constexpr (OT == T_F32 || OT == T_BF16 || OT == T_F16) {
                if (p.bias) epilogue_g(ot, IC<0>{}, IC<1>{});
                else epilogue_g(ot, IC<0>{}, IC<0>{});
            } else {
                epilogue_g(ot, IC<0>{}, IC<0>{});
            }
        });
    }
    if (want_amax) amax_commit<NT>(p, kb, kk);
}

// ------------------------------------------------------------------ skinny kernel
//
// For M <= 16 * MT (MT <= 4) with per-tensor scales the run is bound by
// streaming B (N x K bytes) once from HBM; A is small and every workgroup reads
// all of it from L2. A workgroup owns 16 columns of the output (one workgroup
// per CU at N = 4096); its NW waves split the K steps round-robin (wave w
// takes steps w, w + NW, ...) with KU steps in flight each, so that most of B
// is in flight at once. B fragments go straight from memory into registers.
// A is read in contiguous 1 KB pieces (8 rows of 128 bytes per instruction:
// read in fragment order, 16 rows per instruction, the L2 -> CU path delivers
// it at a fraction of the rate), written to the wave's own LDS slot and read
// back as fragments. Lane (r, g) holds k = 32 g .. 32 g + 31 of row r in each
// step. The waves' partial tiles are added in a fixed order at the end.
template <int MT, int MODE, int FA, int FB, int NW, int KU>
__global__ void __launch_bounds__(NW * 64) gemm_skinny(GemmArgs p) {
    static_assert(KU >= 1 && KU <= 4, "steps in flight per wave");
    constexpr int AROWS = 16 * MT;
    constexpr int A_INS = AROWS / 8;     // 1 KB loads of A per step
    constexpr int SLOT = AROWS * kBK;    // one step of A
    constexpr int RED = (NW - 1) * MT * 64 * 16;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NW * SLOT > RED ? NW * SLOT : RED];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 16;
    const int K = p.K, KT = (K + kBK - 1) / kBK;
    const int fr = lane & 15, fg = lane >> 4;
    const rsrc_t rb = make_rsrc(p.b + (int64_t)n0 * p.ldb, operand_extent(min(16, p.N - n0), p.ldb, K));
    const rsrc_t ra = make_rsrc(p.a, operand_extent(p.M, p.lda, K));
    const uint32_t boff = (uint32_t)(fr * p.ldb + 32 * fg);
    // epilogue scales, read now so that their latency hides behind the main loop
    const float alpha = p.sa[0] * p.sb[0];
    const bool fp8_out = p.d_type == T_E4M3 || p.d_type == T_E5M2;
    const float sr = (fp8_out && p.scale_result) ? p.scale_result[0] : 1.0f;

    // A: instruction q reads rows 8q .. 8q+7 of the step; lane l takes row
    // 8q + l/8, chunk c = l%8, and stores it at chunk c ^ swz(row),
    // swz(r) = (r & 7) ^ ((r >> 3) & 1), so that the fragment reads below are
    // free of LDS bank conflicts.
    const int ld_row = lane >> 3, ld_chunk = lane & 7;
    uint32_t aoff[A_INS];
    int awr[A_INS];
#pragma unroll
    for (int q = 0; q < A_INS; ++q) {
        const int row = q * 8 + ld_row;
        aoff[q] = (uint32_t)(row * p.lda + ld_chunk * 16);
        awr[q] = row * kBK + ((ld_chunk ^ ld_row ^ (q & 1)) << 4);
    }
    const int fsw = (fr & 7) ^ (fr >> 3);
    const int foff0 = fr * kBK + (((2 * fg) ^ fsw) << 4);
    const int foff1 = fr * kBK + (((2 * fg + 1) ^ fsw) << 4);
    uint8_t* const slot = lds + wave * SLOT;

    struct Step {
        i32x4 a[A_INS];
        i32x8 b;
    };
    // Loads of step kt; chunks starting at or past K read zero (the range check
    // returns 0 for an out-of-range offset); a chunk straddling K is masked below.
    auto load = [&](int kt, Step& st) {
        const uint32_t kb = (uint32_t)(kt * kBK);
        const bool tail = kt * kBK + kBK > K;
#pragma unroll
        for (int q = 0; q < A_INS; ++q) {
            uint32_t off = aoff[q] + kb;
            if (tail && (int)kb + ld_chunk * 16 >= K) off = kOOB;
            st.a[q] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
        }
        const int k0 = kt * kBK + 32 * fg;
        uint32_t o0 = boff + kb, o1 = boff + kb + 16;
        if (tail && k0 >= K) o0 = kOOB;
        if (tail && k0 + 16 >= K) o1 = kOOB;
        const i32x4 b0 = __builtin_amdgcn_raw_buffer_load_b128(rb, o0, 0, 0);
        const i32x4 b1 = __builtin_amdgcn_raw_buffer_load_b128(rb, o1, 0, 0);
        st.b = cat(b0, b1);
    };
    auto keep = [&](int ks, int d) -> uint32_t {  // byte mask of dword d of a chunk at ks
        const int nb = K - ks - 4 * d;
        return nb >= 4 ? 0xFFFFFFFFu : (nb <= 0 ? 0u : ((1u << (8 * nb)) - 1u));
    };
    auto mask = [&](int kt, Step& st) {
#pragma unroll
        for (int q = 0; q < A_INS; ++q) {
            const int ks = kt * kBK + ld_chunk * 16;
            if (ks < K && K < ks + 16) {
#pragma unroll
                for (int d = 0; d < 4; ++d) st.a[q][d] = (int)((uint32_t)st.a[q][d] & keep(ks, d));
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ks = kt * kBK + 32 * fg + 16 * h;
            if (ks < K && K < ks + 16) {
#pragma unroll
                for (int d = 0; d < 4; ++d) st.b[4 * h + d] = (int)((uint32_t)st.b[4 * h + d] & keep(ks, d));
            }
        }
    };

    f32x4 acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = KT > wave ? (KT - wave + NW - 1) / NW : 0;  // steps wave, wave + NW, ...
    Step buf[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u)
        if (u < nsteps) load(wave + NW * u, buf[u]);
    for (int s0 = 0; s0 < nsteps; s0 += KU) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int s = s0 + u;
            if (s < nsteps) {
                Step cur = buf[u];
                const int kt = wave + NW * s;
                if (s + KU < nsteps) load(wave + NW * (s + KU), buf[u]);
                if (kt * kBK + kBK > K && (K & 15)) mask(kt, cur);
                // A through the wave's slot: the previous step's fragment reads of
                // the slot are complete (their results fed that step's MFMAs)
#pragma unroll
                for (int q = 0; q < A_INS; ++q) *(i32x4*)(slot + awr[q]) = cur.a[q];
                i32x8 af[MT];
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    af[i] = cat(*(const i32x4*)(slot + i * 16 * kBK + foff0),
                                *(const i32x4*)(slot + i * 16 * kBK + foff1));
                bf16x8 bb[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) bb[q] = to_bf16x8<FB>(cur.b, q, 1.0f);
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    f32x4 part = MODE == MODE_FAST ? acc[i] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int q = 0; q < 4; ++q) part = mfma_bf16(bb[q], to_bf16x8<FA>(af[i], q, 1.0f), part);
                    if (MODE == MODE_FAST) acc[i] = part;
                    else acc[i] += part;
                }
            }
        }
    }

    // Fixed-order reduction of the NW waves' partial tiles (wave 0's, then waves
    // 1, 2, ... in order), in the LDS that held the A slots.
    __syncthreads();
    f32x4* red = (f32x4*)lds;  // [NW - 1][MT][64]
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < MT; ++i) red[((wave - 1) * MT + i) * 64 + lane] = acc[i];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < NW - 1; ++w)
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i] += red[(w * MT + i) * 64 + lane];

    auto epilogue = [&](auto ot, auto bi) {
        constexpr int OT = decltype(ot)::value;
        constexpr bool BI = decltype(bi)::value != 0;
        float bv[4];
        if constexpr (BI) {
#pragma unroll
            for (int r = 0; r < 4; ++r) bv[r] = n0 + 4 * fg + r < p.N ? load_bias<OT>(p.bias, n0 + 4 * fg + r) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int m = i * 16 + fr;
            const int n = n0 + 4 * fg;
            const int valid = (m < p.M) ? max(0, min(4, p.N - n)) : 0;
            uint32_t out[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = (acc[i][r] + 0.0f) * alpha;
                if constexpr (BI) v += bv[r];
                if constexpr (OT == T_E4M3 || OT == T_E5M2) v *= sr;
                out[r] = convert_t<OT>(v);
            }
            if (valid > 0) store4<OT>(p.d, (int64_t)m * p.ldd + n, out, valid, p.vec_store != 0);
        }
    };
    with_out_type(p.d_type, [&](auto ot) {
        constexpr int OT = decltype(ot)::value;
        if constexpr (OT == T_F32 || OT == T_BF16 || OT == T_F16) {
            if (p.bias) epilogue(ot, IC<1>{});
            else epilogue(ot, IC<0>{});
        } else {
            epilogue(ot, IC<0>{});
        }
    });
}

// ------------------------------------------------------------------ K-split tile kernel
//
// For mid-size M (above the skinny range, up to a few hundred rows at
// N = K = 4096) the workgroup tiles of gemm_tile that keep its waves efficient
// are too few to fill the chip, and small tiles leave one wave per SIMD with
// nothing to hide latency behind. Here a workgroup owns a 16 MT x 16 NT output
// tile and its NW waves split the K steps round-robin (wave w takes steps
// w, w + NW, ...): each wave computes the whole tile for its steps from its own
// LDS slot, so the main loop has no barriers and the waves drift freely. Each
// step's A and B rows are read in contiguous 1 KB pieces (8 rows of 128 bytes
// per instruction) into registers, written to the slot with the XOR swizzle of
// gemm_tile, and read back as fragments; the next step's loads are in flight
// meanwhile. At the end the NW partial tiles are added in a fixed order (wave
// 0's first), each wave reducing and storing its share of the fragments.
template <int MT, int NT, int MODE, int FA, int FB, int NW, int KU>
__global__ void __launch_bounds__(NW * 64) gemm_ksplit(GemmArgs p) {
    static_assert(KU >= 1 && KU <= 4, "steps in flight per wave");
    constexpr int AROWS = 16 * MT, BROWS = 16 * NT;
    constexpr int A_INS = AROWS / 8, B_INS = BROWS / 8, INS = A_INS + B_INS;  // 1 KB loads per step
    constexpr int SLOT = INS * 1024;                                          // A rows, then B rows
    constexpr int NFRAG = MT * NT;
    static_assert(NFRAG % NW == 0, "the fragments split evenly over the waves for the reduction");
    constexpr int FPW = NFRAG / NW;
    constexpr int RED = NW * NFRAG * 1024;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NW * SLOT > RED ? NW * SLOT : RED];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int l, tm, tn;
    tile_of(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, 8, l, tm, tn);
    const int m0 = tm * AROWS, n0 = tn * BROWS;
    const int K = p.K, KT = (K + kBK - 1) / kBK;
    const int fr = lane & 15, fg = lane >> 4;
    const rsrc_t ra = make_rsrc(p.a + (int64_t)m0 * p.lda, operand_extent(min(AROWS, p.M - m0), p.lda, K));
    const rsrc_t rb = make_rsrc(p.b + (int64_t)n0 * p.ldb, operand_extent(min(BROWS, p.N - n0), p.ldb, K));
    // epilogue scales, read now so that their latency hides behind the main loop
    const float alpha = p.sa[0] * p.sb[0];
    const bool fp8_out = p.d_type == T_E4M3 || p.d_type == T_E5M2;
    const float sr = (fp8_out && p.scale_result) ? p.scale_result[0] : 1.0f;

    // Loader: instruction q reads slot rows 8q .. 8q+7 (A rows first); lane l
    // takes row 8q + l/8, chunk c = l%8, and stores it at chunk c ^ swz(row),
    // swz(r) = (r & 7) ^ ((r >> 3) & 1).
    const int ld_row = lane >> 3, ld_chunk = lane & 7;
    uint32_t goff[INS];
    int wr[INS];
#pragma unroll
    for (int q = 0; q < INS; ++q) {
        const int grow = (q < A_INS ? q : q - A_INS) * 8 + ld_row;
        goff[q] = (uint32_t)(grow * (q < A_INS ? p.lda : p.ldb) + ld_chunk * 16);
        wr[q] = (q * 8 + ld_row) * kBK + ((ld_chunk ^ ld_row ^ (q & 1)) << 4);
    }
    const int fsw = (fr & 7) ^ (fr >> 3);
    const int foff0 = fr * kBK + (((2 * fg) ^ fsw) << 4);
    const int foff1 = fr * kBK + (((2 * fg + 1) ^ fsw) << 4);
    uint8_t* const slot = lds + wave * SLOT;

    struct Step {
        i32x4 v[INS];
    };
    // Loads of step kt; chunks starting at or past K read zero (out-of-range
    // offsets return 0); a chunk straddling K is masked after it lands.
    auto load = [&](int kt, Step& st) {
        const uint32_t kb = (uint32_t)(kt * kBK);
        const bool z = kt * kBK + kBK > K && (int)kb + ld_chunk * 16 >= K;
#pragma unroll
        for (int q = 0; q < INS; ++q) {
            uint32_t off = goff[q] + kb;
            if (z) off = kOOB;
            st.v[q] = q < A_INS ? __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0)
                                : __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
        }
    };
    auto mask = [&](int kt, Step& st) {
        const int ks = kt * kBK + ld_chunk * 16;
        if (ks < K && K < ks + 16) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int nb = K - ks - 4 * d;
                const uint32_t m = nb >= 4 ? 0xFFFFFFFFu : (nb <= 0 ? 0u : ((1u << (8 * nb)) - 1u));
#pragma unroll
                for (int q = 0; q < INS; ++q) st.v[q][d] = (int)((uint32_t)st.v[q][d] & m);
            }
        }
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = KT > wave ? (KT - wave + NW - 1) / NW : 0;  // steps wave, wave + NW, ...
    Step buf[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u)
        if (u < nsteps) load(wave + NW * u, buf[u]);
    for (int s0 = 0; s0 < nsteps; s0 += KU)
#pragma unroll
    for (int u = 0; u < KU; ++u) {
        const int s = s0 + u;
        if (s >= nsteps) break;
        const int kt = wave + NW * s;
        if (kt * kBK + kBK > K && (K & 15)) mask(kt, buf[u]);
        // into the slot (the previous step's fragment reads were issued before,
        // and LDS operations of one wave complete in order)
#pragma unroll
        for (int q = 0; q < INS; ++q) *(i32x4*)(slot + wr[q]) = buf[u].v[q];
        if (s + KU < nsteps) load(kt + NW * KU, buf[u]);
        const uint8_t* As = slot;
        const uint8_t* Bs = slot + AROWS * kBK;
        // Fast: one chain into the accumulators. Slow: a fresh fp32 partial per
        // 128-chunk (this step), promoted into the accumulator after.
        constexpr bool chain = MODE == MODE_FAST;
        if constexpr (!chain && NW == 8) {
            // Eight waves (two per SIMD): B fragment by B fragment, each 128-chunk partial finished and
            // promoted before the next (the chunk sums keep their order), so that only MT partials are live
            // next to the A operands converted once for the whole step
            i32x4 ar[2][MT];
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                ar[0][i] = *(const i32x4*)(As + i * 16 * kBK + foff0);
                ar[1][i] = *(const i32x4*)(As + i * 16 * kBK + foff1);
            }
            bf16x8 xa[4][MT];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < MT; ++i) xa[u][i] = to_bf16x8<FA>(ar[u / 2][i], u & 1, 1.0f);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const i32x4 b0 = *(const i32x4*)(Bs + j * 16 * kBK + foff0);
                const i32x4 b1 = *(const i32x4*)(Bs + j * 16 * kBK + foff1);
                f32x4 pt[MT];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const bf16x8 xb = to_bf16x8<FB>(u < 2 ? b0 : b1, u & 1, 1.0f);
#pragma unroll
                    for (int i = 0; i < MT; ++i) pt[i] = mfma_bf16(xb, xa[u][i], u == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : pt[i]);
                }
#pragma unroll
                for (int i = 0; i < MT; ++i) acc[i][j] += pt[i];
            }
            continue;
        }

        f32x4 part[chain ? 1 : MT][chain ? 1 : NT];
        if constexpr (!chain) {
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) part[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // two 16-byte halves of the lane's 32 bytes: sub-steps 0-1, then 2-3
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int fo = h ? foff1 : foff0;
            i32x4 ar[MT], br[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i) ar[i] = *(const i32x4*)(As + i * 16 * kBK + fo);
#pragma unroll
            for (int j = 0; j < NT; ++j) br[j] = *(const i32x4*)(Bs + j * 16 * kBK + fo);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                bf16x8 ab[MT];
#pragma unroll
                for (int i = 0; i < MT; ++i) ab[i] = to_bf16x8<FA>(ar[i], q, 1.0f);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const bf16x8 bb = to_bf16x8<FB>(br[j], q, 1.0f);
#pragma unroll
                    for (int i = 0; i < MT; ++i) {
                        if constexpr (chain) acc[i][j] = mfma_bf16(bb, ab[i], acc[i][j]);
                        else part[i][j] = mfma_bf16(bb, ab[i], part[i][j]);
                    }
                }
            }
        }
        if constexpr (!chain) {
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[i][j] += part[i][j];
        }
    }

    // Fixed-order reduction: every wave's partial tile goes to LDS (over the
    // slots, once all waves are done with them); wave w then adds fragments
    // w FPW .. w FPW + FPW - 1 over the waves in order 0, 1, ... and stores them.
    __syncthreads();
    f32x4* red = (f32x4*)lds;  // [NW][NFRAG][64]
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) red[(wave * NFRAG + i * NT + j) * 64 + lane] = acc[i][j];
    __syncthreads();
    auto epilogue = [&](auto ot, auto bi) {
        constexpr int OT = decltype(ot)::value;
        constexpr bool BI = decltype(bi)::value != 0;
#pragma unroll
        for (int u = 0; u < FPW; ++u) {
            const int f = wave * FPW + u;
            f32x4 v = red[f * 64 + lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) v += red[(w * NFRAG + f) * 64 + lane];
            const int i = f / NT, j = f % NT;
            const int m = m0 + i * 16 + fr;
            const int n = n0 + j * 16 + 4 * fg;
            const int valid = (m < p.M) ? max(0, min(4, p.N - n)) : 0;
            uint32_t out[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = (v[r] + 0.0f) * alpha;
                if constexpr (BI) x += n + r < p.N ? load_bias<OT>(p.bias, n + r) : 0.0f;
                if constexpr (OT == T_E4M3 || OT == T_E5M2) x *= sr;
                out[r] = convert_t<OT>(x);
            }
            if (valid > 0) store4<OT>(p.d, (int64_t)m * p.ldd + n, out, valid, p.vec_store != 0);
        }
    };
    with_out_type(p.d_type, [&](auto ot) {
        constexpr int OT = decltype(ot)::value;
        if constexpr (OT == T_F32 || OT == T_BF16 || OT == T_F16) {
            if (p.bias) epilogue(ot, IC<1>{});
            else epilogue(ot, IC<0>{});
        } else {
            epilogue(ot, IC<0>{});
        }
    });
}

}  // namespace mmfp8
