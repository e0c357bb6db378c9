/*
 * oracle.cpp -- plain, slow CPU reference for the FP8 scaled GEMM and for the
 * batched block-scaled GEMM + global amax.
 *
 * TEST INFRASTRUCTURE. This is the checker, not the product. Only the test
 * suite, the package's smoke check and the benchmark's CPU-baseline leg load
 * it. It shares no source, header, table or helper with the GPU library, and
 * the GPU library never calls it.
 *
 * What it computes, and where each step comes from:
 *
 *  - Operands are FP8 codes, decoded by their bit fields (OCP 8-bit floating
 *    point formats E4M3FN and E5M2, the float8_e4m3fn / float8_e5m2 dtypes of
 *    "mmaemu API reference (v0.1)", scaled_mm argument table, and of
 *    "cuDNN frontend: GEMM + Amax (SM100)", Parameters), or, for the
 *    block-scaled GEMM + amax, E2M1 pairs (that page's float4_e2m1fn_x2).
 *  - scaled GEMM: d[m,n] = (a * s_a) @ (b * s_b)^T with a [M,K] and b [N,K]
 *    ("TileOPs: Linear Algebra Operators", tileops.gemm.GemmFP8FwdOp). With
 *    per-tensor scales the unscaled sum is multiplied by both scales
 *    (mmaemu API reference, scaled_mm argument table); with 1x128 / 128x128
 *    block scales each operand element is multiplied by the scale of its block
 *    before the product (GemmFP8FwdOp, scale shapes).
 *  - FP8 outputs are additionally multiplied by scale_result (mmaemu API
 *    reference, scaled_mm argument table; None means 1).
 *  - grouped GEMM ("TileOPs: Linear Algebra Operators",
 *    tileops.gemm.GroupedGemmFwdOp, NT layout): group g owns a run of rows of
 *    a and multiplies them by its own b; with FP8 operands each scaled by one
 *    factor (tileops.gemm.BmmFP8FwdOp's per-tensor scales). Each group is the
 *    scaled GEMM above on its rows.
 *  - block-scaled GEMM + amax: C[m,n,l] = sum_k A^[m,k,l] B^[n,k,l] with
 *    A^ = A * SFA[l, m, k / sf_vec_size]; Amax = max over m,n,l of |C|
 *    ("cuDNN frontend: GEMM + Amax (SM100)", Equations).
 *  - The page-native scale-factor tensors of that operator ("cuDNN frontend:
 *    GEMM + Amax (SM100)", Shapes, Parameters and the JAX contract) are
 *    unpacked into plain [L][MN][groups] factors first (orc_sf_atom_unpack);
 *    the GEMM itself is then the one above.
 *
 * Arithmetic:
 *  - accum = ORC_ACC_EXACT: the sum is taken in float64 from +0 in increasing
 *    k. Every E4M3 x E4M3 product is a multiple of 2^-18 below 2^18, so for
 *    K < 2^17 every partial sum is exact and the result is the exact sum. With
 *    E5M2 operands the float64 error is at most K * 2^-53 * sum|t|.
 *  - accum = ORC_ACC_F32_CHUNKS: the "slow" accumulation of the scaled_mm
 *    argument table (128-element K chunks promoted into an fp32 accumulator),
 *    written out in fp32: chunks [128c, 128c+128) aligned at k = 0 (the last one
 *    partial); each chunk's exact sum is rounded to fp32; the fp32 accumulator
 *    starts at +0 and adds the chunks in increasing c with fp32 rounding. The
 *    per-tensor result is then fp32(acc * fp32(s_a * s_b)). For block scales
 *    the chunk sum is taken over the unscaled codes and folded as
 *    acc = fp32(acc + fp32(part * fp32(sa * sb))). The pages do not state the
 *    order of these roundings; this is one plain reading of them.
 *  - The output is rounded ONCE from that value to the output type with
 *    round-to-nearest-even. FP8 outputs saturate (|v| above the largest finite
 *    value, and +-Inf, become +-max; NaN stays NaN); bf16 / f16 / f32 overflow
 *    to +-Inf as IEEE rounding does. NaN outputs take the canonical encodings
 *    of "mmaemu testing", Bitwise policy: f32 0x7FFFFFFF, bf16 / f16 0x7FFF,
 *    FP8 0x7F.
 *  - Non-finite inputs follow IEEE float64 arithmetic (NaN codes give NaN,
 *    Inf * 0 gives NaN, +Inf + -Inf gives NaN).
 *  - Amax is the maximum of |v| over the computed outputs (v before the output
 *    cast), returned as fp32; NaN if any v is NaN; the index is the smallest
 *    linear index l*M*N + m*N + n among the maxima. +0 and index -1 when there
 *    are no outputs.
 *
 * The oracle refuses to run (returns ORC_ERR_FPENV) when the host flushes
 * subnormals to zero (FTZ or DAZ set), which would silently change results.
 */
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>
#include <algorithm>
#include <xmmintrin.h>

extern "C" {

/* Format numbers used by this file's C interface (its own, documented in
 * oracle.py; nothing here is shared with the GPU library). */
enum { ORC_E4M3FN = 0, ORC_E5M2 = 1, ORC_F32 = 2, ORC_BF16 = 3, ORC_F16 = 4, ORC_E2M1 = 5 };
enum { ORC_SCALE_TENSOR = 0, ORC_SCALE_1x128 = 1, ORC_SCALE_128x128 = 2 };
enum { ORC_ACC_EXACT = 0, ORC_ACC_F32_CHUNKS = 1 };
enum { ORC_OK = 0, ORC_ERR_ARG = 1, ORC_ERR_FPENV = 2 };
enum { ORC_SF_E8M0 = 0, ORC_SF_E4M3FN = 1 };

}  // extern "C"

namespace {

/* ---------------------------------------------------------------- decode */

/* E4M3FN: sign s, 4 exponent bits (bias 7), 3 mantissa bits. No infinities;
 * exponent 15 with mantissa 7 is NaN (0x7F, 0xFF). Largest finite 448. */
double decode_e4m3fn(uint8_t c) {
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return std::nan("");
    const double mag = (e == 0) ? std::ldexp((double)m, -9)           /* m/8 * 2^(1-7) */
                                : std::ldexp((double)(8 + m), e - 10); /* (1+m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

/* E5M2: sign s, 5 exponent bits (bias 15), 2 mantissa bits, IEEE-like:
 * exponent 31 is Inf (mantissa 0) or NaN. Largest finite 57344. */
double decode_e5m2(uint8_t c) {
    const int s = c >> 7, e = (c >> 2) & 31, m = c & 3;
    if (e == 31) {
        if (m != 0) return std::nan("");
        return s ? -INFINITY : INFINITY;
    }
    const double mag = (e == 0) ? std::ldexp((double)m, -16)          /* m/4 * 2^(1-15) */
                                : std::ldexp((double)(4 + m), e - 17); /* (1+m/4) * 2^(e-15) */
    return s ? -mag : mag;
}

double decode(uint8_t c, int fmt) { return fmt == ORC_E4M3FN ? decode_e4m3fn(c) : decode_e5m2(c); }

/* E2M1 (FP4, the float4_e2m1fn_x2 operand type of "cuDNN frontend: GEMM +
 * Amax (SM100)", Parameters): sign bit 3, 2 exponent bits (bias 1), 1 mantissa
 * bit, no infinities or NaNs; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double decode_e2m1(uint8_t c) {
    const int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    const double mag = (e == 0) ? std::ldexp((double)m, -1)          /* m/2 * 2^(1-1) */
                                : std::ldexp((double)(2 + m), e - 2); /* (1+m/2) * 2^(e-1) */
    return s ? -mag : mag;
}

/* Element k of an operand row: FP8 formats take one byte per element; E2M1
 * packs two per byte ("float4_e2m1fn_x2": the row holds K/2 bytes). The page
 * does not say which nibble comes first; the reading here is element 2i in
 * the low nibble of byte i and 2i+1 in the high nibble. (A sum over k pairs
 * every element of a with the element of b at the same k and the two
 * elements of a byte always share a scale group, so C does not depend on
 * this order.) */
double element(const uint8_t* row, int64_t k, int fmt) {
    if (fmt == ORC_E2M1) return decode_e2m1((uint8_t)((row[k >> 1] >> (4 * (k & 1))) & 15));
    return decode(row[k], fmt);
}

/* E8M0 (the float8_e8m0fnu scale-factor type of "cuDNN frontend: GEMM + Amax
 * (SM100)", Parameters): an unsigned, biased exponent only, value 2^(e - 127);
 * the code 0xFF is NaN; there is no zero and no infinity. */
double decode_e8m0(uint8_t e) {
    if (e == 0xFF) return std::nan("");
    return std::ldexp(1.0, (int)e - 127);
}

/* ---------------------------------------------------------------- rounding */

/* A binary floating-point format: `mant` stored mantissa bits, exponent bias,
 * smallest normal exponent emin = 1 - bias, largest finite value, whether it
 * has infinities, and whether overflow saturates (the FP8 outputs). */
struct Format {
    int mant;
    int bias;
    int bits;          /* storage width */
    double maxv;       /* largest finite magnitude */
    bool has_inf;
    bool saturate;
    uint32_t nan_bits; /* canonical NaN */
};

Format format_of(int t) {
    switch (t) {
        case ORC_E4M3FN: return {3, 7, 8, 448.0, false, true, 0x7Fu};
        case ORC_E5M2:   return {2, 15, 8, 57344.0, true, true, 0x7Fu};
        case ORC_F16:    return {10, 15, 16, 65504.0, true, false, 0x7FFFu};
        /* E2M1 output: saturating like the FP8 outputs; the format has no NaN code, so NaN takes the largest
         * value's code 0x7 (a reading: the page gives FP4 C a shape but no conversion rule) */
        case ORC_E2M1:   return {1, 1, 4, 6.0, false, true, 0x7u};
        case ORC_BF16:   return {7, 127, 16, std::ldexp(255.0, 120), true, false, 0x7FFFu};
        default:         return {23, 127, 32, std::ldexp(16777215.0, 104), true, false, 0x7FFFFFFFu};
    }
}

/* Round x to the nearest value of format f, ties to even, with the format's
 * overflow rule. Works on magnitudes: for the binade [2^E, 2^(E+1)) the
 * representable values are multiples of q = 2^(E - mant); below the smallest
 * normal binade q stays 2^(emin - mant) (subnormals). x/q and n*q are exact in
 * float64 for every format here, so nearbyint (round-half-even in the default
 * rounding mode) does the only rounding. */
double round_to(double x, const Format& f) {
    if (std::isnan(x)) return x;
    if (std::isinf(x)) {
        if (f.saturate) return std::copysign(f.maxv, x);
        return f.has_inf ? x : std::nan("");
    }
    if (x == 0.0) return x;
    const double ax = std::fabs(x);
    int e2;
    std::frexp(ax, &e2);                 /* ax = fr * 2^e2, fr in [0.5, 1) */
    int E = e2 - 1;                      /* floor(log2(ax)) */
    const int emin = 1 - f.bias;
    if (E < emin) E = emin;
    const double q = std::ldexp(1.0, E - f.mant);
    double r = std::nearbyint(ax / q) * q;
    if (r > f.maxv) {
        if (f.saturate) r = f.maxv;
        else if (f.has_inf) r = INFINITY;
        else return std::nan("");
    }
    return std::copysign(r, x);
}

/* Encode a value that is already representable in f (the output of round_to). */
uint32_t encode(double r, const Format& f) {
    if (std::isnan(r)) return f.nan_bits;
    const uint32_t sign = std::signbit(r) ? (1u << (f.bits - 1)) : 0u;
    const int ebits = f.bits - 1 - f.mant;
    if (std::isinf(r)) return sign | (((1u << ebits) - 1u) << f.mant);
    const double ar = std::fabs(r);
    if (ar == 0.0) return sign;
    int e2;
    std::frexp(ar, &e2);
    const int E = e2 - 1;
    const int emin = 1 - f.bias;
    if (E < emin) { /* subnormal: exponent field 0, mantissa = ar / 2^(emin - mant) */
        const uint32_t m = (uint32_t)std::ldexp(ar, f.mant - emin);
        return sign | m;
    }
    const uint32_t m = (uint32_t)(std::ldexp(ar, f.mant - E) - std::ldexp(1.0, f.mant));
    const uint32_t ef = (uint32_t)(E + f.bias);
    return sign | (ef << f.mant) | m;
}

void store_bits(void* out, int64_t i, uint32_t bits, int width) {
    if (width <= 8) ((uint8_t*)out)[i] = (uint8_t)bits; /* E2M1 codes here are one per byte */
    else if (width == 16) ((uint16_t*)out)[i] = (uint16_t)bits;
    else ((uint32_t*)out)[i] = bits;
}

float to_f32(double x) { return (float)round_to(x, format_of(ORC_F32)); }

bool fpenv_flushes() {
    const unsigned csr = _mm_getcsr();
    return (csr & (1u << 15)) || (csr & (1u << 6)); /* FTZ, DAZ */
}

/* Run body(i) for i in [0, n) on `threads` std::threads, static blocks. */
template <class F>
void parallel_rows(int64_t n, int threads, F body) {
    if (threads < 1) threads = 1;
    if (threads > n) threads = (int)std::max<int64_t>(n, 1);
    if (threads == 1) {
        for (int64_t i = 0; i < n; ++i) body(i);
        return;
    }
    std::vector<std::thread> pool;
    for (int t = 0; t < threads; ++t) {
        pool.emplace_back([=]() {
            const int64_t lo = n * t / threads, hi = n * (t + 1) / threads;
            for (int64_t i = lo; i < hi; ++i) body(i);
        });
    }
    for (auto& th : pool) th.join();
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" {

/* Decode n FP8 codes of format fmt to float64. */
int orc_decode_fp8(const uint8_t* codes, int64_t n, int fmt, double* out) {
    if (fmt != ORC_E4M3FN && fmt != ORC_E5M2) return ORC_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = decode(codes[i], fmt);
    return ORC_OK;
}

/* Round n float64 values to dtype (RNE, the output rules above) and store the
 * bit patterns (uint8 / uint16 / uint32 by width). */
/* Decode n E2M1 codes (one per byte, values 0..15) to float64. */
int orc_decode_fp4(const uint8_t* codes, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) {
        if (codes[i] > 15) return ORC_ERR_ARG;
        out[i] = decode_e2m1(codes[i]);
    }
    return ORC_OK;
}

int orc_round(const double* x, int64_t n, int dtype, void* out_bits) {
    if (dtype < ORC_E4M3FN || dtype > ORC_E2M1) return ORC_ERR_ARG; /* E2M1: one code per byte */
    const Format f = format_of(dtype);
    for (int64_t i = 0; i < n; ++i) store_bits(out_bits, i, encode(round_to(x[i], f), f), f.bits);
    return ORC_OK;
}

/*
 * The scaled GEMM for the rows listed in `rows` (all M rows when rows is NULL).
 * Output arrays are [n_rows, N] row-major. value: the result before the output
 * cast, after every scale and the bias. sum_abs (may be NULL): sum over k of
 * |term|, each term with every scale applied. d_bits: value rounded to d_type.
 * bias (may be NULL): [N] values added to the scaled sum (TileOPs
 * GemmFP8FwdOp: "apply the scales, and add the bias"); only for non-FP8
 * outputs. In the emulated-fp32 mode the addition is an fp32 addition.
 */
int orc_scaled_gemm(int64_t M, int64_t N, int64_t K,
                    const uint8_t* a, int a_fmt, int64_t lda,
                    const uint8_t* b, int b_fmt, int64_t ldb,
                    const float* scale_a, int sa_mode,
                    const float* scale_b, int sb_mode,
                    const float* scale_result, const double* bias, int d_type, int accum,
                    const int64_t* rows, int64_t n_rows,
                    double* value, double* sum_abs, void* d_bits, int threads) {
    if (fpenv_flushes()) return ORC_ERR_FPENV;
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K) return ORC_ERR_ARG;
    if (d_type < ORC_E4M3FN || d_type > ORC_F16) return ORC_ERR_ARG;
    if (bias && (d_type == ORC_E4M3FN || d_type == ORC_E5M2)) return ORC_ERR_ARG;
    const bool block = sa_mode != ORC_SCALE_TENSOR;
    if (block != (sb_mode != ORC_SCALE_TENSOR) || sa_mode == ORC_SCALE_128x128) return ORC_ERR_ARG;
    if (!rows) n_rows = M;
    const int64_t KB = ceil_div(K, 128);
    const bool fp8_out = d_type == ORC_E4M3FN || d_type == ORC_E5M2;
    const double sr = (fp8_out && scale_result) ? (double)scale_result[0] : 1.0;
    const Format out_f = format_of(d_type);

    for (int64_t i = 0; i < n_rows; ++i)
        if (rows && (rows[i] < 0 || rows[i] >= M)) return ORC_ERR_ARG;

    /* Decode once: the decoded operands as float64 (only the requested rows of a). */
    std::vector<double> A((size_t)n_rows * K), B((size_t)N * K);
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t m = rows ? rows[i] : i;
        for (int64_t k = 0; k < K; ++k) A[(size_t)i * K + k] = decode(a[m * lda + k], a_fmt);
    }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) B[(size_t)n * K + k] = decode(b[n * ldb + k], b_fmt);

    auto sa_at = [&](int64_t m, int64_t kb) -> double { return scale_a[m * KB + kb]; };
    auto sb_at = [&](int64_t n, int64_t kb) -> double {
        return sb_mode == ORC_SCALE_1x128 ? scale_b[n * KB + kb] : scale_b[(n / 128) * KB + kb];
    };

    parallel_rows(n_rows, threads, [&](int64_t i) {
        const int64_t m = rows ? rows[i] : i;
        const double* Am = A.data() + (size_t)i * K;
        for (int64_t n = 0; n < N; ++n) {
            const double* Bn = B.data() + (size_t)n * K;
            double v, sabs = 0.0;
            if (accum == ORC_ACC_EXACT) {
                if (!block) {
                    double S = +0.0, T = 0.0;
                    for (int64_t k = 0; k < K; ++k) {
                        const double t = Am[k] * Bn[k];
                        S += t;
                        T += std::fabs(t);
                    }
                    const double s = (double)scale_a[0] * (double)scale_b[0];
                    v = S * (double)scale_a[0] * (double)scale_b[0];
                    sabs = T * std::fabs(s);
                } else {
                    /* Dequantize each element by its block scale, then the plain sum. */
                    double S = +0.0, T = 0.0;
                    for (int64_t k = 0; k < K; ++k) {
                        const double ah = Am[k] * sa_at(m, k / 128);
                        const double bh = Bn[k] * sb_at(n, k / 128);
                        const double t = ah * bh;
                        S += t;
                        T += std::fabs(t);
                    }
                    v = S;
                    sabs = T;
                }
            } else { /* ORC_ACC_F32_CHUNKS */
                float acc = +0.0f;
                double T = 0.0;
                for (int64_t kb = 0; kb < KB; ++kb) {
                    double P = +0.0;
                    const int64_t k1 = std::min<int64_t>(K, kb * 128 + 128);
                    for (int64_t k = kb * 128; k < k1; ++k) {
                        const double t = Am[k] * Bn[k];
                        P += t;
                        T += std::fabs(t) * (block ? std::fabs(sa_at(m, kb) * sb_at(n, kb)) : 1.0);
                    }
                    const float part = to_f32(P);
                    if (!block) {
                        acc = to_f32((double)acc + (double)part);
                    } else {
                        const float s = to_f32((double)(float)sa_at(m, kb) * (double)(float)sb_at(n, kb));
                        acc = to_f32((double)acc + (double)to_f32((double)part * (double)s));
                    }
                }
                if (!block) {
                    const float alpha = to_f32((double)scale_a[0] * (double)scale_b[0]);
                    v = (double)to_f32((double)acc * (double)alpha);
                    sabs = T * std::fabs((double)scale_a[0] * (double)scale_b[0]);
                } else {
                    v = (double)acc;
                    sabs = T;
                }
            }
            v *= sr;
            sabs *= std::fabs(sr);
            if (bias) v = accum == ORC_ACC_EXACT ? v + bias[n] : (double)to_f32(v + bias[n]);
            const size_t o = (size_t)i * N + n;
            if (value) value[o] = v;
            if (sum_abs) sum_abs[o] = sabs;
            if (d_bits) store_bits(d_bits, (int64_t)o, encode(round_to(v, out_f), out_f), out_f.bits);
        }
    });
    return ORC_OK;
}

/*
 * Grouped GEMM: group g owns rows offsets[g] .. offsets[g] + sizes[g] - 1 of
 * a [batch_sum][lda] and multiplies them by its operand b + g * stride_b
 * ([N][ldb]), per-tensor scales as orc_scaled_gemm. value / sum_abs / d_bits
 * are [batch_sum][N]; each group writes its own rows. The metadata must be
 * what the page asks for: sizes >= 0 adding up to batch_sum, offsets their
 * exclusive prefix sum (ORC_ERR_ARG otherwise).
 */
int orc_grouped_gemm(int64_t batch_sum, int64_t N, int64_t K, int64_t G,
                     const uint8_t* a, int a_fmt, int64_t lda,
                     const uint8_t* b, int b_fmt, int64_t ldb, int64_t stride_b,
                     const int32_t* sizes, const int32_t* offsets,
                     const float* scale_a, const float* scale_b, const float* scale_result,
                     int d_type, int accum,
                     double* value, double* sum_abs, void* d_bits, int threads) {
    if (batch_sum < 0 || N < 0 || K < 0 || G < 0 || stride_b < 0) return ORC_ERR_ARG;
    if (d_type < ORC_E4M3FN || d_type > ORC_F16) return ORC_ERR_ARG;
    int64_t next = 0;
    for (int64_t g = 0; g < G; ++g) {
        if (sizes[g] < 0 || offsets[g] != next) return ORC_ERR_ARG;
        next += sizes[g];
    }
    if (next != batch_sum) return ORC_ERR_ARG;
    const int width = format_of(d_type).bits / 8;
    for (int64_t g = 0; g < G; ++g) {
        if (sizes[g] == 0) continue;
        const int64_t r0 = offsets[g];
        const int rc = orc_scaled_gemm(sizes[g], N, K, a + r0 * lda, a_fmt, lda, b + g * stride_b, b_fmt, ldb,
                                       scale_a, ORC_SCALE_TENSOR, scale_b, ORC_SCALE_TENSOR, scale_result, nullptr,
                                       d_type, accum, nullptr, sizes[g], value ? value + r0 * N : nullptr,
                                       sum_abs ? sum_abs + r0 * N : nullptr,
                                       d_bits ? (uint8_t*)d_bits + r0 * N * width : nullptr, threads);
        if (rc != ORC_OK) return rc;
    }
    return ORC_OK;
}

/*
 * The batched block-scaled GEMM + amax. a[l][m][k], b[l][n][k] FP8 codes of one
 * format (row pitch K bytes), or E2M1 pairs (ab_fmt ORC_E2M1, K even, row pitch
 * K/2 bytes); sfa[l][m][ceil(K/sf)], sfb[l][n][ceil(K/sf)] fp32 scale
 * factors; outputs for the listed rows m (all M when NULL) of every batch item:
 * value / sum_abs / c_bits are [L, n_rows, N]. amax and amax_index cover the
 * computed outputs (linear index l*M*N + m*N + n).
 */
int orc_blockscaled_gemm_amax(int64_t M, int64_t N, int64_t K, int64_t L,
                              const uint8_t* a, const uint8_t* b, int ab_fmt,
                              const float* sfa, const float* sfb, int sf_vec,
                              int c_type, const int64_t* rows, int64_t n_rows,
                              double* value, double* sum_abs, void* c_bits,
                              float* amax, int64_t* amax_index, int threads) {
    if (fpenv_flushes()) return ORC_ERR_FPENV;
    if (M < 0 || N < 0 || K < 0 || L < 0 || sf_vec <= 0) return ORC_ERR_ARG;
    if (c_type < ORC_E4M3FN || c_type > ORC_E2M1) return ORC_ERR_ARG;
    if (ab_fmt != ORC_E4M3FN && ab_fmt != ORC_E5M2 && ab_fmt != ORC_E2M1) return ORC_ERR_ARG;
    /* E2M1 C is packed like the FP4 operands: rows of ceil(N/2) bytes, element 2i in the low nibble; an odd
     * N leaves the last byte's high nibble 0 */
    const int64_t c_row_bytes = (N + 1) / 2;
    if (ab_fmt == ORC_E2M1 && (K & 1)) return ORC_ERR_ARG;
    const int64_t pitch = ab_fmt == ORC_E2M1 ? K / 2 : K; /* bytes per operand row */
    if (!rows) n_rows = M;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows && (rows[i] < 0 || rows[i] >= M)) return ORC_ERR_ARG;
    const int64_t KS = ceil_div(K, sf_vec);
    const Format out_f = format_of(c_type);

    std::vector<double> vals((size_t)L * n_rows * N);
    for (int64_t l = 0; l < L; ++l) {
        /* Dequantized operands of this batch item: A^ = A * SFA, B^ = B * SFB. */
        std::vector<double> Ah((size_t)n_rows * K), Bh((size_t)N * K);
        for (int64_t i = 0; i < n_rows; ++i) {
            const int64_t m = rows ? rows[i] : i;
            for (int64_t k = 0; k < K; ++k)
                Ah[(size_t)i * K + k] = element(&a[(l * M + m) * pitch], k, ab_fmt) *
                                        (double)sfa[(l * M + m) * KS + k / sf_vec];
        }
        for (int64_t n = 0; n < N; ++n)
            for (int64_t k = 0; k < K; ++k)
                Bh[(size_t)n * K + k] = element(&b[(l * N + n) * pitch], k, ab_fmt) *
                                        (double)sfb[(l * N + n) * KS + k / sf_vec];
        parallel_rows(n_rows, threads, [&](int64_t i) {
            const double* Am = Ah.data() + (size_t)i * K;
            for (int64_t n = 0; n < N; ++n) {
                const double* Bn = Bh.data() + (size_t)n * K;
                double S = +0.0, T = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const double t = Am[k] * Bn[k];
                    S += t;
                    T += std::fabs(t);
                }
                const size_t o = ((size_t)l * n_rows + i) * N + n;
                vals[o] = S;
                if (value) value[o] = S;
                if (sum_abs) sum_abs[o] = T;
                if (c_bits && c_type == ORC_E2M1) {
                    uint8_t* cb = (uint8_t*)c_bits + ((size_t)l * n_rows + i) * c_row_bytes + n / 2;
                    const uint8_t code = (uint8_t)encode(round_to(S, out_f), out_f);
                    *cb = (n & 1) ? (uint8_t)((*cb & 0x0F) | (code << 4)) : code;
                } else if (c_bits) {
                    store_bits(c_bits, (int64_t)o, encode(round_to(S, out_f), out_f), out_f.bits);
                }
            }
        });
    }

    /* Amax over the computed outputs, in increasing linear index. */
    double best = 0.0;
    int64_t best_idx = -1;
    bool seen_nan = false;
    for (int64_t l = 0; l < L; ++l)
        for (int64_t i = 0; i < n_rows; ++i) {
            const int64_t m = rows ? rows[i] : i;
            for (int64_t n = 0; n < N; ++n) {
                const double v = vals[((size_t)l * n_rows + i) * N + n];
                const int64_t idx = l * M * N + m * N + n;
                if (std::isnan(v)) { /* NaN beats every number; the smallest NaN index wins */
                    if (!seen_nan || idx < best_idx) best_idx = idx;
                    seen_nan = true;
                    continue;
                }
                if (seen_nan) continue;
                const double av = std::fabs(v);
                if (best_idx < 0 || av > best || (av == best && idx < best_idx)) {
                    best = av;
                    best_idx = idx;
                }
            }
        }
    if (amax) *amax = seen_nan ? std::nanf("") : to_f32(best);
    if (amax_index) *amax_index = best_idx;
    return ORC_OK;
}

/*
 * Page-native scale factors -> plain factors.
 *
 * "cuDNN frontend: GEMM + Amax (SM100)" gives SFA / SFB the logical shape
 * (32, 4, ceil(MN/128), 4, ceil(K/(4 sf)), L) and says (JAX contract) that this
 * is a view of the C-contiguous storage (L, ceil(MN/128), ceil(K/(4 sf)), 32,
 * 4, 4) permuted by (3, 4, 1, 5, 2, 0): logical coordinate (i0, i1, i2, j0, j1,
 * l) is storage element [l][i2][j1][i0][i1][j0]. The page gives the shapes
 * only; the reading taken here (parity unpinned beyond the permutation) is
 * that the two M-side atom modes enumerate the rows of a 128-row block
 * first-mode-fastest, row mn = i0 + 32 i1 + 128 i2, and the two K-side modes
 * the scale groups likewise, g = j0 + 4 j1.
 *
 * sf: the storage bytes; sf_type ORC_SF_E8M0 (int8 tensors are read as E8M0,
 * as the page says) or ORC_SF_E4M3FN. Writes out[l][mn][g] for mn < MN and
 * g < ceil(K/sf_vec) as fp32 (every E8M0 and E4M3 value is an fp32 value);
 * storage elements past MN or past the last group are padding and are not
 * read.
 */
int orc_sf_atom_unpack(const uint8_t* sf, int sf_type, int64_t MN, int64_t K, int64_t L, int sf_vec,
                       float* out) {
    if (MN < 0 || K < 0 || L < 0 || sf_vec <= 0) return ORC_ERR_ARG;
    if (sf_type != ORC_SF_E8M0 && sf_type != ORC_SF_E4M3FN) return ORC_ERR_ARG;
    const int64_t G = ceil_div(K, sf_vec);       /* scale groups along K */
    const int64_t MB = ceil_div(MN, 128);        /* 128-row blocks */
    const int64_t KB = ceil_div(K, 4 * sf_vec);  /* 4-group blocks */
    for (int64_t l = 0; l < L; ++l)
        for (int64_t i2 = 0; i2 < MB; ++i2)
            for (int64_t j1 = 0; j1 < KB; ++j1)
                for (int64_t i0 = 0; i0 < 32; ++i0)
                    for (int64_t i1 = 0; i1 < 4; ++i1)
                        for (int64_t j0 = 0; j0 < 4; ++j0) {
                            const int64_t storage = ((((l * MB + i2) * KB + j1) * 32 + i0) * 4 + i1) * 4 + j0;
                            const int64_t mn = i0 + 32 * i1 + 128 * i2;
                            const int64_t g = j0 + 4 * j1;
                            if (mn >= MN || g >= G) continue; /* padding */
                            const uint8_t c = sf[storage];
                            const double v = sf_type == ORC_SF_E8M0 ? decode_e8m0(c) : decode_e4m3fn(c);
                            out[(l * MN + mn) * G + g] = (float)v;
                        }
    return ORC_OK;
}

}  // extern "C"
