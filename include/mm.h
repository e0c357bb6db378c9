/*
 * mm.h -- C ABI of libmmfp8.so: FP8 scaled GEMM and batched block-scaled
 * GEMM + global amax on AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 *  - All tensor arguments are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or keeps them.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is
 *    enqueued on it and the call returns without waiting for the GPU, so the
 *    calls can be captured into a HIP graph (the library records no memset
 *    nodes: outputs it must clear are cleared by its own kernels).
 *  - Arguments are validated completely before any HIP call. On a status
 *    other than MM_OK and MM_ERR_DEVICE nothing has been enqueued or written.
 *    MM_ERR_DEVICE means that a HIP call failed while the call enqueued its
 *    work; a call may enqueue several kernels (operand packing, or two tile
 *    shapes over different columns), and those enqueued before the failure
 *    may still run. mm_last_error() describes the problem. No C++ exception
 *    crosses the ABI.
 *  - The library uses the calling thread's current HIP device.
 *  - The kernels never fault whatever the byte values of the operands are:
 *    NaN and Inf codes, padding bytes and partial tiles are all handled.
 *  - Integer arguments are int64_t; enumerations are passed as int.
 */
#ifndef MMFP8_MM_H
#define MMFP8_MM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. The error classes of the "mmaemu API reference (v0.1)",
 * Errors and warnings table map onto them: a call the reference platform
 * rejects (ReferenceRejectsError / ValueError) -> MM_ERR_INVALID_ARGUMENT;
 * a feature not provided (UnsupportedFeatureError) -> MM_ERR_UNSUPPORTED. */
typedef enum mm_status {
    MM_OK = 0,
    MM_ERR_INVALID_ARGUMENT = 1, /* malformed call: negative size, bad enum, null pointer, ld < K ... */
    MM_ERR_UNSUPPORTED = 2,      /* well-formed but not provided (scale pairing, sf_vec_size, FP8 C ...) */
    MM_ERR_MISALIGNED = 3,       /* pointer or row pitch alignment violated */
    MM_ERR_DEVICE = 4            /* the HIP runtime reported an error while enqueueing */
} mm_status;

/* Element types. FP8 codes follow the OCP 8-bit formats E4M3FN (largest
 * finite 448, no infinities, NaN = 0x7F / 0xFF) and E5M2 (largest finite
 * 57344, IEEE-like infinities and NaNs): the float8_e4m3fn / float8_e5m2
 * dtypes of the "mmaemu API reference (v0.1)", scaled_mm argument table.
 * MM_F4_E2M1 is FP4 (sign, 2 exponent bits with bias 1, 1 mantissa bit:
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no Inf or NaN) packed two per byte,
 * the float4_e2m1fn_x2 operands of "cuDNN frontend: GEMM + Amax (SM100)";
 * only mm_blockscaled_gemm_amax_atom takes it, as operands. */
typedef enum mm_dtype {
    MM_F8_E4M3FN = 0,
    MM_F8_E5M2 = 1,
    MM_F32 = 2,
    MM_BF16 = 3,
    MM_F16 = 4,
    MM_F4_E2M1 = 5
} mm_dtype;

/* Scale granularities ("TileOPs: Linear Algebra Operators",
 * tileops.gemm.GemmFP8FwdOp): one fp32 per tensor, one per 1x128 block along
 * K, or one per 128x128 block. */
typedef enum mm_scale_mode {
    MM_SCALE_TENSOR = 0,  /* [1]                                 */
    MM_SCALE_1x128 = 1,   /* [rows, ceil(K/128)], row-major      */
    MM_SCALE_128x128 = 2  /* [ceil(rows/128), ceil(K/128)]       */
} mm_scale_mode;

/* Element types of page-native scale-factor tensors ("cuDNN frontend: GEMM +
 * Amax (SM100)", Parameters, SFA / SFB dtypes). E8M0 is an unsigned biased
 * exponent, value 2^(e - 127), code 0xFF NaN; the page's int8 scale tensors
 * are read as E8M0, so they are passed as MM_SF_E8M0. */
typedef enum mm_sf_type {
    MM_SF_E8M0 = 0,
    MM_SF_E4M3FN = 1
} mm_sf_type;

/*
 * mm_scaled_gemm -- d = (a * s_a) @ (b * s_b)^T, cast to d_type.
 *
 * Defined by "TileOPs: Linear Algebra Operators", tileops.gemm.GemmFP8FwdOp
 * (the FP8 NT GEMM with per-tensor, 1x128 or 128x128 scales) and
 * "mmaemu API reference (v0.1)", mmaemu.scaled_mm (torch._scaled_mm's
 * arguments: per-tensor scales multiply the result, scale_result for FP8
 * outputs, fast or slow accumulation, output dtypes).
 *
 *  a        [M, K] FP8 codes of a_type, row-major with row pitch lda bytes
 *           (lda >= K). The caller guarantees (M-1)*lda + K readable bytes.
 *  b        [N, K] FP8 codes of b_type, row pitch ldb bytes (ldb >= K): the
 *           [N, K] weight, i.e. scaled_mm's column-major mat2 [K, N] read as
 *           its transpose. a_type and b_type may differ (E4M3 x E5M2 mixes).
 *  scale_a  fp32, by sa_mode: [1] or [M, ceil(K/128)] (1x128).
 *  scale_b  fp32, by sb_mode: [1], [N, ceil(K/128)] (1x128) or
 *           [ceil(N/128), ceil(K/128)] (128x128).
 *           Accepted pairs: (TENSOR, TENSOR), (1x128, 1x128), (1x128, 128x128);
 *           any other pair -> MM_ERR_UNSUPPORTED.
 *  scale_result  fp32 [1] or NULL (= 1). Read only when d_type is an FP8
 *           type; the value is multiplied into the result before the cast.
 *  d        [M, N] of d_type (F32, BF16, F16, F8_E4M3FN or F8_E5M2), row pitch
 *           ldd ELEMENTS (ldd >= N). Previous contents never matter.
 *  use_fast_accum  nonzero: one fp32 accumulation chain over all of K;
 *           zero: each 128-element K chunk is summed into a fresh fp32
 *           partial that is then added to the fp32 accumulator ("slow").
 *           Block-scaled modes always promote per 128-chunk (the scale changes
 *           per chunk), so the flag does not change them.
 *
 * Result, per output element: every FP8 value is converted exactly to bf16
 * and the sum over k of the products is formed in fp32 by the bf16 MFMA units
 * (every product of two FP8 values is exact there); per-tensor scales multiply it as fp32(s_a * s_b); block scales multiply each
 * 128-chunk partial as fp32(sa[m,kb] * sb[n,kb]) in a fused multiply-add; an
 * FP8 output is then multiplied by scale_result. The cast rounds to nearest
 * even: bf16 / f16 / f32 overflow to +-Inf, FP8 outputs saturate to +-max
 * (+-Inf included); NaN is stored as the canonical pattern of its type (f32
 * 0x7FFFFFFF, bf16 / f16 0x7FFF, FP8 0x7F), the encodings of "mmaemu
 * testing", Bitwise policy. An exactly-zero sum is +0 before the scales.
 *
 * Sizes and alignment: M, N, K in [0, 2^31); M == 0 or N == 0 returns MM_OK
 * with nothing enqueued; K == 0 gives the empty sum (+0) times the scales.
 * a and b must be 16-byte aligned, lda and ldb multiples of 8 and at most
 * 2^22 bytes; d aligned to its element size; scale pointers 4-byte aligned.
 * Violations -> MM_ERR_MISALIGNED.
 */
mm_status mm_scaled_gemm(int64_t M, int64_t N, int64_t K,
                         const void* a, int a_type, int64_t lda,
                         const void* b, int b_type, int64_t ldb,
                         const float* scale_a, int sa_mode,
                         const float* scale_b, int sb_mode,
                         const float* scale_result,
                         void* d, int d_type, int64_t ldd,
                         int use_fast_accum,
                         void* stream);

/*
 * mm_scaled_gemm_bias -- mm_scaled_gemm with a bias added after the scales.
 *
 * Defined by "TileOPs: Linear Algebra Operators", tileops.gemm.GemmFP8FwdOp,
 * forward(a, b, scale_a, scale_b, bias): the product with its scales applied,
 * plus an optional bias vector of the output type, one value per column.
 *
 *  bias     [N] of d_type, or NULL (then the call is mm_scaled_gemm's). d_type
 *           must be F32, BF16 or F16 when bias is given (the page's outputs
 *           are bf16 and f16); an FP8 d_type with a bias -> MM_ERR_UNSUPPORTED.
 *           Aligned to its element size, else MM_ERR_MISALIGNED.
 *  Every other argument is mm_scaled_gemm's (there is no scale_result: it only
 *  applies to FP8 outputs).
 *
 * Result: d[m, n] = cast(v + bias[n]) where v is mm_scaled_gemm's fp32 value
 * before the cast (the scaled sum); the bias is widened exactly to fp32 and
 * added in one fp32 addition, then the result is rounded once to d_type.
 */
mm_status mm_scaled_gemm_bias(int64_t M, int64_t N, int64_t K,
                              const void* a, int a_type, int64_t lda,
                              const void* b, int b_type, int64_t ldb,
                              const float* scale_a, int sa_mode,
                              const float* scale_b, int sb_mode,
                              const void* bias,
                              void* d, int d_type, int64_t ldd,
                              int use_fast_accum,
                              void* stream);

/*
 * mm_scaled_gemm_batched -- L independent per-tensor-scaled FP8 GEMMs,
 * d[l] = (a[l] * s_a) @ (b[l] * s_b)^T cast to d_type, for l = 0 .. L-1.
 *
 * Defined by "TileOPs: Linear Algebra Operators", tileops.gemm.BmmFP8FwdOp
 * (batched FP8 GEMM, one per-tensor scale for a and one for b shared by the
 * whole batch). b is taken with K innermost, the page's trans_b layout
 * [B, N, K], which the page names as the layout that needs no transposed
 * copy; a caller holding b as [B, K, N] transposes it first (mm_transpose_u8).
 *
 *  L        batch count, in [0, 2^31); L == 0 returns MM_OK, nothing enqueued.
 *  a        item l at a + l * stride_a bytes: [M, K], row pitch lda bytes.
 *  b        item l at b + l * stride_b bytes: [N, K], row pitch ldb bytes.
 *  scale_a, scale_b  fp32 [1] each, for every item.
 *  scale_result, d_type, use_fast_accum  as in mm_scaled_gemm.
 *  d        item l at d + l * stride_d ELEMENTS: [M, N], row pitch ldd.
 *  Strides are >= 0 (items may alias for the inputs; outputs that overlap
 *  give an unspecified result). With L > 1, stride_a and stride_b must be
 *  multiples of 16 bytes (MM_ERR_MISALIGNED otherwise). The other rules are
 *  mm_scaled_gemm's, applied to every item.
 *
 * Result: item by item, exactly mm_scaled_gemm's with TENSOR scale modes.
 */
mm_status mm_scaled_gemm_batched(int64_t L, int64_t M, int64_t N, int64_t K,
                                 const void* a, int a_type, int64_t lda, int64_t stride_a,
                                 const void* b, int b_type, int64_t ldb, int64_t stride_b,
                                 const float* scale_a, const float* scale_b,
                                 const float* scale_result,
                                 void* d, int d_type, int64_t ldd, int64_t stride_d,
                                 int use_fast_accum,
                                 void* stream);

/*
 * mm_scaled_gemm_grouped -- grouped FP8 GEMM: one GEMM per group, the groups'
 * rows packed along M, as "TileOPs: Linear Algebra Operators",
 * tileops.gemm.GroupedGemmFwdOp defines it in its default NT layout
 * (forward(a, b, batch_sizes, batch_offsets)), with FP8 operands scaled as
 * tileops.gemm.BmmFP8FwdOp's: one fp32 scale for a and one for b.
 *
 *  a        [batch_sum][lda] FP8 codes: the rows of every group; group g owns
 *           rows batch_offsets[g] .. batch_offsets[g] + batch_sizes[g] - 1.
 *  b        [G][N][ldb] FP8 codes (K innermost, the page's NT), group g's
 *           operand at b + g * stride_b bytes.
 *  batch_sizes, batch_offsets  int32 [G], DEVICE pointers: rows and first row
 *           of each group. As on the page they are not checked (that would
 *           synchronise): the sizes must add up to batch_sum and the offsets be
 *           their exclusive prefix sum. Values that do not give unspecified
 *           rows, never an access outside a, b, d or the two arrays: each
 *           group's rows are clamped to [0, batch_sum).
 *  d        [batch_sum][ldd] of d_type: row r of group g is
 *           d[r, n] = (a[r,:] . b[g][n,:]) * scale_a * scale_b, cast as in
 *           mm_scaled_gemm (scale_result for FP8 outputs, fast or slow
 *           accumulation). Rows no group covers are not written.
 *
 * Sizes: batch_sum, N, K and G in [0, 2^31), (ceil(batch_sum/64) + G) *
 * ceil(N/64) < 2^31. G, batch_sum or N == 0: nothing is launched. Alignment as
 * mm_scaled_gemm (stride_b a multiple of 16 when G > 1); batch_sizes and
 * batch_offsets 4-byte aligned. Errors as mm_scaled_gemm.
 */
mm_status mm_scaled_gemm_grouped(int64_t batch_sum, int64_t N, int64_t K, int64_t G,
                                 const void* a, int a_type, int64_t lda,
                                 const void* b, int b_type, int64_t ldb, int64_t stride_b,
                                 const int32_t* batch_sizes, const int32_t* batch_offsets,
                                 const float* scale_a, const float* scale_b,
                                 const float* scale_result,
                                 void* d, int d_type, int64_t ldd,
                                 int use_fast_accum,
                                 void* stream);

/*
 * mm_transpose_u8 -- byte transpose, dst[l][c][r] = src[l][r][c]: the copy
 * that "TileOPs: Linear Algebra Operators", tileops.gemm.BmmFP8FwdOp makes of
 * a b that arrives as [B, K, N] (N innermost), since the GEMM reads b with K
 * innermost. One extra read and write of the operand.
 *
 *  L, R, C  items, rows and columns of src, each >= 0; L < 2^16, C < 2^22,
 *           R < 2^30 (MM_ERR_UNSUPPORTED otherwise). Any of them 0: MM_OK,
 *           nothing enqueued.
 *  src      item l at src + l * stride_src bytes: [R][ld_src], ld_src >= C.
 *  dst      item l at dst + l * stride_dst bytes: [C][ld_dst], ld_dst >= R.
 *           Bytes of dst past R in a row are not written. src and dst must
 *           not overlap. Both are DEVICE pointers owned by the caller.
 * No alignment is required. Errors as mm_scaled_gemm.
 */
mm_status mm_transpose_u8(int64_t L, int64_t R, int64_t C,
                          const void* src, int64_t ld_src, int64_t stride_src,
                          void* dst, int64_t ld_dst, int64_t stride_dst,
                          void* stream);

/*
 * mm_grouped_workspace_bytes -- bytes of device workspace that
 * mm_scaled_gemm_grouped_layout needs for these sizes and layout (written to
 * *bytes; 0 for NT and when G, N or K is 0). Needs no GPU. Negative sizes: MM_ERR_INVALID_ARGUMENT.
 */
mm_status mm_grouped_workspace_bytes(int64_t batch_sum, int64_t N, int64_t K, int64_t G,
                                     int transpose_a, int transpose_b, uint64_t* bytes);

/*
 * mm_scaled_gemm_grouped_layout -- the grouped FP8 GEMM in the four layouts of
 * "TileOPs: Linear Algebra Operators", tileops.gemm.GroupedGemmFwdOp (its
 * layout table and forward's argument shapes), selected by (transpose_a,
 * transpose_b), with one fp32 scale for a and one for b as in
 * mm_scaled_gemm_grouped. The metadata rules are that function's.
 *
 * Without transpose_a the groups split the rows of a [batch_sum][lda] (K
 * used), d is [batch_sum][ldd] (stride_d is ignored):
 *  NT (0, 1)  b [G][N][ldb], K used: exactly mm_scaled_gemm_grouped (no
 *             workspace).
 *  NN (0, 0)  b [G][K][ldb], N used, group g's at b + g * stride_b bytes:
 *             d[r, n] = sum_k a[r, k] b[g][k, n] * scale_a * scale_b.
 * With transpose_a the groups split the contraction; a is [batch_sum][lda]
 * (N used) and group g yields the [N][K] block
 *   d[g][n, k] = sum over g's rows r of a[r, n] * B(r, k) * scale_a * scale_b
 * at d + g * stride_d ELEMENTS, rows of ldd (>= K) elements; an empty group
 * gives +0. (N and K name the block's extents as on the page.)
 *  TN (1, 0)  b [batch_sum][ldb], K used: B(r, k) = b[r, k].
 *  TT (1, 1)  b [K][ldb], batch_sum used: B(r, k) = b[k, r].
 * Each group's product is mm_scaled_gemm's (the slow mode's 128-element
 * chunks counted from the group's first row), cast to d_type as there.
 *
 *  workspace  DEVICE memory of at least mm_grouped_workspace_bytes bytes,
 *           16-byte aligned, owned by the caller, used by this call's kernels
 *           on `stream` until they finish: the operands repacked with the
 *           contraction innermost, each group starting on a 16-byte boundary.
 *           Its previous contents never matter. NULL is accepted when 0 bytes
 *           are needed.
 * Limits (MM_ERR_UNSUPPORTED): NN: G < 2^16, N < 2^22, round16(K) <= 2^22;
 * TN / TT: round16(batch_sum) + 16 G <= 2^22, N and K < 2^22,
 * G ceil(N/64) ceil(K/64) < 2^31. G, N or K == 0 with transpose_a: MM_OK,
 * nothing enqueued. Errors as mm_scaled_gemm; a workspace that is too small
 * is MM_ERR_INVALID_ARGUMENT. Bad metadata gives unspecified values, never an
 * access outside the arguments.
 */
mm_status mm_scaled_gemm_grouped_layout(int64_t batch_sum, int64_t N, int64_t K, int64_t G,
                                        int transpose_a, int transpose_b,
                                        const void* a, int a_type, int64_t lda,
                                        const void* b, int b_type, int64_t ldb, int64_t stride_b,
                                        const int32_t* batch_sizes, const int32_t* batch_offsets,
                                        const float* scale_a, const float* scale_b,
                                        const float* scale_result,
                                        void* d, int d_type, int64_t ldd, int64_t stride_d,
                                        void* workspace, uint64_t workspace_bytes,
                                        int use_fast_accum,
                                        void* stream);

/*
 * mm_blockscaled_gemm_amax -- batched block-scaled GEMM with a global amax.
 *
 * Defined by "cuDNN frontend: GEMM + Amax (SM100)", Overview, Shapes and
 * Equations: A^[m,k,l] = A[m,k,l] * SFA(m, k / sf_vec_size, l),
 * B^[n,k,l] = B[n,k,l] * SFB(n, k / sf_vec_size, l),
 * C[m,n,l] = sum_k A^[m,k,l] B^[n,k,l], Amax = max over m,n,l of |C[m,n,l]|.
 *
 *  a        [L][M][K] FP8 codes (k-major), b [L][N][K], both of ab_type (the
 *           two operands must have the same type, as the page requires).
 *  sfa      [L][M][ceil(K/sf_vec_size)] fp32 scale factors, sfb
 *           [L][N][ceil(K/sf_vec_size)]. Each value must be a power of two
 *           2^e with -127 <= e <= 127 (an E8M0 value carried in fp32; 2^-127
 *           is the fp32 subnormal 0x00400000). Only the exponent field is
 *           read: any other value x acts as 2^floor(log2|x|), zero as 2^-127,
 *           Inf / NaN as the E8M0 NaN.
 *  sf_vec_size  32. The page's other value, 16, is not supported with FP8
 *           operands there either -> MM_ERR_UNSUPPORTED; anything else ->
 *           MM_ERR_INVALID_ARGUMENT.
 *  c        [L][M][N] of c_type (F32, BF16 or F16), i.e. the page's (M, N, L)
 *           tensor in n-major order. FP8 C with FP8 operands is disabled on
 *           the page as well -> MM_ERR_UNSUPPORTED.
 *  amax     fp32 [1] or NULL: max over all outputs of |C| taken on the fp32
 *           value before the cast to c_type. NaN if any output is NaN; +0 when
 *           M*N*L == 0.
 *  amax_index  int64 [1] or NULL: linear index l*M*N + m*N + n of the
 *           maximum, the smallest such index on ties; -1 when M*N*L == 0.
 *           Requires M*N*L < 2^33.
 *
 * Each FP8 value is multiplied by its group's scale factor as it is
 * converted to bf16, which is exact while the scaled value stays in bf16's
 * range (E4M3: e in [-124, 119], E5M2: e in [-117, 112]; outside it the
 * operand loses precision, nothing faults); the products are summed over K in
 * one fp32 chain by the bf16 MFMA units. The cast to c_type and NaN encodings follow mm_scaled_gemm.
 * The library clears amax / amax_index itself, with its own kernels on
 * `stream`; the outputs are final when the stream reaches the end of the call.
 *
 * Sizes and alignment: M, N, K, L in [0, 2^31) with L*M*K, L*N*K and L*M*N
 * below 2^48. a, b and c 16-byte aligned and K a multiple of 16 (the page
 * asks for 16-byte alignment along the contiguous dimension); sfa, sfb, amax
 * 4-byte and amax_index 8-byte aligned -> else MM_ERR_MISALIGNED.
 * M, N or L == 0: no GEMM is launched; amax / amax_index are still written.
 */
mm_status mm_blockscaled_gemm_amax(int64_t M, int64_t N, int64_t K, int64_t L,
                                   const void* a, const void* b, int ab_type,
                                   const float* sfa, const float* sfb, int sf_vec_size,
                                   void* c, int c_type,
                                   float* amax, int64_t* amax_index,
                                   void* stream);

/*
 * mm_blockscaled_gemm_amax_atom -- mm_blockscaled_gemm_amax with the scale
 * factors in the page's own format (E8M0 bytes in the atom layout of
 * "cuDNN frontend: GEMM + Amax (SM100)", Shapes and Parameters, SFA and SFB),
 * and with the page's FP4 operands.
 *
 *  a, b     ab_type MM_F8_E4M3FN or MM_F8_E5M2: [L][M][K] and [L][N][K]
 *           codes, as mm_blockscaled_gemm_amax. MM_F4_E2M1: [L][M][K/2] and
 *           [L][N][K/2] bytes of two E2M1 values each (element 2i in the low
 *           nibble of byte i: the page does not say, and C does not depend
 *           on it), K a multiple of 32.
 *  sf_vec_size  32, or 16 with FP4 operands (16 with FP8 operands ->
 *           MM_ERR_UNSUPPORTED, as on the page).
 *  sfa      the page's SFA of logical shape (32, 4, ceil(M/128), 4,
 *           ceil(K/(4 sf)), L), sf = sf_vec_size, passed as its C-contiguous
 *           storage (L, ceil(M/128), ceil(K/(4 sf)), 32, 4, 4) bytes, which the
 *           page's JAX contract says the logical view is a permutation of
 *           (3, 4, 1, 5, 2, 0). Row m and group g (values [g sf, g sf + sf))
 *           of batch item l use the byte at
 *           [l][m / 128][g / 4][m % 32][(m / 32) % 4][g % 4] (the page gives
 *           shapes only: row m = i0 + 32 i1 + 128 i2 and group g = j0 + 4 j1 of
 *           the logical coordinates is the reading taken). Every byte of the
 *           padded shape must be readable; bytes of rows past M or groups past
 *           ceil(K/sf) are never used.
 *  sfb      the same for B with N rows.
 *  sf_type  MM_SF_E8M0 (int8 tensors included), or MM_SF_E4M3FN with FP4
 *           operands and sf_vec_size 16, the one combination the page allows
 *           for E4M3 factors (others -> MM_ERR_UNSUPPORTED); other values ->
 *           MM_ERR_INVALID_ARGUMENT. An E4M3 factor is any E4M3 value (signed,
 *           subnormal, NaN codes give NaN).
 *  c_type   F32, BF16 or F16; with FP4 operands also MM_F8_E4M3FN or
 *           MM_F8_E5M2 (rounded to nearest even, saturating, as
 *           mm_scaled_gemm's FP8 outputs with scale_result 1) and MM_F4_E2M1:
 *           c is then [L][M][ceil(N/2)] bytes, two values each (low nibble
 *           first, an odd N's last high nibble 0), rounded to nearest even,
 *           saturating at +-6, NaN written as the code of +6 (E2M1 has no
 *           NaN; the page gives no rule). FP8 or FP4 C with FP8 operands ->
 *           MM_ERR_UNSUPPORTED.
 *
 * Everything else (amax, amax_index, stream, the arithmetic, sizes, alignment
 * and errors) is as mm_blockscaled_gemm_amax; in addition each batch item's
 * factor tensor must stay below 2^31 bytes (else MM_ERR_UNSUPPORTED). Every
 * E2M1 value times a factor 2^e is a bf16 value for e <= 125, so FP4 operands
 * are converted exactly with every E8M0 factor but 2^126 and 2^127; times an
 * E4M3 factor it is an f16 value (those operands are contracted in f16), so
 * E4M3 factors are exact throughout.
 */
mm_status mm_blockscaled_gemm_amax_atom(int64_t M, int64_t N, int64_t K, int64_t L,
                                        const void* a, const void* b, int ab_type,
                                        const void* sfa, const void* sfb, int sf_type, int sf_vec_size,
                                        void* c, int c_type,
                                        float* amax, int64_t* amax_index,
                                        void* stream);

/*
 * mm_scaled_gemm_grouped_layout_noalloc -- mm_scaled_gemm_grouped_layout for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same arguments
 * and result without the workspace, whose role a scratch array of the
 * library takes. Nothing is allocated or freed by the call.
 *
 *  The scratch array is MM_NOALLOC_SCRATCH_BYTES bytes of device memory in
 *  the library's code object: every GPU the library is used on holds one copy
 *  from the library's load until the process ends. A layout and size whose
 *  mm_grouped_workspace_bytes exceeds it -> MM_ERR_UNSUPPORTED (nothing
 *  enqueued). The NT layout needs none. Nothing in the array needs clearing:
 *  the packing kernels write every byte the GEMM reads.
 *  All calls on one GPU share its array (it keeps the last call's contents):
 *  calls that overlap on one GPU (on different streams, or from different
 *  threads) race and give unspecified results. Calls on one stream are ordered
 *  and safe.
 *  The first call on a device that needs the array resolves its device
 *  address (hipGetSymbolAddress, with the device current; a HIP query, no
 *  work enqueued) before the remaining arguments are validated; a failure
 *  there is MM_ERR_DEVICE.
 * Everything else (arguments, layouts, limits, errors) is
 * mm_scaled_gemm_grouped_layout's.
 */
#define MM_NOALLOC_SCRATCH_BYTES (160ull << 20)
mm_status mm_scaled_gemm_grouped_layout_noalloc(int64_t batch_sum, int64_t N, int64_t K, int64_t G,
                                                int transpose_a, int transpose_b,
                                                const void* a, int a_type, int64_t lda,
                                                const void* b, int b_type, int64_t ldb, int64_t stride_b,
                                                const int32_t* batch_sizes, const int32_t* batch_offsets,
                                                const float* scale_a, const float* scale_b,
                                                const float* scale_result,
                                                void* d, int d_type, int64_t ldd, int64_t stride_d,
                                                int use_fast_accum,
                                                void* stream);

/* Message for the last non-OK status returned on the calling thread ("" if
 * none). The pointer stays valid until the thread's next mm_* call. */
const char* mm_last_error(void);

/* Library name, version and target, e.g. "mmfp8 0.1.0 gfx950". */
const char* mm_version(void);

/*
 * mm_debug_convert -- test hook, not part of the GEMM contract: rounds n fp32
 * values x (device) to dtype with exactly the conversion the GEMM epilogues
 * use (round to nearest even, FP8 saturating, canonical NaN) and writes the
 * bit patterns to y (device; 1, 2 or 4 bytes per element). x and y must be
 * aligned to their element sizes.
 */
mm_status mm_debug_convert(const float* x, void* y, int dtype, int64_t n, void* stream);

/*
 * mm_debug_mfma_gemm -- test hook, not part of the GEMM contract: a plain
 * GEMM whose products are summed by the gfx950 scaled FP8 / FP4 MFMA
 * (v_mfma_scale_f32_16x16x128_f8f6f4, one fp32 chain over K), to measure how
 * exactly that instruction sums ("mmaemu API reference (v0.1)", instruction
 * model, is the pages' account of such limited tensor-core sums).
 * d[m][n] = sum_k A[m][k] B[n][k] 2^(sfa[m][k/32] - 127) 2^(sfb[n][k/32] - 127).
 *  a, b     [M][K] / [N][K] codes of ab_type (MM_F8_E4M3FN, MM_F8_E5M2, or
 *           MM_F4_E2M1 two per byte, rows of K/2 bytes), 16-byte aligned.
 *  sfa, sfb [M][K/32] / [N][K/32] E8M0 bytes, or NULL (all 127, i.e. 1).
 *  d        [M][N] fp32.
 * M and N multiples of 16, K of 128 (else MM_ERR_UNSUPPORTED). Device
 * pointers; asynchronous on stream.
 */
mm_status mm_debug_mfma_gemm(int64_t M, int64_t N, int64_t K, const void* a, const void* b, int ab_type,
                             const void* sfa, const void* sfb, float* d, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MMFP8_MM_H */
