"""GPU parity: the C ABI on an MI355X against the CPU oracle, element by element.

Bars: bit-exact where the result is exact by construction (single products,
conversions, closed forms, amax against the GPU's own C, batch vs separate
calls); otherwise the tolerances of tests/compare.py (fp32 out: 2^-20 * sum|t|;
bf16 / f16 / FP8 out: 1 ulp after rounding).
"""
import numpy as np
import pytest

import compare
import datagen
import oracle
from oracle import E4M3FN, E5M2, F32, BF16, F16

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")
DTYPES = (F32, BF16, F16, E4M3FN, E5M2)
DT_NAME = {F32: "f32", BF16: "bf16", F16: "f16", E4M3FN: "e4m3", E5M2: "e5m2"}


def sample_rows(M, n_each=16, seed=0):
    """Rows checked at sizes where every row would take the oracle too long: tile_rows with `n_each` rows at
    each edge."""
    return tile_rows(M, band=64, edge=n_each, seed=seed)


def tile_rows(M, band=64, edge=16, seed=0):
    """The first and last `edge` rows and one seeded row in every `band`-row band: every workgroup tile row of
    every kernel (tiles are 64 to 256 rows high, all aligned to 64) has at least one checked row, over all
    columns."""
    if M <= 2 * edge + band:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    starts = np.arange(0, M, band)
    pick = starts + rng.integers(0, band, size=starts.size)
    pick = pick[pick < M]
    return np.unique(np.concatenate([np.arange(edge), pick, np.arange(M - edge, M)]))


def check_gemm(d, sa_mode, sb_mode, d_type, fast, rows=None, scale_result=None, what="", ldd=None):
    a, b, K = d["a"], d["b"], d["K"]
    gpu = gu.scaled_gemm(a, d["a_fmt"], b, d["b_fmt"], K, d["scale_a"], sa_mode, d["scale_b"], sb_mode, d_type,
                         scale_result=scale_result, fast=fast, ldd=ldd)
    value, sabs, bits = oracle.scaled_gemm_k(a, d["a_fmt"], b, d["b_fmt"], K, d["scale_a"], sa_mode, d["scale_b"],
                                             sb_mode, d_type, scale_result=scale_result, rows=rows)
    g = gpu if rows is None else gpu[rows]
    return compare.check(g, value, sabs, bits, d_type, what), gpu, value, bits


# ------------------------------------------------------------------ exact cases

@pytest.mark.parametrize("fa,fb", [(E4M3FN, E4M3FN), (E5M2, E5M2), (E4M3FN, E5M2), (E5M2, E4M3FN)])
@pytest.mark.parametrize("fast", [True, False])
def test_product_table_bit_exact(fa, fb, fast):
    """All 256 x 256 code pairs as single products (K = 128, codes in column 0):
    every output is one exact product, NaN / Inf included."""
    a = np.zeros((256, 128), np.uint8); a[:, 0] = np.arange(256)
    b = np.zeros((256, 128), np.uint8); b[:, 0] = np.arange(256)
    gpu = gu.scaled_gemm(a, fa, b, fb, 128, 1.0, 0, 1.0, 0, F32, fast=fast)
    _, _, bits = oracle.scaled_gemm(a, fa, b, fb, np.float32(1), 0, np.float32(1), 0, F32)
    compare.assert_bitwise_equal(gpu, bits, f"product table {fa}x{fb}")


@pytest.mark.parametrize("dtype", DTYPES, ids=[DT_NAME[t] for t in DTYPES])
def test_epilogue_conversion_bit_exact(dtype):
    """The epilogue cast alone (test hook) on 2^24 sampled fp32 patterns plus
    dense sweeps of every binade near the output ranges."""
    rng = np.random.default_rng(1)
    bits = (np.arange(1 << 24, dtype=np.uint64) * 256 + rng.integers(0, 256, 1 << 24)).astype(np.uint32)
    dense = [np.float32(2.0 ** e).view(np.uint32) + (np.arange(8192, dtype=np.uint32) << 10) for e in range(-30, 20)]
    bits = np.concatenate([bits] + dense + [np.array([0x7FC00000, 0x7F800001, 0xFFFFFFFF, 0x7F800000, 0, 0x80000000],
                                                     np.uint32)])
    x = bits.view(np.float32)
    gpu = gu.debug_convert(x, dtype)
    want = oracle.round_to(x.astype(np.float64), dtype)
    compare.assert_bitwise_equal(gpu, want, f"convert to {DT_NAME[dtype]}")


def test_adversarial_structured_rows_bit_exact():
    d = datagen.set_adversarial_n4096(64, 4096, 4096)
    gpu = gu.scaled_gemm(d["a"], 0, d["b"], 0, 4096, 1.0, 0, 1.0, 0, BF16, fast=False)
    _, _, bits = oracle.scaled_gemm(d["a"], 0, d["b"], 0, np.float32(1), 0, np.float32(1), 0, BF16, rows=[0, 1, 2, 3])
    assert gpu[0, 0] == bits[0, 0] and gpu[0, 0] != 0          # K * 448^2, exact in bf16
    assert gpu[1, 1] == 0x0000                                 # alternating +-448 against +448: +0
    assert gpu[2, 2] == bits[2, 2]                             # K * 2^-18
    assert np.all(gpu[3] == 0x0000)                            # all -0 codes: +0 everywhere


# ------------------------------------------------------------------ 256 x 256 x 256, scales 0.5 / 0.25, f32 out

@pytest.mark.parametrize("fast", [True, False])
def test_gemm_256_cubed(fast):
    d = datagen.set_256_cubed()
    check_gemm(d, 0, 0, F32, fast, what="256^3")


# ------------------------------------------------------------------ per-tensor, N = K = 4096, M = 16 .. 8192 (the benchmark shapes)

@pytest.mark.parametrize("M", datagen.BENCH_MS)
def test_gauss_n4096_full_size(M):
    d = datagen.set_gauss_n4096(M)
    rows = None if M <= 256 else tile_rows(M, seed=M)
    check_gemm(d, 0, 0, BF16, fast=False, rows=rows, what=f"gauss N=K=4096 M={M}")


@pytest.mark.parametrize("M", datagen.BENCH_MS)
def test_adversarial_n4096_full_size(M):
    d = datagen.set_adversarial_n4096(M)
    rows = None if M <= 256 else tile_rows(M, seed=M + 1)
    check_gemm(d, 0, 0, BF16, fast=False, rows=rows, what=f"adversarial N=K=4096 M={M}")


@pytest.mark.parametrize("M", [16, 64, 256, 2048])
def test_gauss_n4096_fast_accumulation(M):
    d = datagen.set_gauss_n4096(M)
    check_gemm(d, 0, 0, BF16, fast=True, rows=None if M <= 256 else tile_rows(M, seed=2), what=f"fast M={M}")


# ------------------------------------------------------------------ ragged shapes, padding, all output types

RAGGED = [(300, 520, 1000), (17, 33, 132), (1, 1, 1), (5, 7, 3), (257, 129, 4104), (65, 100, 200),
          (40, 4096, 520), (130, 260, 136), (33, 48, 8200)]


@pytest.mark.parametrize("M,N,K", RAGGED)
@pytest.mark.parametrize("fast", [True, False])
def test_ragged_shapes_with_padding(M, N, K, fast):
    """Row pitches padded past K with NaN codes (never read as data), output
    rows padded (scalar stores), every output type."""
    g = np.random.default_rng(M * 7 + N * 3 + K)
    lda = (K + 7) // 8 * 8 + 8
    ldb = (K + 7) // 8 * 8 + 16
    a = np.full((M, lda), 0x7F, np.uint8); a[:, :K] = datagen.gauss_codes(g, (M, K), 64.0)
    b = np.full((N, ldb), 0x7F, np.uint8); b[:, :K] = datagen.gauss_codes(g, (N, K), 64.0)
    d = dict(a=a, b=b, K=K, a_fmt=E4M3FN, b_fmt=E4M3FN, scale_a=np.float32(0.75), scale_b=np.float32(-0.375))
    for i, dt in enumerate(DTYPES):
        ldd = N + (3 if i % 2 else 0)
        check_gemm(d, 0, 0, dt, fast, scale_result=np.float32(1 / 64) if dt in (E4M3FN, E5M2) else None,
                   what=f"{M}x{N}x{K} {DT_NAME[dt]}", ldd=ldd)


def test_zero_k_gives_scaled_zero():
    a = np.zeros((20, 8), np.uint8); b = np.zeros((30, 8), np.uint8)
    gpu = gu.scaled_gemm(a, 0, b, 0, 0, 2.0, 0, -1.0, 0, F32)
    assert np.all(gpu == 0x80000000)        # (+0) * 2 * (-1) = -0
    gpu = gu.scaled_gemm(a, 0, b, 0, 0, 2.0, 0, 1.0, 0, BF16)
    assert np.all(gpu == 0)


def test_nan_and_inf_inputs():
    d = datagen.set_256_cubed(64, 80, 384)
    a = d["a"].copy(); b = d["b"].copy()
    a[5, 17] = 0x7F                          # E4M3 NaN code: row 5 is NaN everywhere
    b_e5 = datagen.gauss_codes(np.random.default_rng(3), (80, 384), 4.0, E5M2)
    b_e5[7, 100] = 0x7C                      # +Inf in column 7
    dd = dict(a=a, b=b_e5, K=384, a_fmt=E4M3FN, b_fmt=E5M2, scale_a=np.float32(1), scale_b=np.float32(1))
    for dt in (F32, BF16, E4M3FN):
        _, gpu, value, _ = check_gemm(dd, 0, 0, dt, False, what=f"nan/inf {DT_NAME[dt]}")
        assert np.all(gpu[5] == compare.CANON_NAN[dt])


@pytest.mark.parametrize("fa,fb", [(E4M3FN, E5M2), (E5M2, E4M3FN), (E5M2, E5M2)])
def test_mixed_and_e5m2_formats(fa, fb):
    g = np.random.default_rng(fa * 2 + fb)
    a = datagen.gauss_codes(g, (150, 640), 8.0, fa)
    b = datagen.gauss_codes(g, (270, 640), 8.0, fb)
    d = dict(a=a, b=b, K=640, a_fmt=fa, b_fmt=fb, scale_a=np.float32(0.5), scale_b=np.float32(0.125))
    for dt in (F32, F16):
        check_gemm(d, 0, 0, dt, False, what=f"mixed {fa}x{fb} {DT_NAME[dt]}")


# ------------------------------------------------------------------ every production tile shape

# (M, N, K, fast) chosen so that each workgroup tile the library picks for
# per-tensor scales runs at least once at a size that selects it, with a ragged
# K whose last chunk straddles a 16-byte boundary (K % 16 == 8).
TILE_CASES = [(4096, 4096, 1032, True),    # fast: 256x256 tile, eight 64x128 waves
              (2048, 4096, 1032, True),    # fast: 128x256
              (1024, 4096, 1032, True),    # fast: 128x128, one per CU: two K groups of four waves
              (1536, 4096, 1032, True),    # fast: 128x128, pipelined fragment reads
              (2048, 4096, 1032, False),   # slow: 128x128, two workgroups per CU
              (1000, 4096, 1032, False),   # slow: 128x128, ragged M, one per CU: two K groups
              (256, 4096, 1032, False),    # K split over the waves, 64x64 tiles (slow: eight waves)
              (300, 4100, 1000, False),    # the same with ragged M, N and K
              (100, 4096, 1032, True)]     # K split over the waves, 32x64 tiles


@pytest.mark.parametrize("M,N,K,fast", TILE_CASES)
def test_production_tiles_per_tensor(M, N, K, fast):
    g = np.random.default_rng(M + K + int(fast))
    a = datagen.gauss_codes(g, (M, K), 64.0)
    b = datagen.gauss_codes(g, (N, K), 64.0)
    d = dict(a=a, b=b, K=K, a_fmt=E4M3FN, b_fmt=E4M3FN, scale_a=np.float32(0.5), scale_b=np.float32(0.25))
    check_gemm(d, 0, 0, BF16, fast, rows=sample_rows(M, 8), what=f"{M}x{N}x{K} fast={fast}")


# Slow accumulation with at least one 256x256 tile per CU runs the 256x256 tile's row-chunk loop: square,
# ragged M and N with mixed formats, FP8 out, ragged K (its last step's chunks at or past K zeroed in LDS; the
# row pitches padded with NaN codes, which must not reach the sums), a K below one step, and a batch of eight
@pytest.mark.parametrize("M,N,K,fa,fb,d_type", [(4096, 4096, 1024, E4M3FN, E4M3FN, BF16),
                                                (4056, 4072, 512, E5M2, E4M3FN, F32),
                                                (4096, 4096, 256, E4M3FN, E5M2, E4M3FN),
                                                (4096, 4096, 1000, E4M3FN, E4M3FN, F32),
                                                (4000, 4096, 1032, E5M2, E5M2, BF16),
                                                (4096, 4096, 40, E4M3FN, E4M3FN, F32),
                                                (4096, 4096, 0, E4M3FN, E4M3FN, F32),
                                                (4001, 4095, 1000, E4M3FN, E5M2, BF16)])
def test_production_tiles_slow_256(M, N, K, fa, fb, d_type):
    g = np.random.default_rng(M + N + K)
    a, b = _nan_padded(g, M, K, fa, 24), _nan_padded(g, N, K, fb, 8)
    d = dict(a=a, b=b, K=K, a_fmt=fa, b_fmt=fb, scale_a=np.float32(0.5), scale_b=np.float32(0.25))
    sr = np.float32(1 / 16) if d_type in (E4M3FN, E5M2) else None
    check_gemm(d, 0, 0, d_type, False, rows=sample_rows(M, 8), scale_result=sr, ldd=N + 3 if d_type == F32 else None,
               what=f"slow 256x256 {M}x{N}x{K}")


def _nan_padded(g, rows, K, fmt, pad):
    """Gaussian codes [rows, K] in a row pitch of K + pad bytes whose padding holds NaN codes."""
    x = np.full((rows, K + pad), 0x7F, np.uint8)
    x[:, :K] = datagen.gauss_codes(g, (rows, K), 64.0, fmt)
    return x


@pytest.mark.parametrize("K", [1024, 1000])
def test_slow_256_matches_128_bitwise(K):
    """The row-chunk loop sums each 128-chunk in the same order as the 128x128 tiles' loop: the first 2048 rows of
    a 4096 x 4096 x K product (256x256 tiles) equal, bit for bit, the 2048 x 4096 x K product of those rows
    (128x128 tiles, two per CU); with a ragged K in NaN-padded pitches too."""
    M, N = 4096, 4096
    g = np.random.default_rng(77 + K)
    a, b = _nan_padded(g, M, K, E4M3FN, 16), _nan_padded(g, N, K, E4M3FN, 16)
    big = gu.scaled_gemm(a, E4M3FN, b, E4M3FN, K, 0.5, 0, 0.25, 0, F32)
    half = gu.scaled_gemm(np.ascontiguousarray(a[:2048]), E4M3FN, b, E4M3FN, K, 0.5, 0, 0.25, 0, F32)
    assert np.all(np.isfinite(half.view(np.float32)))
    compare.assert_bitwise_equal(big[:2048], half, f"256x256 slow rows vs 128x128 slow, K = {K}")


# M = 4096, N = 14336 takes 3.5 rounds of 256x256 tiles: the first 12288 columns run on them (three whole rounds),
# the last 2048 on 128x128 tiles in a second launch (b, d, bias and scale_b moved to those columns)
# (N = 14000: the second launch's 1712 columns end in a partial 128-column tile)
@pytest.mark.parametrize("N,K,sb_mode,d_type", [(14336, 1000, 0, BF16), (14336, 520, 2, BF16), (14336, 136, 2, F32),
                                                (14336, 256, 0, E4M3FN), (14000, 264, 2, BF16), (14000, 392, 0, F16)],
                         ids=["tensor-bf16", "block-bf16", "block-f32", "tensor-e4m3", "block-ragged-n",
                              "tensor-ragged-n"])
def test_split_256_and_128_columns(N, K, sb_mode, d_type):
    M = 4096
    g = np.random.default_rng(K + sb_mode)
    a, b = _nan_padded(g, M, K, E4M3FN, 8), _nan_padded(g, N, K, E4M3FN, 24)
    if sb_mode:
        kb = -(-K // 128)
        sa, sb, sa_mode = datagen.log_uniform_scales(g, (M, kb)), datagen.log_uniform_scales(g, (-(-N // 128), kb)), 1
    else:
        sa, sb, sa_mode = np.float32(0.5), np.float32(0.25), 0
    d = dict(a=a, b=b, K=K, a_fmt=E4M3FN, b_fmt=E4M3FN, scale_a=sa, scale_b=sb)
    sr = np.float32(1 / 16) if d_type == E4M3FN else None
    rows = tile_rows(M, band=256, edge=8)
    check_gemm(d, sa_mode, sb_mode, d_type, False, rows=rows, scale_result=sr, what=f"split {M}x{N}x{K} sb={sb_mode}")


@pytest.mark.parametrize("sb_mode", [0, 2], ids=["tensor", "block"])
def test_split_256_matches_128_bitwise(sb_mode):
    """The split plan's rows equal, bit for bit, those of a 1024-row product on 128x128 tiles only."""
    M, N, K = 4096, 14336, 1000
    g = np.random.default_rng(5 + sb_mode)
    a, b = _nan_padded(g, M, K, E4M3FN, 8), _nan_padded(g, N, K, E4M3FN, 8)
    kb = -(-K // 128)
    if sb_mode:
        sa, sb, sa_mode = datagen.log_uniform_scales(g, (M, kb)), datagen.log_uniform_scales(g, (N // 128, kb)), 1
    else:
        sa, sb, sa_mode = 0.5, 0.25, 0
    big = gu.scaled_gemm(a, E4M3FN, b, E4M3FN, K, sa, sa_mode, sb, sb_mode, F32)
    part = gu.scaled_gemm(np.ascontiguousarray(a[:1024]), E4M3FN, b, E4M3FN, K, sa[:1024] if sb_mode else sa, sa_mode,
                          sb, sb_mode, F32)
    assert np.all(np.isfinite(part.view(np.float32)))
    compare.assert_bitwise_equal(big[:1024], part, f"split plan rows vs 128x128 tiles, sb={sb_mode}")


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 1024), (4096, 14336, 256)], ids=["256x256", "split"])
def test_bias_slow_256(M, N, K):
    g = np.random.default_rng(91 + N)
    a = datagen.gauss_codes(g, (M, K), 64.0)
    b = datagen.gauss_codes(g, (N, K), 64.0)
    bias_bits = _bias_bits(g, N, BF16)
    gpu = gu.scaled_gemm_bias(a, E4M3FN, b, E4M3FN, K, 0.5, 0, 0.25, 0, bias_bits, BF16)
    rows = sample_rows(M, 8)
    value, sabs, bits = oracle.scaled_gemm(a, E4M3FN, b, E4M3FN, np.float32(0.5), 0, np.float32(0.25), 0, BF16,
                                           rows=rows, bias=_bias_values(bias_bits, BF16))
    compare.check(gpu[rows], value, sabs, bits, BF16, f"bias slow {M}x{N}x{K}")


# M = 33 .. 64 with K <= 4096 runs the skinny kernel with sixteen waves and two K steps each in flight (K = 4096,
# a ragged K = 4040 whose last chunk straddles a 16-byte boundary, K = 136), a longer K the eight-wave one
# (K = 8200)
@pytest.mark.parametrize("M,N,K,fast,d_type", [(64, 4096, 4096, False, BF16), (33, 1000, 4040, True, F32),
                                               (48, 777, 8200, False, E4M3FN), (64, 130, 8200, True, F16),
                                               (40, 4100, 136, False, E5M2)])
def test_skinny_m33_to_64(M, N, K, fast, d_type):
    g = np.random.default_rng(M * 31 + K)
    lda, ldb = (K + 7) // 8 * 8 + 8, (K + 7) // 8 * 8
    a = np.full((M, lda), 0x7F, np.uint8); a[:, :K] = datagen.gauss_codes(g, (M, K), 64.0)
    b = np.full((N, ldb), 0x7F, np.uint8); b[:, :K] = datagen.gauss_codes(g, (N, K), 64.0, E5M2 if fast else E4M3FN)
    d = dict(a=a, b=b, K=K, a_fmt=E4M3FN, b_fmt=E5M2 if fast else E4M3FN, scale_a=np.float32(0.5),
             scale_b=np.float32(2.0 ** -7))
    sr = np.float32(1 / 8) if d_type in (E4M3FN, E5M2) else None
    check_gemm(d, 0, 0, d_type, fast, scale_result=sr, what=f"skinny {M}x{N}x{K}", ldd=N + 3)


@pytest.mark.parametrize("sb_mode", [1, 2], ids=["1x128", "128x128"])
@pytest.mark.parametrize("M", [2048, 1024, 200], ids=["128x128", "128x128-kgroups", "64x64"])
def test_production_tiles_block_scaled(M, sb_mode):
    N, K = 4096, 1032
    g = np.random.default_rng(M + sb_mode)
    a = datagen.gauss_codes(g, (M, K), 64.0)
    b = datagen.gauss_codes(g, (N, K), 64.0)
    kb = -(-K // 128)
    sa = datagen.log_uniform_scales(g, (M, kb))
    sb = datagen.log_uniform_scales(g, (N if sb_mode == 1 else -(-N // 128), kb))
    d = dict(a=a, b=b, K=K, a_fmt=E4M3FN, b_fmt=E4M3FN, scale_a=sa, scale_b=sb)
    check_gemm(d, 1, sb_mode, BF16, False, rows=sample_rows(M, 8), what=f"block {M}x{N}x{K} sb={sb_mode}")


# ------------------------------------------------------------------ block scales: 1x128 / 128x128, 4096 x 14336 x 4096

@pytest.mark.parametrize("sb_mode", [1, 2], ids=["1x128", "128x128"])
@pytest.mark.parametrize("M,N,K", [(300, 400, 1000), (64, 256, 512), (260, 130, 4096)])
def test_block_scales_small(M, N, K, sb_mode):
    g = oracle  # noqa
    rng = np.random.default_rng(M + N + K + sb_mode)
    a = datagen.gauss_codes(rng, (M, K), 64.0)
    b = datagen.gauss_codes(rng, (N, K), 64.0)
    kb = -(-K // 128)
    sa = datagen.log_uniform_scales(rng, (M, kb))
    sb = datagen.log_uniform_scales(rng, (N if sb_mode == 1 else -(-N // 128), kb))
    d = dict(a=a, b=b, K=K, a_fmt=E4M3FN, b_fmt=E4M3FN, scale_a=sa, scale_b=sb)
    for dt in (F32, BF16):
        check_gemm(d, 1, sb_mode, dt, False, what=f"block {M}x{N}x{K} sb={sb_mode} {DT_NAME[dt]}")


# block scaling on the production tiles: 128x128 with two K groups (one tile per CU) and with two workgroups per
# CU, a ragged M, and a K whose last chunk straddles a 16-byte boundary; with a 128x128 scale_b these run the
# interleaved main loop (one s_b per wave and step), with a 1x128 scale_b the plain one
BLOCK_TILE_CASES = [(1024, 4096, 1032, 2), (2048, 4096, 1032, 2), (1000, 4096, 1032, 2),
                    (1024, 4096, 1032, 1), (2048, 4096, 1032, 1),
                    (4096, 4096, 1024, 2), (4000, 4072, 1000, 2)]  # 256x256 row-chunk tiles (128x128 scale_b)


@pytest.mark.parametrize("M,N,K,sb_mode", BLOCK_TILE_CASES)
def test_production_tiles_block(M, N, K, sb_mode):
    rng = np.random.default_rng(M * 7 + K + sb_mode)
    a = datagen.gauss_codes(rng, (M, K), 64.0)
    b = datagen.gauss_codes(rng, (N, K), 64.0)
    kb = -(-K // 128)
    sa = datagen.log_uniform_scales(rng, (M, kb))
    sb = datagen.log_uniform_scales(rng, (N if sb_mode == 1 else -(-N // 128), kb))
    d = dict(a=a, b=b, K=K, a_fmt=E4M3FN, b_fmt=E4M3FN, scale_a=sa, scale_b=sb)
    check_gemm(d, 1, sb_mode, BF16, False, rows=tile_rows(M, seed=M + sb_mode),
               what=f"block tiles {M}x{N}x{K} sb={sb_mode}")


def test_block_scaled_full_size():
    d = datagen.set_block_scaled_4096x14336x4096()
    check_gemm(d, 1, 2, BF16, False, rows=tile_rows(4096, seed=3), what="block-scaled 4096x14336x4096")


# ------------------------------------------------------------------ MX factors per 32 + amax: L = 8, 2048 x 2048 x 8192

def check_amax_index_against_oracle(idx, value, sabs):
    """The GPU's amax index is the oracle's, unless the runner-up |C| lies within twice the fp32 bound of the
    maximum (then either may be the maximum after rounding); `value` / `sabs` cover every output."""
    v = np.abs(value.reshape(-1))
    if np.isnan(v).any():
        return
    order = np.argsort(-v, kind="stable")
    top, second = order[0], order[1]
    bound = 2.0 ** -20 * (sabs.reshape(-1)[top] + sabs.reshape(-1)[second])
    if v[top] - v[second] > 2 * bound:
        assert idx == int(top), (idx, int(top))


def check_amax_case(w, c_type, rows=None):
    c, amax, idx = gu.blockscaled_gemm_amax(w["a"], w["b"], w["ab_fmt"], w["sfa"], w["sfb"], c_type)
    value, sabs, bits, _, _ = oracle.blockscaled_gemm_amax(w["a"], w["b"], w["ab_fmt"], w["sfa"], w["sfb"], 32,
                                                           c_type, rows=rows)
    cg = c if rows is None else c[:, rows]
    compare.check(cg, value, sabs, bits, c_type, "sf32 gemm")
    return c, amax, idx, value, sabs


def test_sf32_amax_small_with_oracle():
    w = datagen.set_mx_l8_2048x2048x8192(3, 200, 136, 1024)
    c, amax, idx, value, sabs = check_amax_case(w, F32)
    check_amax_index_against_oracle(idx, value, sabs)
    cf = c.view(np.float32).astype(np.float64).reshape(-1)
    # amax and its index are bit-exact against the GPU's own C
    assert amax == float(np.max(np.abs(cf))) and idx == int(np.argmax(np.abs(cf)))
    # and within the bound of the oracle's amax
    v = np.abs(value.reshape(-1))
    assert abs(amax - v.max()) <= 2.0 ** -20 * sabs.reshape(-1)[np.argmax(v)]


@pytest.mark.parametrize("c_type", [BF16, F16])
def test_sf32_low_precision_outputs(c_type):
    w = datagen.set_mx_l8_2048x2048x8192(2, 96, 200, 512)
    c, amax, idx, value, sabs = check_amax_case(w, c_type)
    # amax is taken before the cast: within the fp32 bound of the oracle's max |C|
    v = np.abs(value.reshape(-1))
    assert abs(amax - v.max()) <= 2.0 ** -20 * sabs.reshape(-1)[np.argmax(v)] + 0.0


def test_sf32_batch_equals_separate_calls():
    w = datagen.set_mx_l8_2048x2048x8192(3, 72, 80, 256)
    c, amax, idx = gu.blockscaled_gemm_amax(w["a"], w["b"], 0, w["sfa"], w["sfb"], F32)
    best = None
    for l in range(3):
        cl, al, il = gu.blockscaled_gemm_amax(w["a"][l:l + 1], w["b"][l:l + 1], 0, w["sfa"][l:l + 1],
                                              w["sfb"][l:l + 1], F32)
        compare.assert_bitwise_equal(cl[0], c[l], f"batch item {l}")
        cand = (al, -(l * 72 * 80 + il))
        best = cand if best is None or cand > best else best
    assert amax == best[0] and idx == -best[1]


def test_sf32_nan_and_empty():
    w = datagen.set_mx_l8_2048x2048x8192(2, 40, 48, 128)
    a = w["a"].copy(); a[1, 7, 3] = 0x7F
    c, amax, idx = gu.blockscaled_gemm_amax(a, w["b"], 0, w["sfa"], w["sfb"], F32)
    assert np.isnan(amax) and idx == 1 * 40 * 48 + 7 * 48 + 0
    z = np.zeros((0, 40, 128), np.uint8)
    c, amax, idx = gu.blockscaled_gemm_amax(z, np.zeros((0, 48, 128), np.uint8), 0, np.ones((0, 40, 4), np.float32),
                                            np.ones((0, 48, 4), np.float32), F32)
    assert amax == 0.0 and idx == -1


def test_sf32_amax_without_index():
    w = datagen.set_mx_l8_2048x2048x8192(2, 100, 60, 256)
    c, amax, _ = gu.blockscaled_gemm_amax(w["a"], w["b"], 0, w["sfa"], w["sfb"], F32, with_index=False)
    assert amax == float(np.max(np.abs(c.view(np.float32))))


def factors_as_read(f):
    """The factor each fp32 scale factor acts as in mm_blockscaled_gemm_amax (its contract in include/mm.h):
    only the exponent field e is read, as an E8M0 code, so x acts as 2^(e - 127): 2^floor(log2|x|) for a
    normal x whatever its sign and mantissa, 2^-127 for zero and fp32 subnormals (e = 0), and NaN for Inf and
    NaN (e = 255)."""
    e = (np.asarray(f, np.float32).view(np.uint32) >> 23) & 0xFF
    out = np.ldexp(1.0, e.astype(np.int64) - 127)
    out[e == 255] = np.nan
    return out.astype(np.float32)


def test_sf32_factors_read_by_their_exponent_field():
    """Non-power-of-two, negative, zero, subnormal, Inf and NaN fp32 factors: the GPU result equals the
    oracle's on the factors as read (2^floor(log2|x|), 2^-127 for zero, NaN for Inf / NaN), element by
    element; the factors' own values would differ by up to 2x."""
    L, M, N, K = 2, 96, 136, 512
    w = datagen.set_mx_l8_2048x2048x8192(L, M, N, K)
    g = np.random.default_rng(77)
    for key in ("sfa", "sfb"):
        f = w[key] * g.uniform(1.0, 2.0, size=w[key].shape).astype(np.float32)  # mantissas other than 1
        f = np.where(g.random(f.shape) < 0.3, -f, f).astype(np.float32)          # negative factors
        zero = g.random(f.shape) < 0.02
        f[zero] = 0.0
        f.reshape(-1)[g.choice(f.size, 5, replace=False)] = np.float32(1e-40)   # fp32 subnormals
        w[key] = f
    w["sfa"][1, 7, 3] = np.float32(np.inf)   # row 7 of item 1: NaN
    w["sfb"][0, 11, 0] = np.float32(np.nan)  # column 11 of item 0: NaN
    assert np.any(w["sfa"] < 0) and np.any(w["sfa"] == 0)
    c, amax, idx = gu.blockscaled_gemm_amax(w["a"], w["b"], 0, w["sfa"], w["sfb"], F32)
    value, sabs, bits, _, _ = oracle.blockscaled_gemm_amax(w["a"], w["b"], 0, factors_as_read(w["sfa"]),
                                                           factors_as_read(w["sfb"]), 32, F32)
    compare.check(c, value, sabs, bits, F32, "fp32 factors as read")
    cf = c.view(np.float32)
    assert np.isnan(cf[1, 7]).all() and np.isnan(cf[0, :, 11]).all() and np.isnan(amax)
    # and the factors taken at face value would not pass: the reading is what the kernel does
    v_face, s_face, _, _, _ = oracle.blockscaled_gemm_amax(w["a"], w["b"], 0, np.abs(np.nan_to_num(w["sfa"])),
                                                           np.abs(np.nan_to_num(w["sfb"])), 32, F32)
    fin = np.isfinite(cf)
    assert (np.abs(cf[fin] - v_face[fin]) > 2.0 ** -20 * s_face[fin]).mean() > 0.5


def test_sf32_e5m2_unit_scales_is_plain_gemm():
    """The cuDNN example shape (m, n, k = 512, 256, 256, sf 32, E5M2, all-ones scales)."""
    g = np.random.default_rng(0)
    a = datagen.gauss_codes(g, (1, 512, 256), 1.0, E5M2)
    b = datagen.gauss_codes(g, (1, 256, 256), 1.0, E5M2)
    w = dict(a=a, b=b, ab_fmt=E5M2, sfa=np.ones((1, 512, 8), np.float32), sfb=np.ones((1, 256, 8), np.float32))
    check_amax_case(w, F32)


@pytest.mark.parametrize("L", [2, 1], ids=["128x256", "128x128-kgroups"])
def test_production_tiles_sf32(L):
    """MX-scaled GEMM + amax at sizes that select the 128x256 tile and the
    128x128 tile with two K groups (one tile per CU: 256 of them); the
    full-size workload below selects 256x256."""
    w = datagen.set_mx_l8_2048x2048x8192(L, 2048, 2048, 1040)
    rows = sample_rows(2048, 4)
    c, amax, idx, value, sabs = check_amax_case(w, F32, rows=rows)
    cf = np.abs(c.view(np.float32).reshape(-1))
    assert amax == float(cf.max()) and idx == int(np.argmax(cf))


def test_mx_full_size():
    """L = 8, 2048 x 2048 x 8192 with fp32 factors: every output of every batch item against the oracle, the
    amax and its index against the oracle's (and bit-exact against the GPU's own C)."""
    w = datagen.set_mx_l8_2048x2048x8192()
    c, amax, idx, value, sabs = check_amax_case(w, F32)
    check_amax_index_against_oracle(idx, value, sabs)
    v = np.abs(value.reshape(-1))
    assert abs(amax - v.max()) <= 2.0 ** -20 * sabs.reshape(-1)[np.argmax(v)]
    cf = np.abs(c.view(np.float32).reshape(-1))
    assert amax == float(cf.max()) and idx == int(np.argmax(cf))


# ------------------------------------------------------------------ page-native E8M0 factors (atom layout)

def check_atom_case(w, c_type, rows=None):
    c, amax, idx = gu.blockscaled_gemm_amax_atom(w["a"], w["b"], w["ab_fmt"], w["sfa"], w["sfb"], c_type)
    value, sabs, bits, _, _ = oracle.blockscaled_gemm_amax_atom(w["a"], w["b"], w["ab_fmt"], w["sfa"], w["sfb"],
                                                                oracle.SF_E8M0, 32, c_type, rows=rows)
    cg = c if rows is None else c[:, rows]
    compare.check(cg, value, sabs, bits, c_type, "atom gemm")
    return c, amax, idx, value, sabs


def atom_padding_mask(MN, K, L, sf=32):
    """True on the storage bytes no factor uses: logical (i0, i1, i2, j0, j1, l) is storage
    [l][i2][j1][i0][i1][j0] (the page's permutation); row i0 + 32 i1 + 128 i2 and group j0 + 4 j1
    (the reading of the page's shapes) past MN or ceil(K/sf) are padding."""
    shape = oracle.sf_atom_shape(MN, K, L, sf)
    l, i2, j1, i0, i1, j0 = np.indices(shape)
    return (i0 + 32 * i1 + 128 * i2 >= MN) | (j0 + 4 * j1 >= -(-K // sf))


@pytest.mark.parametrize("L,M,N,K,c_type", [(3, 200, 136, 1024, F32), (2, 96, 200, 512, BF16),
                                            (1, 130, 70, 1008, F16), (2, 257, 129, 96, F32)])
def test_atom_against_oracle(L, M, N, K, c_type):
    w = datagen.set_mx_atom_l8_2048x2048x8192(L, M, N, K)
    c, amax, idx, value, sabs = check_atom_case(w, c_type)
    check_amax_index_against_oracle(idx, value, sabs)
    v = np.abs(value.reshape(-1))
    assert abs(amax - v.max()) <= 2.0 ** -20 * sabs.reshape(-1)[np.argmax(v)]
    if c_type == F32:  # bit-exact against the GPU's own C
        cf = np.abs(c.view(np.float32).astype(np.float64).reshape(-1))
        assert amax == float(cf.max()) and idx == int(np.argmax(cf))


@pytest.mark.parametrize("L,M,N,K", [(3, 200, 136, 1024), (1, 130, 70, 1008), (2, 2048, 2048, 1040),
                                     (1, 2048, 2048, 1040)], ids=["64x64", "64x64-ragged", "128x256",
                                                                  "128x128-kgroups"])
def test_atom_equals_fp32_factor_entry(L, M, N, K):
    """The same factors as fp32 powers of two through mm_blockscaled_gemm_amax: bitwise the same C,
    amax and index (the two entries differ only in how the factors are read)."""
    w = datagen.set_mx_atom_l8_2048x2048x8192(L, M, N, K)
    c1, a1, i1 = gu.blockscaled_gemm_amax_atom(w["a"], w["b"], 0, w["sfa"], w["sfb"], F32)
    fa = oracle.sf_atom_unpack(w["sfa"], oracle.SF_E8M0, M, K, L, 32)
    fb = oracle.sf_atom_unpack(w["sfb"], oracle.SF_E8M0, N, K, L, 32)
    c2, a2, i2 = gu.blockscaled_gemm_amax(w["a"], w["b"], 0, fa, fb, F32)
    compare.assert_bitwise_equal(c1, c2, "atom vs fp32 factors")
    assert a1 == a2 and i1 == i2


def test_atom_e5m2_operands():
    L, M, N, K = 2, 150, 90, 416
    w = datagen.set_mx_atom_l8_2048x2048x8192(L, M, N, K)
    w["a"] = datagen.gauss_codes(datagen.rng(47, 0), (L, M, K), 64.0, E5M2)
    w["b"] = datagen.gauss_codes(datagen.rng(47, 1), (L, N, K), 64.0, E5M2)
    w["ab_fmt"] = E5M2
    c, amax, idx, value, sabs = check_atom_case(w, F32)
    check_amax_index_against_oracle(idx, value, sabs)


def test_atom_padding_is_not_read():
    L, M, N, K = 2, 100, 72, 208  # 28 / 56 padding rows, group 7 of the second 4-group block unused
    w = datagen.set_mx_atom_l8_2048x2048x8192(L, M, N, K)
    c1, a1, i1 = gu.blockscaled_gemm_amax_atom(w["a"], w["b"], 0, w["sfa"], w["sfb"], F32)
    sfa, sfb = w["sfa"].copy(), w["sfb"].copy()
    sfa[atom_padding_mask(M, K, L)] = 0xFF  # NaN factors
    sfb[atom_padding_mask(N, K, L)] = 0xFF
    assert (sfa == 0xFF).sum() > 0 and (sfb == 0xFF).sum() > 0
    c2, a2, i2 = gu.blockscaled_gemm_amax_atom(w["a"], w["b"], 0, sfa, sfb, F32)
    compare.assert_bitwise_equal(c1, c2, "padding factors")
    assert a1 == a2 and i1 == i2 and not np.isnan(a2)


def test_atom_nan_factor_poisons_one_row():
    L, M, N, K = 2, 72, 80, 256
    w = datagen.set_mx_atom_l8_2048x2048x8192(L, M, N, K)
    # row 5, group 2 of item 1 (storage [l][m/128][g/4][m%32][(m/32)%4][g%4])
    w["sfa"][1, 0, 0, 5, 0, 2] = 0xFF
    c, amax, idx, value, sabs = check_atom_case(w, F32)
    cf = c.view(np.float32)
    assert np.isnan(cf[1, 5]).all() and not np.isnan(np.delete(cf.reshape(L * M, N), M + 5, axis=0)).any()
    assert np.isnan(amax) and idx == 1 * M * N + 5 * N


def test_atom_mx_full_size():
    """The MX set (L=8, 2048 x 2048 x 8192) with E8M0 atom factors, on the 256x256 tile: sampled rows
    against the oracle, the whole C bitwise against the fp32-factor entry."""
    w = datagen.set_mx_atom_l8_2048x2048x8192()
    rows = tile_rows(2048, seed=4)
    c, amax, idx, value, sabs = check_atom_case(w, F32, rows=rows)
    cf = np.abs(c.view(np.float32).reshape(-1))
    assert amax == float(cf.max()) and idx == int(np.argmax(cf))
    fa = oracle.sf_atom_unpack(w["sfa"], oracle.SF_E8M0, 2048, 8192, 8, 32)
    fb = oracle.sf_atom_unpack(w["sfb"], oracle.SF_E8M0, 2048, 8192, 8, 32)
    c2, a2, i2 = gu.blockscaled_gemm_amax(w["a"], w["b"], 0, fa, fb, F32)
    compare.assert_bitwise_equal(c, c2, "atom vs fp32 factors, full size")
    assert amax == a2 and idx == i2


# ------------------------------------------------------------------ FP4 with E4M3 factors per 16 (the page's NVFP4)

def check_nvfp4_case(w, c_type, rows=None):
    c, amax, idx = gu.blockscaled_gemm_amax_atom(w["a"], w["b"], 5, w["sfa"], w["sfb"], c_type, sf=16,
                                                 sf_type=gu.mm.MM_SF_E4M3FN)
    value, sabs, bits, _, _ = oracle.blockscaled_gemm_amax_atom(w["a"], w["b"], oracle.E2M1, w["sfa"], w["sfb"],
                                                                oracle.SF_E4M3FN, 16, c_type, rows=rows)
    cg = c if rows is None else c[:, rows]
    compare.check(cg, value, sabs, bits, c_type, "fp4 gemm, E4M3 factors")
    return c, amax, idx, value, sabs


@pytest.mark.parametrize("L,M,N,K,c_type", [
    (3, 200, 136, 1024, F32), (2, 96, 200, 512, BF16), (1, 130, 70, 992, F16), (2, 257, 129, 800, E4M3FN),
    (1, 40, 48, 32, F32)])
def test_nvfp4_against_oracle(L, M, N, K, c_type):
    w = datagen.set_nvfp4_l8_2048x2048x8192(L, M, N, K, config=30 + L)
    c, amax, idx, value, sabs = check_nvfp4_case(w, c_type)
    check_amax_index_against_oracle(idx, value, sabs)
    v = np.abs(value.reshape(-1))
    assert abs(amax - v.max()) <= 2.0 ** -20 * sabs.reshape(-1)[np.argmax(v)]
    if c_type == F32:
        cf = np.abs(c.view(np.float32).astype(np.float64).reshape(-1))
        assert amax == float(cf.max()) and idx == int(np.argmax(cf))


def test_nvfp4_signed_subnormal_and_nan_factors():
    L, M, N, K = 1, 72, 80, 256
    w = datagen.set_nvfp4_l8_2048x2048x8192(L, M, N, K, config=35)
    g = np.random.default_rng(35)
    codes = np.array([0x01, 0x07, 0x81, 0xB8, 0x7E, 0xFE], np.uint8)  # subnormals, negative, largest
    w["sfa"] = w["sfa"].copy()
    w["sfa"].reshape(-1)[g.choice(w["sfa"].size, 200, replace=False)] = g.choice(codes, 200)
    w["sfb"] = w["sfb"].copy()
    w["sfb"][0, 0, 0, 9, 0, 1] = 0x7F  # NaN factor: row 9, group 1 of B
    c, amax, idx, value, sabs = check_nvfp4_case(w, F32)
    cf = c.view(np.float32)
    assert np.isnan(cf[0, :, 9]).all() and np.isnan(amax) and idx == 9


@pytest.mark.parametrize("L", [2, 1], ids=["128x256", "128x128"])
def test_nvfp4_production_tiles(L):
    w = datagen.set_nvfp4_l8_2048x2048x8192(L, 2048, 2048, 1024, config=36)
    rows = sample_rows(2048, 4)
    c, amax, idx, value, sabs = check_nvfp4_case(w, F32, rows=rows)
    cf = np.abs(c.view(np.float32).reshape(-1))
    assert amax == float(cf.max()) and idx == int(np.argmax(cf))


def test_nvfp4_full_size():
    w = datagen.set_nvfp4_l8_2048x2048x8192()
    check_nvfp4_case(w, F32, rows=tile_rows(2048, seed=5))


# ------------------------------------------------------------------ FP4 (E2M1) C with FP4 operands

def unpack_e2m1(packed, N):
    """[..., ceil(N/2)] bytes -> [..., N] codes, low nibble first."""
    p = np.asarray(packed, np.uint8)
    codes = np.stack([p & 15, p >> 4], axis=-1).reshape(*p.shape[:-1], 2 * p.shape[-1])
    return codes[..., :N]


@pytest.mark.parametrize("L,M,N,K,sf,e4m3", [
    (2, 96, 136, 512, 32, False),   # N % 4 == 0: 2-byte stores
    (1, 130, 71, 992, 16, False),   # odd N: the last byte's high nibble
    (2, 64, 99, 256, 16, True),     # N % 4 == 3 with E4M3 factors
    (1, 200, 2, 64, 32, False),     # two columns: one byte per row
])
def test_fp4_c_output(L, M, N, K, sf, e4m3):
    w = (datagen.set_nvfp4_l8_2048x2048x8192(L, M, N, K, config=70) if e4m3 else
         datagen.set_fp4_l8_2048x2048x8192(L, M, N, K, sf, config=70))
    sft = oracle.SF_E4M3FN if e4m3 else oracle.SF_E8M0
    # A's factors lowered so that the outputs spread over the whole E2M1 range, saturation included
    s = w["sfa"].astype(np.int64)
    if e4m3:  # exponent field - 6 (at least 1)
        w["sfa"] = ((np.maximum((s >> 3) - 6, 1) << 3) | (s & 7)).astype(np.uint8)
    else:  # factor / 2^9
        w["sfa"] = np.clip(s - 9, 1, 254).astype(np.uint8)
    es = -(-N // 2)
    ta, tb = gu.dev_u8(w["a"]), gu.dev_u8(w["b"])
    tsa, tsb = gu.dev_u8(w["sfa"]), gu.dev_u8(w["sfb"])
    tc = gu.torch.full((L * M * es,), 0x5A, dtype=gu.torch.uint8, device=gu.DEV)
    tam = gu.torch.zeros((1,), dtype=gu.torch.float32, device=gu.DEV)
    st = gu.mm.mm_blockscaled_gemm_amax_atom(M, N, K, L, ta.data_ptr(), tb.data_ptr(), gu.mm.MM_F4_E2M1,
                                             tsa.data_ptr(), tsb.data_ptr(),
                                             gu.mm.MM_SF_E4M3FN if e4m3 else gu.mm.MM_SF_E8M0, 16 if e4m3 else sf,
                                             tc.data_ptr(), gu.mm.MM_F4_E2M1, tam.data_ptr(), 0, gu.stream())
    assert st == gu.mm.MM_OK, (st, gu.mm.mm_last_error())
    gu.torch.cuda.synchronize()
    packed = tc.cpu().numpy().reshape(L, M, es)
    if N % 2:
        assert np.all(packed[..., -1] >> 4 == 0)  # the pad nibble
    value, sabs, bits, _, _ = oracle.blockscaled_gemm_amax_atom(w["a"], w["b"], oracle.E2M1, w["sfa"], w["sfb"],
                                                                sft, 16 if e4m3 else sf, 5)
    g = unpack_e2m1(packed, N)
    assert np.any(g & 7 == 7) and np.any(g & 7 == 1)  # saturated and small values both present
    compare.check(g, value, sabs, unpack_e2m1(bits, N), 5, "fp4 C")
    v = np.abs(value.reshape(-1))
    assert abs(float(tam.item()) - v.max()) <= 2.0 ** -20 * sabs.reshape(-1)[np.argmax(v)]


# ------------------------------------------------------------------ grouped GEMM (GroupedGemmFwdOp, NT, FP8)

def check_grouped(w, d_type, fast=False, scale_result=None, rows=None, fmt=(E4M3FN, E4M3FN)):
    gpu = gu.scaled_gemm_grouped(w["a"], fmt[0], w["b"], fmt[1], w["sizes"], w["offsets"], w["scale_a"],
                                 w["scale_b"], d_type, scale_result=scale_result, fast=fast)
    value, sabs, bits = oracle.grouped_gemm(w["a"], fmt[0], w["b"], fmt[1], w["sizes"], w["offsets"], w["scale_a"],
                                            w["scale_b"], d_type, scale_result=scale_result)
    r = np.arange(w["a"].shape[0]) if rows is None else rows
    compare.check(gpu[r], value[r], sabs[r], bits[r], d_type, "grouped gemm")
    return gpu


@pytest.mark.parametrize("G,batch_sum,N,K,empty,fast,d_type", [
    (5, 300, 136, 256, 1, False, BF16),     # ragged groups, one empty, partial tiles (64x64 tiles)
    (3, 1000, 200, 1040, 0, True, F32),     # K tail
    (100, 1500, 64, 128, 20, False, F16),   # more than 64 groups (two rounds of the wave scan), many empty
    (8, 4096, 1024, 512, 2, False, BF16),   # 128x128 tiles, one per CU (two K groups)
    (8, 8192, 2048, 512, 0, True, E4M3FN),  # 128x128 tiles, two per CU; FP8 out
])
def test_grouped_against_oracle(G, batch_sum, N, K, empty, fast, d_type):
    w = datagen.set_grouped_8x8192x4096x4096(G, batch_sum, N, K, empty, config=10 + G)
    sr = 1.0 / 16 if d_type == E4M3FN else None
    rows = None if batch_sum <= 1500 else sample_rows(batch_sum, 16, seed=G)
    check_grouped(w, d_type, fast=fast, scale_result=sr, rows=rows)


def test_grouped_e5m2_and_single_group():
    w = datagen.set_grouped_8x8192x4096x4096(1, 257, 96, 384, 0, config=21)
    w["a"] = datagen.gauss_codes(datagen.rng(21, 4), w["a"].shape, 64.0, E5M2)
    check_grouped(w, F32, fmt=(E5M2, E4M3FN))


def test_grouped_rows_of_no_group_are_not_written():
    # sizes that cover only part of the rows (the page makes this the caller's error): the covered rows are
    # right and the others keep their previous contents
    w = datagen.set_grouped_8x8192x4096x4096(4, 400, 72, 256, 0, config=22)
    w["sizes"] = np.array([50, 0, 30, 100], np.int32)
    w["offsets"] = np.array([0, 60, 60, 250], np.int32)
    gpu = gu.scaled_gemm_grouped(w["a"], E4M3FN, w["b"], E4M3FN, w["sizes"], w["offsets"], w["scale_a"],
                                 w["scale_b"], BF16)
    for g, (sz, of) in enumerate(zip(w["sizes"], w["offsets"])):
        if sz == 0:
            continue
        value, sabs, bits = oracle.scaled_gemm(w["a"][of:of + sz], E4M3FN, w["b"][g], E4M3FN, w["scale_a"], 0,
                                               w["scale_b"], 0, BF16)
        compare.check(gpu[of:of + sz], value, sabs, bits, BF16, f"group {g}")
    covered = np.zeros(400, bool)
    for sz, of in zip(w["sizes"], w["offsets"]):
        covered[of:of + sz] = True
    assert np.all(gpu[~covered] == 0x5A5A)


def test_grouped_full_size():
    """The grouped bench workload: 8 groups, 8192 packed rows, N = K = 4096, slow, bf16 out; sampled rows."""
    w = datagen.set_grouped_8x8192x4096x4096()
    check_grouped(w, BF16, rows=tile_rows(8192, seed=6))


# ------------------------------------------------------------------ FP4 (E2M1) operands, page-native factors

def check_fp4_case(w, c_type, rows=None):
    c, amax, idx = gu.blockscaled_gemm_amax_atom(w["a"], w["b"], 5, w["sfa"], w["sfb"], c_type, sf=w["sf_vec"])
    value, sabs, bits, _, _ = oracle.blockscaled_gemm_amax_atom(w["a"], w["b"], oracle.E2M1, w["sfa"], w["sfb"],
                                                                oracle.SF_E8M0, w["sf_vec"], c_type, rows=rows)
    cg = c if rows is None else c[:, rows]
    compare.check(cg, value, sabs, bits, c_type, "fp4 gemm")
    return c, amax, idx, value, sabs


@pytest.mark.parametrize("L,M,N,K,sf,c_type", [
    (3, 200, 136, 1024, 32, F32), (2, 96, 200, 512, 16, BF16), (1, 130, 70, 992, 16, F16),
    (2, 257, 129, 800, 32, F32),  # the last step's second factor block lies past the tensor's
    (1, 100, 72, 256, 32, E4M3FN), (2, 64, 96, 1056, 16, E5M2), (1, 40, 48, 32, 16, F32)])
def test_fp4_against_oracle(L, M, N, K, sf, c_type):
    w = datagen.set_fp4_l8_2048x2048x8192(L, M, N, K, sf)
    c, amax, idx, value, sabs = check_fp4_case(w, c_type)
    check_amax_index_against_oracle(idx, value, sabs)
    v = np.abs(value.reshape(-1))
    assert abs(amax - v.max()) <= 2.0 ** -20 * sabs.reshape(-1)[np.argmax(v)]
    if c_type == F32:
        cf = np.abs(c.view(np.float32).astype(np.float64).reshape(-1))
        assert amax == float(cf.max()) and idx == int(np.argmax(cf))


@pytest.mark.parametrize("L,sf", [(2, 32), (1, 16)], ids=["128x256", "128x128"])
def test_fp4_production_tiles(L, sf):
    w = datagen.set_fp4_l8_2048x2048x8192(L, 2048, 2048, 1024, sf)
    rows = sample_rows(2048, 4)
    c, amax, idx, value, sabs = check_fp4_case(w, F32, rows=rows)
    cf = np.abs(c.view(np.float32).reshape(-1))
    assert amax == float(cf.max()) and idx == int(np.argmax(cf))


def test_fp4_worst_case_factor_spread():
    """Factors 2^-8 and 2^4 alternating per group of 32 on both operands (products 2^24 apart inside one
    scaled MFMA instruction), sf 32, every output against the oracle."""
    L, M, N, K = 2, 200, 136, 2048
    w = datagen.set_fp4_l8_2048x2048x8192(L, M, N, K, 32, config=71)
    for key in ("sfa", "sfb"):
        sf = w[key].copy()
        sf[..., 0::2] = 127 - 8  # storage [l][mn/128][g/4][mn%32][(mn/32)%4][g%4]: g even at j0 = 0, 2
        sf[..., 1::2] = 127 + 4
        w[key] = sf
    c, amax, idx, value, sabs = check_fp4_case(w, F32)
    check_amax_index_against_oracle(idx, value, sabs)


def test_fp4_nan_and_extreme_factors():
    """E8M0 NaN (0xFF) poisons its row; factors at 2^-127 and 2^64 elsewhere stay within the bound."""
    L, M, N, K = 1, 96, 80, 512
    w = datagen.set_fp4_l8_2048x2048x8192(L, M, N, K, 32, config=72)
    w["sfa"] = w["sfa"].copy()
    w["sfa"][0, 0, 0, 7, 0, 1] = 0xFF  # row 7, group 1: NaN
    w["sfb"] = w["sfb"].copy()
    w["sfb"][0, 0, 1, 3, 0, 2] = 0x00  # column 3, group 6: 2^-127
    w["sfb"][0, 0, 0, 9, 0, 0] = 127 + 64  # column 9, group 0: 2^64
    c, amax, idx, value, sabs = check_fp4_case(w, F32)
    cf = c.view(np.float32)
    assert np.isnan(cf[0, 7]).all() and np.isnan(amax)


def test_fp4_padding_is_not_read():
    L, M, N, K, sf = 2, 100, 72, 224, 16  # 14 groups: two unused in the last 4-group block
    w = datagen.set_fp4_l8_2048x2048x8192(L, M, N, K, sf)
    c1, a1, i1 = gu.blockscaled_gemm_amax_atom(w["a"], w["b"], 5, w["sfa"], w["sfb"], F32, sf=sf)
    sfa, sfb = w["sfa"].copy(), w["sfb"].copy()
    sfa[atom_padding_mask(M, K, L, sf)] = 0xFF
    sfb[atom_padding_mask(N, K, L, sf)] = 0xFF
    c2, a2, i2 = gu.blockscaled_gemm_amax_atom(w["a"], w["b"], 5, sfa, sfb, F32, sf=sf)
    compare.assert_bitwise_equal(c1, c2, "padding factors")
    assert a1 == a2 and i1 == i2 and not np.isnan(a2)


def test_fp4_full_size():
    """L=8, 2048 x 2048 x 8192 FP4 with factors per 32 (the FP4 bench workload): sampled rows."""
    w = datagen.set_fp4_l8_2048x2048x8192()
    rows = tile_rows(2048, seed=7)
    c, amax, idx, value, sabs = check_fp4_case(w, F32, rows=rows)
    cf = np.abs(c.view(np.float32).reshape(-1))
    assert amax == float(cf.max()) and idx == int(np.argmax(cf))


# ------------------------------------------------------------------ K tail (K = 8200), FP8 / f16 out: 8192 x 28672 x 8200

def test_k_tail_small():
    for d, dt, sr in ((datagen.set_e4m3_out_8192x28672x8200(200, 300, 8200), E4M3FN, np.float32(1 / 16)),
                      (datagen.set_e5m2_f16_8192x28672x8200(200, 300, 8200), F16, None)):
        check_gemm(d, 0, 0, dt, False, scale_result=sr, what=f"K tail small {DT_NAME[dt]}")


def test_e4m3_out_saturation_edge():
    d = datagen.set_e4m3_out_8192x28672x8200(96, 160, 8200)
    d["scale_a"] = np.float32(1.0); d["scale_b"] = np.float32(1.0)
    _, gpu, value, _ = check_gemm(d, 0, 0, E4M3FN, False, scale_result=np.float32(1 / 16), what="saturation")
    assert np.mean((gpu & 0x7F) == 0x7E) > 0.9       # almost every output saturates


@pytest.mark.parametrize("which", ["5a", "5b"])
def test_k_tail_full_size(which):
    if which == "5a":
        d, dt, sr = datagen.set_e4m3_out_8192x28672x8200(), E4M3FN, np.float32(1 / 16)
    else:
        d, dt, sr = datagen.set_e5m2_f16_8192x28672x8200(), F16, None
    rows = tile_rows(8192, seed=8 if which == "5a" else 9)
    check_gemm(d, 0, 0, dt, False, rows=rows, scale_result=sr, what=f"K tail 8192x28672x8200 ({which}) full size")


# ------------------------------------------------------------------ bias (TileOPs GemmFP8FwdOp, forward)

def _bias_bits(rng, N, d_type):
    x = rng.normal(0, 16, size=N).astype(np.float32)
    if d_type == BF16:
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    if d_type == F16:
        return x.astype(np.float16).view(np.uint16)
    return x.view(np.uint32)


def _bias_values(bits, d_type):
    if d_type == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if d_type == F16:
        return bits.view(np.float16).astype(np.float64)
    return bits.view(np.float32).astype(np.float64)


@pytest.mark.parametrize("d_type", [BF16, F16, F32], ids=["bf16", "f16", "f32"])
@pytest.mark.parametrize("M,N,K,fast", [(16, 4100, 1032, False),    # skinny
                                        (64, 4100, 1032, True),      # skinny, sixteen waves of two steps
                                        (200, 4096, 1032, True),     # K split
                                        (1000, 1030, 1032, False),   # 128x128 tiles, ragged N and K
                                        (2048, 2048, 520, True)])    # 256x256 / 128x256 tiles
def test_bias_per_tensor(M, N, K, fast, d_type):
    g = np.random.default_rng(M + N + d_type)
    a = datagen.gauss_codes(g, (M, K), 64.0)
    b = datagen.gauss_codes(g, (N, K), 64.0)
    bias_bits = _bias_bits(g, N, d_type)
    gpu = gu.scaled_gemm_bias(a, E4M3FN, b, E4M3FN, K, 0.5, 0, 0.25, 0, bias_bits, d_type, fast=fast)
    rows = sample_rows(M, 8)
    value, sabs, bits = oracle.scaled_gemm(a, E4M3FN, b, E4M3FN, np.float32(0.5), 0, np.float32(0.25), 0, d_type,
                                           rows=rows, bias=_bias_values(bias_bits, d_type))
    compare.check(gpu[rows], value, sabs, bits, d_type, f"bias {M}x{N}x{K} fast={fast}")


@pytest.mark.parametrize("sb_mode", [1, 2], ids=["1x128", "128x128"])
def test_bias_block_scaled(sb_mode):
    M, N, K = 1024, 2056, 1032
    g = np.random.default_rng(40 + sb_mode)
    a = datagen.gauss_codes(g, (M, K), 64.0)
    b = datagen.gauss_codes(g, (N, K), 64.0)
    kb = -(-K // 128)
    sa = datagen.log_uniform_scales(g, (M, kb))
    sb = datagen.log_uniform_scales(g, (N if sb_mode == 1 else -(-N // 128), kb))
    bias_bits = _bias_bits(g, N, BF16)
    gpu = gu.scaled_gemm_bias(a, E4M3FN, b, E4M3FN, K, sa, 1, sb, sb_mode, bias_bits, BF16)
    rows = sample_rows(M, 8)
    value, sabs, bits = oracle.scaled_gemm(a, E4M3FN, b, E4M3FN, sa, 1, sb, sb_mode, BF16, rows=rows,
                                           bias=_bias_values(bias_bits, BF16))
    compare.check(gpu[rows], value, sabs, bits, BF16, f"bias block sb={sb_mode}")


# block scaling with a 128x128 scale_b and a bias on the 256x256 row-chunk tiles, alone and in the split plan
@pytest.mark.parametrize("M,N,K", [(4096, 4096, 520), (4096, 14336, 264)], ids=["256x256", "split"])
def test_bias_block_scaled_256(M, N, K):
    g = np.random.default_rng(M + N + K)
    a = datagen.gauss_codes(g, (M, K), 64.0)
    b = datagen.gauss_codes(g, (N, K), 64.0)
    kb = -(-K // 128)
    sa = datagen.log_uniform_scales(g, (M, kb))
    sb = datagen.log_uniform_scales(g, (-(-N // 128), kb))
    bias_bits = _bias_bits(g, N, F16)
    gpu = gu.scaled_gemm_bias(a, E4M3FN, b, E4M3FN, K, sa, 1, sb, 2, bias_bits, F16)
    rows = tile_rows(M, band=256, edge=8)
    value, sabs, bits = oracle.scaled_gemm(a, E4M3FN, b, E4M3FN, sa, 1, sb, 2, F16, rows=rows,
                                           bias=_bias_values(bias_bits, F16))
    compare.check(gpu[rows], value, sabs, bits, F16, f"bias block 128x128 {M}x{N}x{K}")


# ------------------------------------------------------------------ batched (TileOPs BmmFP8FwdOp)

@pytest.mark.parametrize("L,M,N,K,fast,d_type,fmt", [
    (3, 100, 300, 520, False, BF16, E4M3FN),     # 64x64 tiles, ragged
    (8, 64, 64, 256, True, F32, E4M3FN),         # small items: tiles, not the skinny kernel
    (16, 256, 1024, 136, True, BF16, E4M3FN),    # 128x128 tiles, one per CU: K groups
    (4, 512, 1024, 1032, False, F16, E5M2),      # 128x128 tiles, two per CU, ragged K
    (2, 2048, 1024, 264, True, BF16, E4M3FN),    # 256x256 tiles
    (3, 70, 200, 136, False, E4M3FN, E4M3FN),    # FP8 out with scale_result
    (8, 2048, 1024, 512, False, BF16, E4M3FN),   # slow, 256x256 tiles (row-chunk loop), padded rows
    (2, 2048, 14336, 136, False, F16, E4M3FN),   # slow, 256x256 tiles on 12288 columns, 128x128 on the rest
])
def test_batched_per_item_against_oracle(L, M, N, K, fast, d_type, fmt):
    g = np.random.default_rng(L * 1000 + M)
    a = np.stack([datagen.gauss_codes(g, (M, K), 64.0) for _ in range(L)]) if fmt == E4M3FN else \
        g.integers(0, 256, size=(L, M, K)).astype(np.uint8) & 0xFB
    b = np.stack([datagen.gauss_codes(g, (N, K), 64.0) for _ in range(L)]) if fmt == E4M3FN else \
        g.integers(0, 256, size=(L, N, K)).astype(np.uint8) & 0xFB
    sr = 0.0625 if d_type in (E4M3FN, E5M2) else None
    gpu = gu.scaled_gemm_batched(a, fmt, b, fmt, K, 0.5, 0.25, d_type, scale_result=sr, fast=fast,
                                 pad_a=32, pad_b=16, pad_d=8)
    rows = sample_rows(M, 6)
    for l in range(L):
        value, sabs, bits = oracle.scaled_gemm(a[l], fmt, b[l], fmt, np.float32(0.5), 0, np.float32(0.25), 0,
                                               d_type, scale_result=sr, rows=rows)
        compare.check(gpu[l][rows], value, sabs, bits, d_type, f"batched item {l} of {L}: {M}x{N}x{K}")


# ------------------------------------------------------------------ seeded random shapes, newer entries

def random_shape(seed, k_mult):
    g = np.random.default_rng(1000 + seed)
    L = int(g.integers(1, 4))
    M, N = (int(x) for x in g.integers(1, 300, size=2))
    K = int(g.integers(1, 24)) * k_mult
    return L, M, N, K


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_page_native_factors(seed):
    L, M, N, K = random_shape(seed, 16)
    w = datagen.set_mx_atom_l8_2048x2048x8192(L, M, N, K)
    c, amax, idx, value, sabs = check_atom_case(w, (F32, BF16, F16)[seed % 3])
    check_amax_index_against_oracle(idx, value, sabs)


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_fp4(seed):
    L, M, N, K = random_shape(seed + 10, 32)
    if seed % 2:
        w = datagen.set_nvfp4_l8_2048x2048x8192(L, M, N, K, config=50 + seed)
        c, amax, idx, value, sabs = check_nvfp4_case(w, (F32, BF16, E4M3FN)[seed % 3])
    else:
        w = datagen.set_fp4_l8_2048x2048x8192(L, M, N, K, 16 if seed % 4 else 32, config=50 + seed)
        c, amax, idx, value, sabs = check_fp4_case(w, (F32, F16, E5M2)[seed % 3])
    check_amax_index_against_oracle(idx, value, sabs)


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_grouped(seed):
    g = np.random.default_rng(2000 + seed)
    G = int(g.integers(1, 20))
    batch_sum = int(g.integers(1, 600))
    N, K = int(g.integers(1, 300)), int(g.integers(1, 38)) * 16  # group strides N K bytes 16-byte aligned
    w = datagen.set_grouped_8x8192x4096x4096(G, batch_sum, N, K, empty=min(G - 1, int(g.integers(0, 3))),
                                             config=60 + seed)
    check_grouped(w, (BF16, F32, E4M3FN, F16, E5M2, BF16)[seed], fast=bool(seed % 2),
                  scale_result=0.0625 if seed in (2, 4) else None)


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes_scaled_gemm(seed):
    """mm_scaled_gemm on seeded random M, N, K with padded pitches, every scale mode, output type and
    accumulation; M up to 1500 so that the skinny, K-split and tile kernels all take part."""
    g = np.random.default_rng(3000 + seed)
    M = int(g.choice([int(g.integers(1, 65)), int(g.integers(65, 400)), int(g.integers(400, 1500))]))
    N = int(g.integers(1, 700))
    K = int(g.integers(1, 900))
    lda = (K + 7) // 8 * 8 + 8 * int(g.integers(0, 3))
    ldb = (K + 7) // 8 * 8 + 8 * int(g.integers(0, 3))
    fa, fb = (E4M3FN, E4M3FN) if seed % 3 else (E5M2, E4M3FN)
    a = np.full((M, lda), 0x7F, np.uint8)  # NaN codes in the padding: never read
    b = np.full((N, ldb), 0x7F, np.uint8)
    a[:, :K] = datagen.gauss_codes(g, (M, K), 64.0, fa)
    b[:, :K] = datagen.gauss_codes(g, (N, K), 64.0, fb)
    d_type = (F32, BF16, F16, E4M3FN, E5M2, BF16, F32, F16)[seed]
    sr = 1.0 / 64 if d_type in (E4M3FN, E5M2) else None
    kb = -(-K // 128)
    if seed % 4 == 3:  # block scales: 1x128 a, 1x128 or 128x128 b
        sa_mode, sb_mode = 1, (1 if seed % 8 == 3 else 2)
        sa = datagen.pow2_scales(g, (M, kb))
        sb = datagen.pow2_scales(g, (N if sb_mode == 1 else -(-N // 128), kb))
        sr = None if d_type not in (E4M3FN, E5M2) else sr
    else:
        sa_mode = sb_mode = 0
        sa, sb = np.float32(2.0 ** -5), np.float32(0.75)
    d = dict(a=a, b=b, K=K, a_fmt=fa, b_fmt=fb, scale_a=sa, scale_b=sb)
    rows = None if M <= 400 else sample_rows(M, 16, seed=seed)
    check_gemm(d, sa_mode, sb_mode, d_type, bool(seed % 2), rows=rows, scale_result=sr,
               what=f"random M={M} N={N} K={K} lda={lda} ldb={ldb}", ldd=N + 4 * (seed % 3))
