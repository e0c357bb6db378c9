"""Pins of the oracle's scaled GEMM and block-scaled GEMM + amax (CPU).

Independent references used here: exact rational arithmetic (fractions) on
values decoded by torch, numpy's float64 matmul (exact for E4M3 sums), numpy
float32 arithmetic, numpy argmax, and closed forms.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3FN, E5M2, F32, BF16, F16, SCALE_TENSOR, SCALE_1x128, SCALE_128x128
from oracle import ACC_EXACT, ACC_F32_CHUNKS
import datagen

TDT = {E4M3FN: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def tdecode(codes, fmt):
    """Decoded values through torch's own float8 dtype (not the oracle's decoder)."""
    return torch.from_numpy(np.ascontiguousarray(codes)).view(TDT[fmt]).to(torch.float64).numpy()


def finite_random_codes(rng, shape, fmt):
    fin = datagen.finite_codes(fmt)
    return fin[rng.integers(0, fin.size, size=shape)].astype(np.uint8)


def exact_gemm(a, a_fmt, b, b_fmt, sa_of, sb_of, K):
    """sum_k (a*sa)(b*sb) in exact rationals; sa_of(m,k), sb_of(n,k) give the scales."""
    A = tdecode(a[:, :K], a_fmt)
    B = tdecode(b[:, :K], b_fmt)
    M, N = A.shape[0], B.shape[0]
    out = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Fraction(A[m, k]) * Fraction(sa_of(m, k)) * Fraction(B[n, k]) * Fraction(sb_of(n, k))
            out[m, n] = s
    return out


# ------------------------------------------------------------------ brute force

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 17), (3, 2, 128), (5, 4, 129), (2, 2, 300), (16, 17, 16)])
@pytest.mark.parametrize("fa,fb", [(E4M3FN, E4M3FN), (E5M2, E5M2), (E4M3FN, E5M2)])
def test_per_tensor_exact_brute_force(M, N, K, fa, fb):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    a = finite_random_codes(rng, (M, K), fa)
    b = finite_random_codes(rng, (N, K), fb)
    sa, sb = np.float32(0.37), np.float32(-1.75)
    value, sabs, _ = oracle.scaled_gemm(a, fa, b, fb, sa, SCALE_TENSOR, sb, SCALE_TENSOR, F32)
    ex = exact_gemm(a, fa, b, fb, lambda m, k: 1, lambda n, k: 1, K)
    for m in range(M):
        for n in range(N):
            want = ex[m, n] * Fraction(float(sa)) * Fraction(float(sb))
            # E4M3 x E4M3 sums are exact in float64; any pair is within float64 rounding
            tol = 0 if (fa, fb) == (E4M3FN, E4M3FN) else 2.0 ** -45 * sabs[m, n]
            assert abs(Fraction(value[m, n]) - want) <= Fraction(tol) + Fraction(abs(float(want))) * Fraction(2.0 ** -52)


@pytest.mark.parametrize("sb_mode", [SCALE_1x128, SCALE_128x128])
@pytest.mark.parametrize("M,N,K", [(3, 5, 129), (2, 130, 260), (4, 3, 1)])
def test_block_scaled_brute_force(M, N, K, sb_mode):
    rng = np.random.default_rng(7 + M + N + K)
    a = finite_random_codes(rng, (M, K), E4M3FN)
    b = finite_random_codes(rng, (N, K), E4M3FN)
    kb = -(-K // 128)
    sa = datagen.log_uniform_scales(rng, (M, kb))
    nb = N if sb_mode == SCALE_1x128 else -(-N // 128)
    sb = datagen.log_uniform_scales(rng, (nb, kb))
    value, sabs, _ = oracle.scaled_gemm(a, E4M3FN, b, E4M3FN, sa, SCALE_1x128, sb, sb_mode, BF16)
    sb_of = (lambda n, k: float(sb[n, k // 128])) if sb_mode == SCALE_1x128 else (lambda n, k: float(sb[n // 128, k // 128]))
    ex = exact_gemm(a, E4M3FN, b, E4M3FN, lambda m, k: float(sa[m, k // 128]), sb_of, K)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(value[m, n]) - ex[m, n]) <= Fraction(2.0 ** -48) * Fraction(sabs[m, n])


def test_sum_abs_is_sum_of_term_magnitudes():
    rng = np.random.default_rng(3)
    a = finite_random_codes(rng, (4, 200), E4M3FN)
    b = finite_random_codes(rng, (6, 200), E4M3FN)
    _, sabs, _ = oracle.scaled_gemm(a, E4M3FN, b, E4M3FN, np.float32(2), 0, np.float32(-0.5), 0, F32)
    A, B = tdecode(a, E4M3FN), tdecode(b, E4M3FN)
    assert np.array_equal(sabs, np.abs(A) @ np.abs(B).T * 1.0)


# ------------------------------------------------------------------ library cross-check

@pytest.mark.parametrize("M,N,K", [(64, 48, 4096), (33, 70, 1000)])
def test_e4m3_exact_equals_numpy_matmul(M, N, K):
    """Every partial sum of E4M3 products is exact in float64, so any summation
    order (BLAS's included) gives the same bits."""
    d = datagen.set_256_cubed(M, N, K)
    value, _, _ = oracle.scaled_gemm(d["a"], E4M3FN, d["b"], E4M3FN, d["scale_a"], 0, d["scale_b"], 0, F32)
    A, B = tdecode(d["a"], E4M3FN), tdecode(d["b"], E4M3FN)
    want = (A @ B.T) * np.float64(d["scale_a"]) * np.float64(d["scale_b"])
    assert np.array_equal(value.view(np.uint64), want.view(np.uint64))


def test_output_bits_are_value_rounded_once():
    d = datagen.set_256_cubed(16, 24, 512)
    for dt in (F32, BF16, F16, E4M3FN, E5M2):
        value, _, bits = oracle.scaled_gemm(d["a"], E4M3FN, d["b"], E4M3FN, d["scale_a"], 0, d["scale_b"], 0, dt,
                                            scale_result=np.float32(0.01))
        assert np.array_equal(bits, oracle.round_to(value, dt)), dt


def test_scale_result_only_for_fp8_outputs():
    d = datagen.set_256_cubed(8, 8, 256)
    v32, _, _ = oracle.scaled_gemm(d["a"], 0, d["b"], 0, d["scale_a"], 0, d["scale_b"], 0, F32, scale_result=np.float32(0.0625))
    v8, _, _ = oracle.scaled_gemm(d["a"], 0, d["b"], 0, d["scale_a"], 0, d["scale_b"], 0, E4M3FN, scale_result=np.float32(0.0625))
    vn, _, _ = oracle.scaled_gemm(d["a"], 0, d["b"], 0, d["scale_a"], 0, d["scale_b"], 0, E4M3FN, scale_result=None)
    assert np.array_equal(v8, v32 * 0.0625)
    assert np.array_equal(vn, v32)


# ------------------------------------------------------------------ closed forms

def test_closed_forms():
    K = 384
    a = np.zeros((4, K), np.uint8)
    b = np.zeros((4, K), np.uint8)
    a[0] = 0x7E; b[0] = 0x7E                        # 448 * 448 per term
    a[1] = 0x7E; a[1, 1::2] = 0xFE; b[1] = 0x7E     # alternating +-448 against +448
    a[2] = 0x01; b[2] = 0x01                        # 2^-9 * 2^-9 per term
    a[3] = 0x80                                     # all -0
    value, _, bits = oracle.scaled_gemm(a, E4M3FN, b, E4M3FN, np.float32(1), 0, np.float32(1), 0, F32)
    assert value[0, 0] == K * 200704.0
    assert value[1, 1] == 0.0 and np.signbit(value[1, 1]) == False
    assert value[2, 2] == K * 2.0 ** -18
    assert np.all(value[3] == 0) and not np.any(np.signbit(value[3]))   # chains start from +0
    assert int(bits[3, 0]) == 0


def test_identity_and_one_hot():
    rng = np.random.default_rng(5)
    K = 130
    b = finite_random_codes(rng, (9, K), E4M3FN)
    eye = np.zeros((K, K), np.uint8)
    eye[np.arange(K), np.arange(K)] = 0x38            # 1.0 in E4M3
    value, _, _ = oracle.scaled_gemm(eye, E4M3FN, b, E4M3FN, np.float32(1), 0, np.float32(1), 0, F32)
    assert np.array_equal(value, tdecode(b, E4M3FN).T)
    # one-hot with a power-of-two scale: a single product
    a = np.zeros((1, K), np.uint8)
    a[0, 77] = 0x40                                   # 2.0 (0 1000 000)
    value, _, _ = oracle.scaled_gemm(a, E4M3FN, b, E4M3FN, np.float32(0.25), 0, np.float32(4), 0, F32)
    assert np.array_equal(value[0], tdecode(b, E4M3FN)[:, 77] * 2.0)


def test_zero_k_and_zero_sign():
    a = np.zeros((2, 0), np.uint8)
    b = np.zeros((3, 0), np.uint8)
    v, _, bits = oracle.scaled_gemm(a, 0, b, 0, np.float32(1), 0, np.float32(1), 0, F32)
    assert np.all(bits == 0)
    v, _, bits = oracle.scaled_gemm(a, 0, b, 0, np.float32(-1), 0, np.float32(1), 0, F32)
    assert np.all(bits == 0x80000000)                 # (+0) * (-1) = -0


def test_power_of_two_scale_change_is_exact():
    d = datagen.set_256_cubed(20, 20, 700)
    v1, _, _ = oracle.scaled_gemm(d["a"], 0, d["b"], 0, np.float32(0.75), 0, np.float32(3), 0, F32)
    v2, _, _ = oracle.scaled_gemm(d["a"], 0, d["b"], 0, np.float32(1.5), 0, np.float32(3), 0, F32)
    assert np.array_equal(v2, 2 * v1)


def test_unit_block_scales_equal_per_tensor():
    d = datagen.set_256_cubed(10, 140, 300)
    kb = 3
    v_t, _, _ = oracle.scaled_gemm(d["a"], 0, d["b"], 0, np.float32(1), 0, np.float32(1), 0, F32)
    v_b, _, _ = oracle.scaled_gemm(d["a"], 0, d["b"], 0, np.ones((10, kb), np.float32), 1,
                                   np.ones((2, kb), np.float32), 2, F32)
    assert np.array_equal(v_t, v_b)


def test_block_scale_on_one_block_scales_that_block_only():
    """Scaling sa[m, kb] by 2 equals doubling the decoded a[m, k] of that block:
    the result moves by exactly that block's contribution."""
    d = datagen.set_256_cubed(6, 5, 384)
    sa = np.ones((6, 3), np.float32)
    sb = np.ones((1, 3), np.float32)
    v0, _, _ = oracle.scaled_gemm(d["a"], 0, d["b"], 0, sa, 1, sb, 2, F32)
    sa2 = sa.copy(); sa2[2, 1] = 2.0
    v1, _, _ = oracle.scaled_gemm(d["a"], 0, d["b"], 0, sa2, 1, sb, 2, F32)
    A, B = tdecode(d["a"], E4M3FN), tdecode(d["b"], E4M3FN)
    blk = A[2, 128:256] @ B[:, 128:256].T
    assert np.array_equal(v1[2] - v0[2], blk)
    assert np.array_equal(np.delete(v1, 2, 0), np.delete(v0, 2, 0))


# ------------------------------------------------------------------ non-finite inputs

def test_non_finite_inputs_follow_ieee():
    K = 4
    a = np.full((4, K), 0x38, np.uint8)   # 1.0
    b = np.full((4, K), 0x3C, np.uint8)   # 1.0 in E5M2
    a[0, 1] = 0x7F                        # E4M3 NaN -> NaN
    b[1, 2] = 0x7C                        # E5M2 +Inf against a 1.0 -> +Inf
    a[2, 3] = 0x00; b[2, 3] = 0x7C        # 0 * Inf -> NaN
    b[3, 0] = 0x7C; b[3, 1] = 0xFC        # +Inf + -Inf -> NaN
    v, _, bits = oracle.scaled_gemm(a, E4M3FN, b, E5M2, np.float32(1), 0, np.float32(1), 0, F32)
    assert np.all(np.isnan(v[0]))
    assert v[0, 1] != v[0, 1] and v[1, 1] == np.inf
    assert np.isnan(v[2, 2]) and np.isnan(v[3, 3])
    assert int(bits[0, 0]) == 0x7FFFFFFF and int(bits[1, 1]) == 0x7F800000
    _, _, b8 = oracle.scaled_gemm(a, E4M3FN, b, E5M2, np.float32(1), 0, np.float32(1), 0, E4M3FN)
    assert int(b8[1, 1]) == 0x7E and int(b8[0, 0]) == 0x7F     # Inf saturates, NaN stays NaN


# ------------------------------------------------------------------ fp32 chunk ("slow") mode

def _chunks_numpy_f32(A, B, K, alpha):
    """The 128-chunk fp32 accumulation written with numpy float32 arithmetic."""
    M, N = A.shape[0], B.shape[0]
    out = np.empty((M, N), np.float32)
    for m in range(M):
        for n in range(N):
            acc = np.float32(0.0)
            for c in range(0, K, 128):
                part = np.float32(float(np.dot(A[m, c:c + 128], B[n, c:c + 128])))
                acc = np.float32(acc + part)
            out[m, n] = np.float32(acc * alpha)
    return out


@pytest.mark.parametrize("kind", ["gauss", "adversarial"])
def test_chunk_mode_matches_numpy_float32(kind):
    # the adversarial codes (subnormals beside +-448) give chunk sums wider than
    # 24 bits, so the rounding of each chunk partial is visible
    if kind == "gauss":
        d = datagen.set_gauss_n4096(12, 9, 1000)
    else:
        d = datagen.set_adversarial_n4096(12, 9, 1000)
    A, B = tdecode(d["a"], E4M3FN), tdecode(d["b"], E4M3FN)
    alpha = np.float32(np.float32(d["scale_a"]) * np.float32(d["scale_b"]))
    want = _chunks_numpy_f32(A, B, 1000, alpha)
    v, _, _ = oracle.scaled_gemm(d["a"], 0, d["b"], 0, d["scale_a"], 0, d["scale_b"], 0, F32, accum=ACC_F32_CHUNKS)
    assert np.array_equal(v.astype(np.float32).view(np.uint32), want.view(np.uint32))


def test_chunk_mode_single_chunk_equals_rounded_exact():
    d = datagen.set_256_cubed(10, 10, 128)
    ve, _, be = oracle.scaled_gemm(d["a"], 0, d["b"], 0, np.float32(1), 0, np.float32(1), 0, F32)
    vc, _, bc = oracle.scaled_gemm(d["a"], 0, d["b"], 0, np.float32(1), 0, np.float32(1), 0, F32, accum=ACC_F32_CHUNKS)
    assert np.array_equal(be, bc)


def test_chunk_mode_integer_data_is_exact():
    rng = np.random.default_rng(2)
    a = rng.choice(np.array([0x38, 0xB8, 0x40, 0x00], np.uint8), size=(7, 1000))   # +-1, 2, 0
    b = rng.choice(np.array([0x38, 0xB8, 0x48], np.uint8), size=(5, 1000))         # +-1, 4
    ve, _, _ = oracle.scaled_gemm(a, 0, b, 0, np.float32(1), 0, np.float32(1), 0, F32)
    vc, _, _ = oracle.scaled_gemm(a, 0, b, 0, np.float32(1), 0, np.float32(1), 0, F32, accum=ACC_F32_CHUNKS)
    assert np.array_equal(ve, vc)


@pytest.mark.parametrize("name", ["w1", "w2g", "w2a", "w3", "w5a", "w5b"])
def test_chunk_mode_meets_tolerance_on_workload_data(name):
    """Attainability: fp32 chunk accumulation stays within 2^-20 * sum|t| of the
    exact result on every workload's kind of data, so the fp32-output bound can be
    met by an fp32 accumulator."""
    rows = None
    if name == "w1":
        d = datagen.set_256_cubed(32, 64, 256); sam = sbm = 0
    elif name == "w2g":
        d = datagen.set_gauss_n4096(16, 64, 4096); sam = sbm = 0
    elif name == "w2a":
        d = datagen.set_adversarial_n4096(16, 64, 4096); sam = sbm = 0
    elif name == "w3":
        d = datagen.set_block_scaled_4096x14336x4096(16, 256, 4096); sam, sbm = 1, 2
    elif name == "w5a":
        d = datagen.set_e4m3_out_8192x28672x8200(8, 32, 8200); sam = sbm = 0
    else:
        d = datagen.set_e5m2_f16_8192x28672x8200(8, 32, 8200); sam = sbm = 0
    fa, fb = d["a_fmt"], d["b_fmt"]
    ve, sabs, _ = oracle.scaled_gemm(d["a"], fa, d["b"], fb, d["scale_a"], sam, d["scale_b"], sbm, F32)
    vc, _, _ = oracle.scaled_gemm(d["a"], fa, d["b"], fb, d["scale_a"], sam, d["scale_b"], sbm, F32, accum=ACC_F32_CHUNKS)
    assert np.all(np.abs(vc - ve) <= 2.0 ** -20 * sabs)


# ------------------------------------------------------------------ block-scaled GEMM + amax

def test_amax_gemm_brute_force():
    rng = np.random.default_rng(9)
    L, M, N, K, sf = 2, 3, 4, 70, 32
    a = finite_random_codes(rng, (L, M, K), E4M3FN)
    b = finite_random_codes(rng, (L, N, K), E4M3FN)
    sfa = datagen.pow2_scales(rng, (L, M, 3))
    sfb = datagen.pow2_scales(rng, (L, N, 3))
    v, _, bits, amax, idx = oracle.blockscaled_gemm_amax(a, b, E4M3FN, sfa, sfb, sf, F32)
    for l in range(L):
        ex = exact_gemm(a[l], E4M3FN, b[l], E4M3FN, lambda m, k: float(sfa[l, m, k // sf]),
                        lambda n, k: float(sfb[l, n, k // sf]), K)
        for m in range(M):
            for n in range(N):
                assert Fraction(v[l, m, n]) == ex[m, n]    # power-of-two scales keep it exact
    flat = np.abs(v).reshape(-1)
    assert amax == np.float32(flat.max()) and idx == int(np.argmax(flat))


def test_amax_unit_scales_equal_plain_gemm():
    """The cuDNN example call shape: m, n, k = 512, 256, 256, sf_vec_size 32,
    E5M2 inputs and all-ones scale factors reduce the block-scaled GEMM to a
    plain GEMM ("cuDNN frontend: GEMM + Amax (SM100)", Using JAX arrays)."""
    g = np.random.default_rng(0)
    a = datagen.gauss_codes(g, (1, 512, 256), 1.0, E5M2)
    b = datagen.gauss_codes(g, (1, 256, 256), 1.0, E5M2)
    ones_a = np.ones((1, 512, 8), np.float32)
    ones_b = np.ones((1, 256, 8), np.float32)
    v, _, _, amax, idx = oracle.blockscaled_gemm_amax(a, b, E5M2, ones_a, ones_b, 32, F32)
    A, B = tdecode(a[0], E5M2), tdecode(b[0], E5M2)
    ref = A @ B.T
    assert np.max(np.abs(v[0] - ref)) <= 2.0 ** -40 * np.max(np.abs(A) @ np.abs(B).T)
    assert amax == np.float32(np.max(np.abs(v)))


def test_amax_batch_equals_separate_calls():
    d = datagen.set_mx_l8_2048x2048x8192(3, 20, 24, 200)
    v, _, bits, amax, idx = oracle.blockscaled_gemm_amax(d["a"], d["b"], 0, d["sfa"], d["sfb"], 32, BF16)
    maxes = []
    for l in range(3):
        vl, _, bl, al, il = oracle.blockscaled_gemm_amax(d["a"][l:l + 1], d["b"][l:l + 1], 0,
                                                         d["sfa"][l:l + 1], d["sfb"][l:l + 1], 32, BF16)
        assert np.array_equal(vl[0], v[l]) and np.array_equal(bl[0], bits[l])
        maxes.append((al, l * 20 * 24 + il))
    best = max(maxes, key=lambda t: (t[0], -t[1]))
    assert amax == best[0] and idx == best[1]


def test_amax_nan_empty_and_ties():
    a = np.full((1, 2, 32), 0x38, np.uint8)
    b = np.full((1, 3, 32), 0x38, np.uint8)
    s1 = np.ones((1, 2, 1), np.float32); s2 = np.ones((1, 3, 1), np.float32)
    v, _, _, amax, idx = oracle.blockscaled_gemm_amax(a, b, 0, s1, s2, 32, F32)
    assert amax == 32.0 and idx == 0                 # all equal: the first index wins
    a[0, 1, 5] = 0x7F
    _, _, _, amax, idx = oracle.blockscaled_gemm_amax(a, b, 0, s1, s2, 32, F32)
    assert np.isnan(amax) and idx == 3               # first NaN at m = 1, n = 0
    z = np.zeros((0, 2, 32), np.uint8)
    _, _, _, amax, idx = oracle.blockscaled_gemm_amax(z, np.zeros((0, 3, 32), np.uint8), 0,
                                                      np.ones((0, 2, 1), np.float32), np.ones((0, 3, 1), np.float32), 32, F32)
    assert amax == 0.0 and idx == -1


def test_row_subset_matches_full():
    d = datagen.set_256_cubed(40, 30, 300)
    vf, sf_, bf = oracle.scaled_gemm(d["a"], 0, d["b"], 0, d["scale_a"], 0, d["scale_b"], 0, BF16)
    rows = np.array([39, 0, 17, 17])
    vr, sr, br = oracle.scaled_gemm(d["a"], 0, d["b"], 0, d["scale_a"], 0, d["scale_b"], 0, BF16, rows=rows)
    assert np.array_equal(vr, vf[rows]) and np.array_equal(br, bf[rows]) and np.array_equal(sr, sf_[rows])


def test_row_pitch_is_respected():
    """Bytes between K and the row pitch never contribute (filled with NaN codes)."""
    d = datagen.set_256_cubed(9, 7, 100)
    a = np.full((9, 112), 0x7F, np.uint8); a[:, :100] = d["a"]
    b = np.full((7, 104), 0x7F, np.uint8); b[:, :100] = d["b"]
    v1, _, _ = oracle.scaled_gemm_k(a, 0, b, 0, 100, np.float32(1), 0, np.float32(1), 0, F32)
    v2, _, _ = oracle.scaled_gemm(d["a"], 0, d["b"], 0, np.float32(1), 0, np.float32(1), 0, F32)
    assert np.array_equal(v1, v2)


# ------------------------------------------------------------------ bias (TileOPs GemmFP8FwdOp, forward)

def _bias_values(rng, N, d_type):
    """Random bias values exactly representable in d_type, as float64."""
    x = rng.normal(0, 4, size=N).astype(np.float32)
    if d_type == BF16:
        return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    if d_type == F16:
        return x.astype(np.float16).astype(np.float64)
    return x.astype(np.float64)


def _bits_of(vals, d_type):
    """Bit patterns of values exactly representable in d_type (numpy, not the oracle)."""
    v = np.asarray(vals, dtype=np.float64)
    if d_type == BF16:
        return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    if d_type == F16:
        return v.astype(np.float16).view(np.uint16)
    return v.astype(np.float32).view(np.uint32)


@pytest.mark.parametrize("d_type", [F32, BF16, F16])
@pytest.mark.parametrize("accum", [ACC_EXACT, ACC_F32_CHUNKS])
def test_bias_alone_when_the_product_is_zero(d_type, accum):
    # zero codes give a zero sum; the result is the bias itself, bit for bit
    rng = np.random.default_rng(11)
    M, N, K = 5, 37, 200
    a = np.zeros((M, K), dtype=np.uint8)
    b = finite_random_codes(rng, (N, K), E4M3FN)
    bias = _bias_values(rng, N, d_type)
    _, _, bits = oracle.scaled_gemm(a, E4M3FN, b, E4M3FN, np.float32(0.5), SCALE_TENSOR, np.float32(2.0),
                                    SCALE_TENSOR, d_type, accum=accum, bias=bias)
    assert np.array_equal(bits, np.broadcast_to(_bits_of(bias, d_type), (M, N)))


@pytest.mark.parametrize("d_type", [F32, BF16, F16])
def test_bias_closed_form_all_ones(d_type):
    # every code 0x38 = 1.0: the sum is K, times 0.5 * 0.25, plus small integer biases
    M, N, K = 3, 9, 256
    a = np.full((M, K), 0x38, dtype=np.uint8)
    b = np.full((N, K), 0x38, dtype=np.uint8)
    bias = np.arange(N, dtype=np.float64) - 4.0
    value, _, bits = oracle.scaled_gemm(a, E4M3FN, b, E4M3FN, np.float32(0.5), SCALE_TENSOR, np.float32(0.25),
                                        SCALE_TENSOR, d_type, bias=bias)
    want = K * 0.125 + bias
    assert np.array_equal(value, np.broadcast_to(want, (M, N)))
    assert np.array_equal(bits, np.broadcast_to(_bits_of(want, d_type), (M, N)))


def test_bias_block_scaled_matches_the_exact_sum_plus_bias():
    # block scales: the exact rational sum (torch-decoded operands) plus the bias
    rng = np.random.default_rng(12)
    M, N, K = 4, 20, 300
    a = finite_random_codes(rng, (M, K), E4M3FN)
    b = finite_random_codes(rng, (N, K), E4M3FN)
    kb = -(-K // 128)
    sa = datagen.log_uniform_scales(rng, (M, kb))
    sb = datagen.log_uniform_scales(rng, (N, kb))
    bias = _bias_values(rng, N, F32)
    v, sabs, _ = oracle.scaled_gemm(a, E4M3FN, b, E4M3FN, sa, SCALE_1x128, sb, SCALE_1x128, F32, bias=bias)
    ex = exact_gemm(a, E4M3FN, b, E4M3FN, lambda m, k: Fraction(float(sa[m, k // 128])),
                    lambda n, k: Fraction(float(sb[n, k // 128])), K)
    for m in range(M):
        for n in range(N):
            err = abs(Fraction(float(v[m, n])) - (ex[m, n] + Fraction(float(bias[n]))))
            assert err <= Fraction(2) ** -40 * (Fraction(float(sabs[m, n])) + abs(Fraction(float(bias[n]))))


def test_bias_with_fp8_output_is_rejected():
    a = np.zeros((2, 32), dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.scaled_gemm(a, E4M3FN, a, E4M3FN, np.float32(1), SCALE_TENSOR, np.float32(1), SCALE_TENSOR,
                           E4M3FN, bias=np.zeros(2))
