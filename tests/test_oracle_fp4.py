"""Pins of the oracle's FP4 (E2M1) operands of the block-scaled GEMM + amax (CPU).

The cuDNN GEMM + Amax (SM100) page takes float4_e2m1fn_x2 operands: E2M1
values packed two per byte, rows of K/2 bytes. What pins the oracle here:

- the 16 codes against the E2M1 format's closed form (sign, 2 exponent bits
  with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6);
- every E2M1 value is an E4M3 value, so the GEMM of FP4 operands must equal,
  bit for bit, the GEMM of the same values written as E4M3 codes (encoded by
  torch's float8_e4m3fn cast) through the already pinned FP8 path, with
  sf_vec_size 32 and 16;
- closed forms: all-6 operands give 36 K per output, alternating signs give 0.

Which nibble of a byte holds the first element is not stated on the page; C
does not depend on it (both operands use the same order and the two elements
of a byte always share a scale group), so no test can or needs to pin it.
"""
import numpy as np
import pytest
import torch

import oracle

MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def test_e2m1_closed_form_table():
    got = oracle.decode_fp4(np.arange(16))
    np.testing.assert_array_equal(np.abs(got), np.concatenate([MAGS, MAGS]))
    assert all(np.signbit(got[8:])) and not any(np.signbit(got[:8]))
    np.testing.assert_array_equal(got[np.arange(16) ^ 8], -got)
    assert np.all(np.diff(got[:8]) > 0)


def pack(codes):
    """[..., K] codes 0..15 -> [..., K/2] bytes, element 2i in the low nibble."""
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def as_e4m3(codes):
    vals = torch.from_numpy(oracle.decode_fp4(codes).astype(np.float32))
    return vals.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("sf", [32, 16])
@pytest.mark.parametrize("L,M,N,K", [(2, 17, 23, 96), (1, 40, 9, 512)])
def test_fp4_equals_fp8_of_the_same_values(L, M, N, K, sf):
    g = np.random.default_rng(K + sf)
    ca = g.integers(0, 16, size=(L, M, K), dtype=np.uint8)
    cb = g.integers(0, 16, size=(L, N, K), dtype=np.uint8)
    G = -(-K // sf)
    sfa = np.ldexp(1.0, g.integers(-8, 5, size=(L, M, G))).astype(np.float32)
    sfb = np.ldexp(1.0, g.integers(-8, 5, size=(L, N, G))).astype(np.float32)
    v4, s4, b4, am4, ix4 = oracle.blockscaled_gemm_amax(pack(ca), pack(cb), oracle.E2M1, sfa, sfb, sf, oracle.F32)
    v8, s8, b8, am8, ix8 = oracle.blockscaled_gemm_amax(as_e4m3(ca), as_e4m3(cb), oracle.E4M3FN, sfa, sfb, sf,
                                                        oracle.F32)
    np.testing.assert_array_equal(v4, v8)
    np.testing.assert_array_equal(s4, s8)
    np.testing.assert_array_equal(b4, b8)
    assert am4 == am8 and ix4 == ix8


def test_fp4_closed_forms():
    K = 256
    six = np.full((1, 3, K), 7, np.uint8)  # +6
    ones = np.ones((1, 3, K // 32), np.float32)
    v, *_ = oracle.blockscaled_gemm_amax(pack(six), pack(six), oracle.E2M1, ones, ones, 32, oracle.F32)
    assert np.all(v == 36.0 * K)
    alt = six.copy()
    alt[..., 1::2] = 7 | 8  # -6 at odd k
    v, *_ = oracle.blockscaled_gemm_amax(pack(alt), pack(six), oracle.E2M1, ones, ones, 32, oracle.F32)
    assert np.all(v == 0.0) and not np.any(np.signbit(v))


# ------------------------------------------------------------------ E2M1 output (FP4 C)

def test_e2m1_output_rounding():
    vals = oracle.decode_fp4(np.arange(8))  # 0, 0.5, 1, 1.5, 2, 3, 4, 6 (pinned above)
    # every value is its own code, both signs
    np.testing.assert_array_equal(oracle.round_to(vals, oracle.E2M1), np.arange(8))
    np.testing.assert_array_equal(oracle.round_to(-vals[1:], oracle.E2M1), np.arange(9, 16))
    # midpoints go to the even code, anything off the midpoint to the nearer value
    for c in range(7):
        mid = (vals[c] + vals[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.round_to(np.array([mid]), oracle.E2M1)[0] == even
        assert oracle.round_to(np.array([np.nextafter(mid, 0)]), oracle.E2M1)[0] == c
        assert oracle.round_to(np.array([np.nextafter(mid, 9)]), oracle.E2M1)[0] == c + 1
    # saturation (no infinities in E2M1), NaN takes the largest value's code (a reading), -0 keeps its sign
    got = oracle.round_to(np.array([6.5, 1e30, np.inf, -7.0, -np.inf, np.nan, -0.0]), oracle.E2M1)
    np.testing.assert_array_equal(got, [7, 7, 7, 15, 15, 7, 8])


@pytest.mark.parametrize("N", [6, 7])
def test_e2m1_c_is_packed_low_nibble_first(N):
    # C rows of ceil(N/2) bytes, element 2i in the low nibble; an odd N leaves the last high nibble 0
    g = np.random.default_rng(N)
    L, M, K = 2, 3, 64
    a = g.integers(0, 256, size=(L, M, K // 2), dtype=np.uint8)
    b = g.integers(0, 256, size=(L, N, K // 2), dtype=np.uint8)
    ones = np.ones((L, M, 2), np.float32), np.ones((L, N, 2), np.float32)
    value, _, packed, _, _ = oracle.blockscaled_gemm_amax(a, b, oracle.E2M1, ones[0], ones[1], 32, oracle.E2M1)
    codes = oracle.round_to(value.reshape(-1), oracle.E2M1).reshape(L, M, N)
    if N % 2:
        codes = np.concatenate([codes, np.zeros((L, M, 1), codes.dtype)], axis=2)
    np.testing.assert_array_equal(packed, codes[..., 0::2] | (codes[..., 1::2] << 4))
