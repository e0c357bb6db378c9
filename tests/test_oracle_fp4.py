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
