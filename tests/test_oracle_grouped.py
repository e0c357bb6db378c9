"""Pins of the oracle's grouped GEMM (CPU).

TileOPs' GroupedGemmFwdOp (NT layout) gives each group a run of packed rows of
a and its own b; here with FP8 operands and one scale per operand. What pins
the oracle's grouped GEMM, against facts other than its own loop:

- a closed form: all-one rows of a against groups whose b is all v_g give
  K * v_g * s_a * s_b on exactly that group's rows (empty groups included);
- one group over every row is the plain (already pinned) scaled GEMM, bit for
  bit, in every output type;
- groups that all use the same b give, together, the plain GEMM of all the
  rows with that b, bit for bit, whatever the ragged sizes;
- metadata that the page forbids (sizes not adding up, offsets that are not
  their exclusive prefix sum, negative sizes) is refused.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3FN, E5M2, F32, BF16, F16


def e4m3(v):
    return int(torch.tensor([float(v)]).to(torch.float8_e4m3fn).view(torch.uint8).item())


def offsets_of(sizes):
    return np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int32)


def test_closed_form_per_group():
    sizes = np.array([3, 0, 5, 1, 0, 7], np.int32)
    G, N, K = sizes.size, 9, 160
    a = np.full((sizes.sum(), K), e4m3(1.0), np.uint8)
    vals = [1.0, 2.0, 4.0, 0.5, 8.0, 3.0]
    b = np.stack([np.full((N, K), e4m3(v), np.uint8) for v in vals])
    value, _, bits = oracle.grouped_gemm(a, E4M3FN, b, E4M3FN, sizes, offsets_of(sizes), 0.5, 0.25, F32)
    r = 0
    for g in range(G):
        want = K * vals[g] * 0.5 * 0.25
        assert np.all(value[r:r + sizes[g]] == want)
        assert np.all(bits[r:r + sizes[g]].view(np.float32) == np.float32(want))
        r += sizes[g]
    assert r == sizes.sum()


@pytest.mark.parametrize("d_type", [F32, BF16, F16, E4M3FN, E5M2])
def test_one_group_is_the_plain_gemm(d_type):
    g = np.random.default_rng(d_type)
    M, N, K = 37, 21, 200
    a = g.integers(0, 0x7F, size=(M, K), dtype=np.uint8)
    b = g.integers(0, 0x7F, size=(1, N, K), dtype=np.uint8)
    sr = 1.0 / 16 if d_type in (E4M3FN, E5M2) else None
    v1, s1, b1 = oracle.grouped_gemm(a, E4M3FN, b, E4M3FN, [M], [0], 2.0 ** -6, 0.75, d_type, scale_result=sr)
    v2, s2, b2 = oracle.scaled_gemm(a, E4M3FN, b[0], E4M3FN, 2.0 ** -6, 0, 0.75, 0, d_type, scale_result=sr)
    np.testing.assert_array_equal(v1, v2)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(b1, b2)


@pytest.mark.parametrize("accum", [oracle.ACC_EXACT, oracle.ACC_F32_CHUNKS])
def test_shared_b_equals_one_gemm_over_all_rows(accum):
    g = np.random.default_rng(7 + accum)
    sizes = np.array([0, 13, 1, 40, 0, 6, 64], np.int32)
    G, N, K = sizes.size, 17, 300
    a = g.integers(0, 0xFF, size=(sizes.sum(), K), dtype=np.uint8)
    a[a == 0x7F] = 0; a[a == 0xFF] = 0  # no NaN codes
    b1 = g.integers(0, 0x7E, size=(N, K), dtype=np.uint8)
    b = np.stack([b1] * G)
    v1, s1, bits1 = oracle.grouped_gemm(a, E4M3FN, b, E4M3FN, sizes, offsets_of(sizes), 0.125, 3.0, BF16, accum=accum)
    v2, s2, bits2 = oracle.scaled_gemm(a, E4M3FN, b1, E4M3FN, 0.125, 0, 3.0, 0, BF16, accum=accum)
    np.testing.assert_array_equal(v1, v2)
    np.testing.assert_array_equal(bits1, bits2)


@pytest.mark.parametrize("rows,sizes,offsets", [
    (5, [2, 3], [0, 3]),         # offsets are not the exclusive prefix sum
    (5, [2, 3], [1, 3]),         # the first group does not start at row 0
    (5, [2, -1, 4], [0, 2, 1]),  # a negative size
    (6, [2, 3], [0, 2]),         # the sizes do not add up to the row count
])
def test_inconsistent_metadata_refused(rows, sizes, offsets):
    a = np.zeros((rows, 32), np.uint8)
    b = np.zeros((len(sizes), 4, 32), np.uint8)
    with pytest.raises(ValueError):
        oracle.grouped_gemm(a, E4M3FN, b, E4M3FN, sizes, offsets, 1.0, 1.0, F32)
