"""Pins of the oracle's grouped GEMM in its four layouts (CPU).

TileOPs' GroupedGemmFwdOp ("Linear Algebra Operators") selects NT, NN, TN or
TT with (transpose_a, transpose_b). Without transpose_a the groups split the
rows of a; with it they split the contraction and each group yields an
[N, K] block. What pins the oracle here, against facts other than its own
code:

- brute force: every layout on tiny ragged inputs (an empty group included)
  against plain Python loops over the operands as the layout table states
  them, decoded by torch's own float8 dtypes; all sums are exact in float64;
- the groups of the contraction-split form add up to the ungrouped product
  A^T B of all rows;
- an empty group's block is +0 in every output type;
- the two storage orders of b give the same product (NN against NT, TT
  against TN) on the same logical operand;
- metadata the page forbids is refused.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3FN, E5M2, F32, BF16, E2M1  # noqa: F401


def dec(codes, fmt):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn if fmt == E4M3FN else torch.float8_e5m2).double().numpy()


def codes(g, shape, fmt=E4M3FN):
    x = torch.from_numpy(g.standard_normal(shape).astype(np.float32) * 4)
    return x.to(torch.float8_e4m3fn if fmt == E4M3FN else torch.float8_e5m2).view(torch.uint8).numpy()


def offsets_of(sizes):
    return np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int32)


SIZES = [3, 0, 5, 2]


@pytest.mark.parametrize("ta,tb", [(False, True), (False, False), (True, False), (True, True)],
                         ids=["NT", "NN", "TN", "TT"])
def test_brute_force_every_layout(ta, tb):
    g = np.random.default_rng(17 + 2 * ta + tb)
    sizes = np.array(SIZES, np.int32)
    offs = offsets_of(sizes)
    G, S, N, K = len(SIZES), int(sizes.sum()), 3, 5
    sa, sb = 0.5, 4.0
    if not ta:
        a = codes(g, (S, K))
        b = codes(g, (G, N, K) if tb else (G, K, N), E5M2)
        A, B = dec(a, E4M3FN), dec(b, E5M2)
        want = np.zeros((S, N))
        for gi in range(G):
            for r in range(offs[gi], offs[gi] + sizes[gi]):
                for n in range(N):
                    acc = 0.0
                    for k in range(K):
                        acc += A[r, k] * (B[gi, n, k] if tb else B[gi, k, n])
                    want[r, n] = acc * sa * sb
    else:
        a = codes(g, (S, N))
        b = codes(g, (K, S) if tb else (S, K), E5M2)
        A, B = dec(a, E4M3FN), dec(b, E5M2)
        want = np.zeros((G, N, K))
        for gi in range(G):
            for n in range(N):
                for k in range(K):
                    acc = 0.0
                    for r in range(offs[gi], offs[gi] + sizes[gi]):
                        acc += A[r, n] * (B[k, r] if tb else B[r, k])
                    want[gi, n, k] = acc * sa * sb
    val, _, bits = oracle.grouped_gemm_layout(a, E4M3FN, b, E5M2, sizes, offs, sa, sb, F32, ta, tb)
    np.testing.assert_array_equal(val, want)
    np.testing.assert_array_equal(bits.view(np.float32), want.astype(np.float32))


@pytest.mark.parametrize("tb", [False, True], ids=["TN", "TT"])
def test_contraction_groups_add_up_to_the_whole_product(tb):
    g = np.random.default_rng(23 + tb)
    sizes = np.array([40, 0, 1, 130, 77, 0, 12], np.int32)
    S, N, K = int(sizes.sum()), 24, 40
    a = codes(g, (S, N))
    b = codes(g, (K, S) if tb else (S, K))
    val, sabs, _ = oracle.grouped_gemm_layout(a, E4M3FN, b, E4M3FN, sizes, offsets_of(sizes), 1.0, 1.0, F32,
                                              True, tb)
    A, B = dec(a, E4M3FN), dec(b.T if tb else b, E4M3FN)
    np.testing.assert_array_equal(val.sum(axis=0), A.T @ B)  # every partial sum here is exact in float64
    np.testing.assert_array_equal(sabs.sum(axis=0), np.abs(A).T @ np.abs(B))


@pytest.mark.parametrize("d_type", [oracle.E4M3FN, oracle.E5M2, oracle.F32, oracle.BF16, oracle.F16])
def test_empty_group_block_is_positive_zero(d_type):
    g = np.random.default_rng(29)
    sizes = np.array([0, 9, 0], np.int32)
    a = codes(g, (9, 8))
    b = codes(g, (9, 16))
    val, sabs, bits = oracle.grouped_gemm_layout(a, E4M3FN, b, E4M3FN, sizes, offsets_of(sizes), 1.0, 1.0, d_type,
                                                 True, False, scale_result=1.0)
    for gi in (0, 2):
        assert (val[gi] == 0).all() and not np.signbit(val[gi]).any() and (sabs[gi] == 0).all()
        assert (bits[gi] == 0).all()
    assert (sabs[1] > 0).any()


def test_storage_orders_of_b_agree():
    g = np.random.default_rng(31)
    sizes = np.array([5, 0, 130, 7], np.int32)
    offs = offsets_of(sizes)
    S, N, K = int(sizes.sum()), 20, 36
    a = codes(g, (S, K))
    b_nk = codes(g, (4, N, K))
    nt = oracle.grouped_gemm_layout(a, E4M3FN, b_nk, E4M3FN, sizes, offs, 0.25, 2.0, BF16, False, True,
                                    accum=oracle.ACC_F32_CHUNKS)
    nn = oracle.grouped_gemm_layout(a, E4M3FN, np.ascontiguousarray(b_nk.transpose(0, 2, 1)), E4M3FN, sizes, offs,
                                    0.25, 2.0, BF16, False, False, accum=oracle.ACC_F32_CHUNKS)
    for x, y in zip(nt, nn):
        np.testing.assert_array_equal(x, y)
    a2 = codes(g, (S, N))
    b_sk = codes(g, (S, K))
    tn = oracle.grouped_gemm_layout(a2, E4M3FN, b_sk, E4M3FN, sizes, offs, 1.0, 1.0, F32, True, False,
                                    accum=oracle.ACC_F32_CHUNKS)
    tt = oracle.grouped_gemm_layout(a2, E4M3FN, np.ascontiguousarray(b_sk.T), E4M3FN, sizes, offs, 1.0, 1.0, F32,
                                    True, True, accum=oracle.ACC_F32_CHUNKS)
    for x, y in zip(tn, tt):
        np.testing.assert_array_equal(x, y)


def test_forbidden_metadata_is_refused():
    a = np.zeros((6, 4), np.uint8)
    b = np.zeros((6, 8), np.uint8)
    for sizes, offs in [([3, 2], [0, 3]), ([3, 3], [0, 2]), ([7, -1], [0, 7])]:
        with pytest.raises(ValueError):
            oracle.grouped_gemm_layout(a, E4M3FN, b, E4M3FN, np.array(sizes), np.array(offs), 1.0, 1.0, F32,
                                       True, False)
