"""Pins of the oracle's page-native scale-factor unpacking (CPU).

The cuDNN GEMM + Amax (SM100) page gives its scale tensors SFA / SFB the
logical shape (32, 4, ceil(MN/128), 4, ceil(K/(4 sf)), L), states that this is
a view of the C-contiguous storage (L, ceil(MN/128), ceil(K/(4 sf)), 32, 4, 4)
permuted by (3, 4, 1, 5, 2, 0), and names the element types float8_e8m0fnu,
float8_e4m3fn and int8 (read as E8M0). What these tests pin:

- element decoding: every code against torch's own float8 dtypes and the
  closed form 2^(e-127);
- the storage-to-logical permutation, by building the logical view with numpy
  exactly as the page states it;
- that every storage byte reaches at most one factor and that padding is
  never read;
- the page's usage example (E5M2 operands, factors all 1.0) reduces to the
  plain product of the decoded codes.

Which logical coordinate is which row and which group (row = i0 + 32 i1 +
128 i2, group = j0 + 4 j1) is a reading of the shapes: the page does not state
it, so that order stays unpinned and the tests that use it say so.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _logical(storage):
    """The page's logical view: storage permuted by (3, 4, 1, 5, 2, 0)."""
    return np.transpose(storage, (3, 4, 1, 5, 2, 0))


def _expected_by_reading(storage, MN, K, sf_vec, decode):
    """Plain factors from the logical view under the row / group reading."""
    logical = _logical(storage)
    L = storage.shape[0]
    G = -(-K // sf_vec)
    out = np.empty((L, MN, G), dtype=np.float64)
    for mn in range(MN):
        i0, i1, i2 = mn % 32, (mn // 32) % 4, mn // 128
        for g in range(G):
            j0, j1 = g % 4, g // 4
            out[:, mn, g] = decode(logical[i0, i1, i2, j0, j1, :])
    return out


def test_atom_shapes_match_the_page():
    # the logical shape that the page lists, from the storage shape it lists
    for MN, K, L, sf in [(128, 128, 1, 32), (300, 1000, 2, 32), (1, 16, 3, 16), (513, 4096, 1, 16)]:
        st = oracle.sf_atom_shape(MN, K, L, sf)
        assert st == (L, -(-MN // 128), -(-K // (4 * sf)), 32, 4, 4)
        assert _logical(np.zeros(st, np.uint8)).shape == (32, 4, -(-MN // 128), 4, -(-K // (4 * sf)), L)


def test_e8m0_every_code():
    # one batch item per code: every factor of item l is code l
    L = 256
    st = oracle.sf_atom_shape(1, 32, L, 32)
    sf = np.broadcast_to(np.arange(L, dtype=np.uint8).reshape(L, 1, 1, 1, 1, 1), st).copy()
    got = oracle.sf_atom_unpack(sf, oracle.SF_E8M0, 1, 32, L, 32)[:, 0, 0].astype(np.float64)
    closed = np.where(np.arange(256) == 255, np.nan, np.ldexp(1.0, np.arange(256) - 127))
    np.testing.assert_array_equal(got, closed)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    np.testing.assert_array_equal(got, ref)
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_e4m3_every_code():
    L = 256
    st = oracle.sf_atom_shape(1, 16, L, 16)
    sf = np.broadcast_to(np.arange(L, dtype=np.uint8).reshape(L, 1, 1, 1, 1, 1), st).copy()
    got = oracle.sf_atom_unpack(sf, oracle.SF_E4M3FN, 1, 16, L, 16)[:, 0, 0].astype(np.float64)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("MN,K,L,sf", [(128, 128, 1, 32), (300, 1000, 2, 32), (257, 96, 1, 16), (64, 4096, 1, 32)])
def test_storage_permutation_and_reading(MN, K, L, sf):
    # reading of the row / group order: parity unpinned for that order; the
    # permutation from storage to the logical view is the page's
    g = np.random.default_rng(MN * 7 + K)
    st = oracle.sf_atom_shape(MN, K, L, sf)
    sf_bytes = g.integers(100, 160, size=st, dtype=np.uint8)
    got = oracle.sf_atom_unpack(sf_bytes, oracle.SF_E8M0, MN, K, L, sf).astype(np.float64)
    want = _expected_by_reading(sf_bytes, MN, K, sf, lambda c: np.ldexp(1.0, c.astype(np.int64) - 127))
    np.testing.assert_array_equal(got, want)


def test_each_byte_reaches_at_most_one_factor_and_padding_is_unread():
    # plant a NaN code in one storage byte at a time: a byte of the tensor's
    # rows and groups turns exactly one factor NaN, a padding byte none
    MN, K, L, sf = 100, 200, 1, 32  # 28 padding rows, groups 7 of 8 used
    st = oracle.sf_atom_shape(MN, K, L, sf)
    base = np.full(st, 127, dtype=np.uint8)
    hit = set()
    n_pad = 0
    flat = base.reshape(-1)
    for pos in range(flat.size):
        flat[pos] = 0xFF
        out = oracle.sf_atom_unpack(base, oracle.SF_E8M0, MN, K, L, sf)
        nan = np.argwhere(np.isnan(out))
        flat[pos] = 127
        assert len(nan) <= 1
        if len(nan) == 0:
            n_pad += 1
        else:
            t = tuple(nan[0])
            assert t not in hit
            hit.add(t)
    G = -(-K // sf)
    assert len(hit) == L * MN * G
    assert n_pad == flat.size - L * MN * G


def test_padding_contents_do_not_matter():
    MN, K, L, sf = 200, 700, 2, 32
    g = np.random.default_rng(5)
    st = oracle.sf_atom_shape(MN, K, L, sf)
    s1 = g.integers(110, 140, size=st, dtype=np.uint8)
    want = oracle.sf_atom_unpack(s1, oracle.SF_E8M0, MN, K, L, sf)
    # overwrite everything that is padding under any reading: rows past MN of
    # the last block and groups past ceil(K/sf) of the last 4-group block are
    # not distinguishable by position alone, so compare on a copy whose every
    # byte outside the used set (found by the planting test's method) is NaN
    s2 = s1.copy()
    flat = s2.reshape(-1)
    probe = np.full(st, 127, np.uint8).reshape(-1)
    for pos in range(flat.size):
        probe[pos] = 0xFF
        if not np.isnan(oracle.sf_atom_unpack(probe, oracle.SF_E8M0, MN, K, L, sf)).any():
            flat[pos] = 0xFF
        probe[pos] = 127
    assert (flat == 0xFF).sum() > 0
    np.testing.assert_array_equal(oracle.sf_atom_unpack(s2, oracle.SF_E8M0, MN, K, L, sf), want)


def test_page_example_unit_factors_give_the_plain_product():
    # the page's usage example: m, n, k = 512, 256, 256, sf_vec_size 32, E5M2
    # operands from standard normal values, factors all 1.0 (E8M0 code 127),
    # f32 C; with unit factors C is the plain product of the decoded codes
    m, n, k, sf = 512, 256, 256, 32
    g = np.random.default_rng(11)
    a = torch.from_numpy(g.standard_normal((1, m, k)).astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    b = torch.from_numpy(g.standard_normal((1, n, k)).astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    sfa = np.full((1, m // 128, k // (4 * sf), 32, 4, 4), 127, dtype=np.uint8)
    sfb = np.full((1, n // 128, k // (4 * sf), 32, 4, 4), 127, dtype=np.uint8)
    val, _, bits, amax, idx = oracle.blockscaled_gemm_amax_atom(a, b, oracle.E5M2, sfa, sfb, oracle.SF_E8M0, sf,
                                                                oracle.F32)
    ad = torch.from_numpy(a[0]).view(torch.float8_e5m2).double().numpy()
    bd = torch.from_numpy(b[0]).view(torch.float8_e5m2).double().numpy()
    want = ad @ bd.T  # every partial sum of these products is exact in float64
    np.testing.assert_array_equal(val[0], want)
    np.testing.assert_array_equal(bits[0].view(np.float32), want.astype(np.float32))
    assert amax == np.float32(np.abs(want).max())
    assert idx == int(np.argmax(np.abs(want).reshape(-1)))


def test_one_factor_scales_one_row_group_exactly():
    # a factor 2^d on one (row, group) multiplies exactly that group's
    # products of that row (reading of the row / group order: unpinned order)
    M, N, K, sf = 130, 20, 320, 32
    g = np.random.default_rng(3)
    a = g.integers(0, 0x70, size=(1, M, K), dtype=np.uint8)
    b = g.integers(0, 0x70, size=(1, N, K), dtype=np.uint8)
    sfa = np.full(oracle.sf_atom_shape(M, K, 1, sf), 127, np.uint8)
    sfb = np.full(oracle.sf_atom_shape(N, K, 1, sf), 127, np.uint8)
    base, *_ = oracle.blockscaled_gemm_amax_atom(a, b, oracle.E4M3FN, sfa, sfb, oracle.SF_E8M0, sf, oracle.F32)
    row, grp, d = 129, 9, 5
    # logical (i0, i1, i2, j0, j1, l) of (row, grp) -> storage [l][i2][j1][i0][i1][j0]
    sfa[0, row // 128, grp // 4, row % 32, (row // 32) % 4, grp % 4] = 127 + d
    got, *_ = oracle.blockscaled_gemm_amax_atom(a, b, oracle.E4M3FN, sfa, sfb, oracle.SF_E8M0, sf, oracle.F32)
    ad = oracle.decode_fp8(a[0], oracle.E4M3FN)
    bd = oracle.decode_fp8(b[0], oracle.E4M3FN)
    part = ad[row, grp * sf:(grp + 1) * sf] @ bd[:, grp * sf:(grp + 1) * sf].T
    want = base.copy()
    want[0, row] += (2.0 ** d - 1.0) * part
    np.testing.assert_array_equal(got, want)
