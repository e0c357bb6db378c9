"""GPU checks of the Python tensor helpers (argument marshalling only).

Each helper of block_scaled_gemm_amd (scaled_gemm, scaled_bmm,
scaled_grouped_mm, blockscaled_gemm_amax) must hand the C ABI exactly the
pointers, pitches, strides and modes that a direct call would: its result is
compared bit for bit with the raw C-ABI call on the same inputs (whose
numerics the parity tests check against the oracle). Error paths raise before
anything is launched.
"""
import numpy as np
import pytest

import datagen
from oracle import E4M3FN, E5M2, F32, BF16, F16

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")
torch = gu.torch
mm = gu.mm
DEV = gu.DEV


def fp8(codes, fmt=E4M3FN):
    t = torch.from_numpy(np.ascontiguousarray(codes)).to(DEV)
    return t.view(torch.float8_e4m3fn if fmt == E4M3FN else torch.float8_e5m2)


def bits(t):
    t = t.contiguous()
    view = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()]
    return t.view(view).cpu().numpy().view({1: np.uint8, 2: np.uint16, 4: np.uint32}[t.element_size()])


def f32(x):
    return torch.tensor(np.atleast_1d(np.asarray(x, np.float32)), device=DEV)


@pytest.mark.parametrize("M,N,K", [(300, 200, 512), (40, 136, 256)], ids=["tiles", "skinny"])
def test_scaled_gemm_matches_raw_abi(M, N, K):
    g = datagen.rng(40, M)
    a = datagen.gauss_codes(g, (M, K), 64.0)
    b = datagen.gauss_codes(g, (N, K), 64.0, E5M2)
    out = mm.scaled_gemm(fp8(a), fp8(b, E5M2), f32(0.5), f32(0.25), torch.bfloat16)
    raw = gu.scaled_gemm(a, E4M3FN, b, E5M2, K, 0.5, 0, 0.25, 0, BF16)
    np.testing.assert_array_equal(bits(out), raw)
    # scaled_mm's column-major mat2 [K, N]: read as its [N, K] transpose
    out_t = mm.scaled_gemm(fp8(a), fp8(b, E5M2).t(), f32(0.5), f32(0.25), torch.bfloat16)
    np.testing.assert_array_equal(bits(out_t), raw)


def test_scaled_gemm_block_scales_bias_and_fp8_out():
    M, N, K = 256, 384, 640
    g = datagen.rng(41, 0)
    a = datagen.gauss_codes(g, (M, K), 64.0)
    b = datagen.gauss_codes(g, (N, K), 64.0)
    kb = -(-K // 128)
    sa = datagen.pow2_scales(g, (M, kb))
    sb = datagen.pow2_scales(g, (-(-N // 128), kb))
    bias = datagen.bias_bf16_bits(N)
    tb = torch.from_numpy(bias.view(np.int16)).to(DEV).view(torch.bfloat16)
    out = mm.scaled_gemm(fp8(a), fp8(b), f32(sa).reshape(M, kb), f32(sb).reshape(-1, kb), torch.bfloat16, bias=tb)
    raw = gu.scaled_gemm_bias(a, E4M3FN, b, E4M3FN, K, sa, 1, sb, 2, bias, BF16)
    np.testing.assert_array_equal(bits(out), raw)
    out8 = mm.scaled_gemm(fp8(a), fp8(b), f32(2.0 ** -6), f32(0.5), torch.float8_e4m3fn,
                          scale_result=f32(1.0 / 16))
    raw8 = gu.scaled_gemm(a, E4M3FN, b, E4M3FN, K, 2.0 ** -6, 0, 0.5, 0, E4M3FN, scale_result=1.0 / 16)
    np.testing.assert_array_equal(bits(out8), raw8)


def test_scaled_bmm_matches_raw_abi():
    L, M, N, K = 3, 130, 96, 384
    g = datagen.rng(42, 0)
    a = datagen.gauss_codes(g, (L, M, K), 64.0)
    b = datagen.gauss_codes(g, (L, N, K), 64.0)
    out = mm.scaled_bmm(fp8(a), fp8(b), f32(0.5), f32(0.125), torch.float16)
    raw = gu.scaled_gemm_batched(a, E4M3FN, b, E4M3FN, K, 0.5, 0.125, F16)
    np.testing.assert_array_equal(bits(out).reshape(L, M, N), raw.reshape(L, M, N))


def test_scaled_grouped_mm_matches_raw_abi():
    w = datagen.set_grouped_8x8192x4096x4096(G=6, batch_sum=700, N=200, K=256, empty=1, config=43)
    sizes = torch.from_numpy(w["sizes"]).to(DEV)
    offsets = torch.from_numpy(w["offsets"]).to(DEV)
    out = mm.scaled_grouped_mm(fp8(w["a"]), fp8(w["b"]), sizes, offsets, f32(w["scale_a"]), f32(w["scale_b"]),
                               torch.float32, use_fast_accum=True)
    raw = gu.scaled_gemm_grouped(w["a"], E4M3FN, w["b"], E4M3FN, w["sizes"], w["offsets"], w["scale_a"],
                                 w["scale_b"], F32, fast=True)
    np.testing.assert_array_equal(bits(out), raw)


def test_blockscaled_gemm_amax_helper_all_factor_forms():
    # fp32 factors
    w = datagen.set_mx_l8_2048x2048x8192(2, 96, 136, 512)
    c, amax, idx = mm.blockscaled_gemm_amax(fp8(w["a"]), fp8(w["b"]), f32(w["sfa"]).reshape(w["sfa"].shape),
                                            f32(w["sfb"]).reshape(w["sfb"].shape), torch.float32, with_index=True)
    rc, ra, ri = gu.blockscaled_gemm_amax(w["a"], w["b"], E4M3FN, w["sfa"], w["sfb"], F32)
    np.testing.assert_array_equal(bits(c), rc)
    assert float(amax.item()) == ra and int(idx.item()) == ri
    # the page's E8M0 bytes, as float8_e8m0fnu tensors
    w = datagen.set_mx_atom_l8_2048x2048x8192(2, 96, 136, 512)
    e8 = lambda x: torch.from_numpy(x).to(DEV).view(torch.float8_e8m0fnu)
    c, amax = mm.blockscaled_gemm_amax(fp8(w["a"]), fp8(w["b"]), e8(w["sfa"]), e8(w["sfb"]), torch.bfloat16)
    rc, ra, _ = gu.blockscaled_gemm_amax_atom(w["a"], w["b"], E4M3FN, w["sfa"], w["sfb"], BF16)
    np.testing.assert_array_equal(bits(c), rc)
    assert float(amax.item()) == ra
    # FP4 operands (uint8 pairs) with E8M0 factors per 16, and with E4M3 factors per 16
    u8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    w = datagen.set_fp4_l8_2048x2048x8192(2, 80, 72, 256, 16, config=44)
    c, amax = mm.blockscaled_gemm_amax(u8(w["a"]), u8(w["b"]), u8(w["sfa"]), u8(w["sfb"]), torch.float32,
                                       sf_vec_size=16, ab_format=mm.MM_F4_E2M1)
    rc, ra, _ = gu.blockscaled_gemm_amax_atom(w["a"], w["b"], 5, w["sfa"], w["sfb"], F32, sf=16)
    np.testing.assert_array_equal(bits(c), rc)
    w = datagen.set_nvfp4_l8_2048x2048x8192(2, 80, 72, 256, config=45)
    e4 = lambda x: torch.from_numpy(x).to(DEV).view(torch.float8_e4m3fn)
    c, amax = mm.blockscaled_gemm_amax(u8(w["a"]), u8(w["b"]), e4(w["sfa"]), e4(w["sfb"]), torch.float32,
                                       sf_vec_size=16, ab_format=mm.MM_F4_E2M1)
    rc, ra, _ = gu.blockscaled_gemm_amax_atom(w["a"], w["b"], 5, w["sfa"], w["sfb"], F32, sf=16,
                                              sf_type=mm.MM_SF_E4M3FN)
    np.testing.assert_array_equal(bits(c), rc)
    assert float(amax.item()) == ra


def test_helper_errors_raise_before_launch():
    a = torch.zeros((64, 128), dtype=torch.uint8, device=DEV)
    with pytest.raises(TypeError):  # uint8 codes need a format
        mm.scaled_gemm(a, a, f32(1.0), f32(1.0), torch.float32)
    with pytest.raises(TypeError):  # scales must be float32
        mm.scaled_gemm(a, a, torch.ones(1, dtype=torch.float16, device=DEV), f32(1.0), torch.float32,
                       a_format=mm.MM_F8_E4M3FN, b_format=mm.MM_F8_E4M3FN)
    with pytest.raises(ValueError):  # a b with neither K nor N innermost is refused
        b = torch.zeros((2, 64, 256), dtype=torch.uint8, device=DEV)
        mm.scaled_bmm(b[:, :, :128].contiguous(), b[:, :, ::2], f32(1.0), f32(1.0), torch.float32, a_format=0,
                      b_format=0)
    # E4M3 factors with 32 values per factor: refused by the library (the page allows them with 16 only)
    w = datagen.set_nvfp4_l8_2048x2048x8192(1, 64, 64, 256, config=46)
    u8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    sfa = torch.zeros(mm_atom_bytes(64, 256, 1, 32), dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
    with pytest.raises(mm.MMError) as e:
        mm.blockscaled_gemm_amax(u8(w["a"]), u8(w["b"]), sfa, sfa, torch.float32, sf_vec_size=32,
                                 ab_format=mm.MM_F4_E2M1)
    assert e.value.status == mm.MM_ERR_UNSUPPORTED


def mm_atom_bytes(MN, K, L, sf):
    return L * -(-MN // 128) * -(-K // (4 * sf)) * 512


def test_square_column_major_mat2_matches_raw_abi():
    """A square weight's .t() (scaled_mm's column-major mat2 [K, N] with N == K) is read as its
    [N, K] transpose, told by its strides alone."""
    M, N, K = 96, 512, 512
    g = datagen.rng(47, 0)
    a = datagen.gauss_codes(g, (M, K), 64.0)
    w = datagen.gauss_codes(g, (N, K), 64.0)
    out = mm.scaled_gemm(fp8(a), fp8(w).t(), f32(0.5), f32(0.25), torch.bfloat16)
    raw = gu.scaled_gemm(a, E4M3FN, w, E4M3FN, K, 0.5, 0, 0.25, 0, BF16)
    np.testing.assert_array_equal(bits(out), raw)


@pytest.mark.parametrize("N", [71, 72])
def test_blockscaled_helper_fp4_c_matches_raw_abi(N):
    """FP4 C through the helper: [L, M, ceil(N/2)] bytes, bitwise the raw call's (odd N included)."""
    L, M, K, sf = 2, 96, 256, 32
    w = datagen.set_fp4_l8_2048x2048x8192(L, M, N, K, sf, config=48)
    u8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    c, amax = mm.blockscaled_gemm_amax(u8(w["a"]), u8(w["b"]), u8(w["sfa"]), u8(w["sfb"]), torch.float4_e2m1fn_x2,
                                       sf_vec_size=sf, ab_format=mm.MM_F4_E2M1)
    torch.cuda.synchronize()
    assert tuple(c.shape) == (L, M, -(-N // 2))
    es = -(-N // 2)
    tc = torch.full((L * M * es,), 0x5A, dtype=torch.uint8, device=DEV)
    tam = torch.zeros((1,), dtype=torch.float32, device=DEV)
    ta, tb, tsa, tsb = u8(w["a"]), u8(w["b"]), u8(w["sfa"]), u8(w["sfb"])
    st = mm.mm_blockscaled_gemm_amax_atom(M, N, K, L, ta.data_ptr(), tb.data_ptr(), mm.MM_F4_E2M1, tsa.data_ptr(),
                                          tsb.data_ptr(), mm.MM_SF_E8M0, sf, tc.data_ptr(), mm.MM_F4_E2M1,
                                          tam.data_ptr(), 0, gu.stream())
    assert st == mm.MM_OK, mm.mm_last_error()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(c.view(torch.uint8).cpu().numpy().reshape(-1), tc.cpu().numpy())
    assert float(amax.item()) == float(tam.item())
