"""CPU checks of the Python helpers' argument marshalling (no GPU needed).

The helpers compute pitches, modes and output shapes from the tensors and hand
them to the C ABI. Here the C calls are either made with MM_TEST_FORCE_FAIL=launch
(the library validates everything, then returns MM_ERR_DEVICE before any HIP
call) or replaced by a recorder, so what reaches the ABI can be checked
without a device.
"""
import pytest
import torch

import block_scaled_gemm_amd as mm


@pytest.fixture
def no_stream(monkeypatch):
    # torch has no current stream without a GPU: pass the null stream
    monkeypatch.setattr(mm, "_stream", lambda: 0)


def fp8_cpu(shape):
    return torch.zeros(shape, dtype=torch.uint8).view(torch.float8_e4m3fn)


@pytest.mark.parametrize("K,N", [(256, 256), (128, 384), (384, 128)], ids=["square", "wide", "tall"])
def test_column_major_mat2_is_read_as_its_transpose(K, N, no_stream, monkeypatch):
    """scaled_mm's mat2 [K, N] in column-major order (a weight's .t()) is told by its strides alone,
    square shapes included, and reaches the ABI as b [N, K] with row pitch K."""
    seen = {}

    def record(M_, N_, K_, a, a_type, lda, b, b_type, ldb, *rest):
        seen.update(M=M_, N=N_, K=K_, lda=lda, ldb=ldb, b=b)
        return mm.MM_OK

    monkeypatch.setattr(mm, "mm_scaled_gemm", record)
    a = fp8_cpu((64, K))
    w = fp8_cpu((N, K))          # the [N, K] weight
    mat2 = w.t()                 # [K, N], strides (1, K)
    one = torch.ones(1, dtype=torch.float32)
    mm.scaled_gemm(a, mat2, one, one, torch.float32)
    assert seen == dict(M=64, N=N, K=K, lda=K, ldb=K, b=w.data_ptr())


def test_row_major_b_is_not_transposed(no_stream, monkeypatch):
    seen = {}

    def record(M_, N_, K_, a, a_type, lda, b, b_type, ldb, *rest):
        seen.update(N=N_, K=K_, ldb=ldb)
        return mm.MM_OK

    monkeypatch.setattr(mm, "mm_scaled_gemm", record)
    a = fp8_cpu((32, 256))
    b = fp8_cpu((256, 256))      # [N, K] row-major, square
    one = torch.ones(1, dtype=torch.float32)
    mm.scaled_gemm(a, b, one, one, torch.float32)
    assert seen == dict(N=256, K=256, ldb=256)


def test_square_column_major_mat2_passes_validation(no_stream, monkeypatch):
    monkeypatch.setenv("MM_TEST_FORCE_FAIL", "launch")
    a = fp8_cpu((64, 512))
    mat2 = fp8_cpu((512, 512)).t()
    one = torch.ones(1, dtype=torch.float32)
    with pytest.raises(mm.MMError) as e:
        mm.scaled_gemm(a, mat2, one, one, torch.bfloat16)
    assert e.value.status == mm.MM_ERR_DEVICE and "forced" in str(e.value)


@pytest.mark.parametrize("N", [71, 72, 1])
def test_fp4_c_is_allocated_two_values_per_byte(N, no_stream, monkeypatch):
    """An FP4 C has rows of ceil(N/2) bytes, the page's (M, ceil(N/2), L) tensor, n-major."""
    seen = {}

    def record(M_, N_, K_, L_, a, b, ab_type, sfa, sfb, sf_type, sf_vec, c, c_type, amax, idx, stream):
        seen.update(M=M_, N=N_, K=K_, L=L_, ab_type=ab_type, c=c, c_type=c_type, sf_vec=sf_vec)
        return mm.MM_OK

    monkeypatch.setattr(mm, "mm_blockscaled_gemm_amax_atom", record)
    L, M, K, sf = 2, 40, 256, 32
    a = torch.zeros((L, M, K // 2), dtype=torch.uint8)
    b = torch.zeros((L, N, K // 2), dtype=torch.uint8)
    sfa = torch.zeros(L * -(-M // 128) * -(-K // (4 * sf)) * 512, dtype=torch.uint8)
    sfb = torch.zeros(L * -(-N // 128) * -(-K // (4 * sf)) * 512, dtype=torch.uint8)
    c, amax = mm.blockscaled_gemm_amax(a, b, sfa, sfb, torch.float4_e2m1fn_x2, sf_vec_size=sf,
                                       ab_format=mm.MM_F4_E2M1)
    assert tuple(c.shape) == (L, M, -(-N // 2)) and c.element_size() == 1 and c.is_contiguous()
    assert seen == dict(M=M, N=N, K=K, L=L, ab_type=mm.MM_F4_E2M1, c=c.data_ptr(), c_type=mm.MM_F4_E2M1,
                        sf_vec=sf)
