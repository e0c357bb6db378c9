"""Helpers for the GPU parity tests: run the C ABI on device buffers, fetch bits."""
import numpy as np
import torch

import block_scaled_gemm_amd as mm

DEV = torch.device("cuda:0")
BITS_TORCH = {0: torch.uint8, 1: torch.uint8, 2: torch.int32, 3: torch.int16, 4: torch.int16}
BITS_NP = {0: np.uint8, 1: np.uint8, 2: np.uint32, 3: np.uint16, 4: np.uint16}


def dev_u8(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(DEV)


def dev_f32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.atleast_1d(np.asarray(x, dtype=np.float32)))).to(DEV)


def stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def scaled_gemm(a, a_fmt, b, b_fmt, K, sa, sa_mode, sb, sb_mode, d_type, scale_result=None, fast=False,
                ldd=None, d_fill=0x5A):
    """a [M, lda], b [N, ldb] uint8 codes (numpy); returns the output bits [M, N] (numpy)."""
    M, lda = a.shape
    N, ldb = b.shape
    ldd = ldd or N
    ta, tb = dev_u8(a), dev_u8(b)
    tsa, tsb = dev_f32(sa), dev_f32(sb)
    tsr = dev_f32(scale_result) if scale_result is not None else None
    es = np.dtype(BITS_NP[d_type]).itemsize
    # output buffer prefilled with junk: previous contents must never matter
    td = torch.full((max(M, 1) * ldd * es,), d_fill, dtype=torch.uint8, device=DEV)
    st = mm.mm_scaled_gemm(M, N, K, ta.data_ptr(), a_fmt, lda, tb.data_ptr(), b_fmt, ldb, tsa.data_ptr(), sa_mode,
                           tsb.data_ptr(), sb_mode, tsr.data_ptr() if tsr is not None else 0, td.data_ptr(), d_type,
                           ldd, int(fast), stream())
    assert st == mm.MM_OK, (st, mm.mm_last_error())
    torch.cuda.synchronize()
    out = td.cpu().numpy().view(BITS_NP[d_type])[: M * ldd].reshape(M, ldd)[:, :N]
    return np.ascontiguousarray(out)


def blockscaled_gemm_amax(a, b, fmt, sfa, sfb, c_type, with_amax=True, with_index=True):
    """a [L, M, K], b [L, N, K] uint8 codes; returns (c bits [L, M, N], amax float or None, index or None)."""
    L, M, K = a.shape
    N = b.shape[1]
    ta, tb = dev_u8(a), dev_u8(b)
    tsa = torch.from_numpy(np.ascontiguousarray(sfa, dtype=np.float32)).to(DEV)
    tsb = torch.from_numpy(np.ascontiguousarray(sfb, dtype=np.float32)).to(DEV)
    es = np.dtype(BITS_NP[c_type]).itemsize
    tc = torch.full((max(L * M * N, 1) * es,), 0x5A, dtype=torch.uint8, device=DEV)
    tam = torch.full((1,), 123.0, dtype=torch.float32, device=DEV)
    tix = torch.full((1,), 777, dtype=torch.int64, device=DEV)
    st = mm.mm_blockscaled_gemm_amax(M, N, K, L, ta.data_ptr(), tb.data_ptr(), fmt, tsa.data_ptr(), tsb.data_ptr(),
                                     32, tc.data_ptr(), c_type, tam.data_ptr() if with_amax else 0,
                                     tix.data_ptr() if with_index else 0, stream())
    assert st == mm.MM_OK, (st, mm.mm_last_error())
    torch.cuda.synchronize()
    c = tc.cpu().numpy().view(BITS_NP[c_type])[: L * M * N].reshape(L, M, N)
    return (np.ascontiguousarray(c), float(tam.item()) if with_amax else None,
            int(tix.item()) if with_index else None)


def blockscaled_gemm_amax_atom(a, b, fmt, sfa, sfb, c_type, with_amax=True, with_index=True, sf=32,
                               sf_type=None):
    """As blockscaled_gemm_amax with E8M0 scale bytes in the page's storage shape (fmt 5: FP4 pairs)."""
    L, M, K = a.shape
    N = b.shape[1]
    if fmt == mm.MM_F4_E2M1:
        K *= 2
    ta, tb, tsa, tsb = dev_u8(a), dev_u8(b), dev_u8(sfa), dev_u8(sfb)
    es = np.dtype(BITS_NP[c_type]).itemsize
    tc = torch.full((max(L * M * N, 1) * es,), 0x5A, dtype=torch.uint8, device=DEV)
    tam = torch.full((1,), 123.0, dtype=torch.float32, device=DEV)
    tix = torch.full((1,), 777, dtype=torch.int64, device=DEV)
    st = mm.mm_blockscaled_gemm_amax_atom(M, N, K, L, ta.data_ptr(), tb.data_ptr(), fmt, tsa.data_ptr(),
                                          tsb.data_ptr(), mm.MM_SF_E8M0 if sf_type is None else sf_type, sf,
                                          tc.data_ptr(), c_type,
                                          tam.data_ptr() if with_amax else 0, tix.data_ptr() if with_index else 0,
                                          stream())
    assert st == mm.MM_OK, (st, mm.mm_last_error())
    torch.cuda.synchronize()
    c = tc.cpu().numpy().view(BITS_NP[c_type])[: L * M * N].reshape(L, M, N)
    return (np.ascontiguousarray(c), float(tam.item()) if with_amax else None,
            int(tix.item()) if with_index else None)


def scaled_gemm_grouped(a, a_fmt, b, b_fmt, sizes, offsets, sa, sb, d_type, scale_result=None, fast=False):
    """a [batch_sum, K], b [G, N, K] uint8 codes; int32 sizes / offsets; returns d bits [batch_sum, N]
    (rows of no group keep the fill pattern 0x5A)."""
    batch_sum, K = a.shape
    G, N, _ = b.shape
    ta, tb = dev_u8(a), dev_u8(b)
    ts = torch.from_numpy(np.ascontiguousarray(sizes, dtype=np.int32)).to(DEV)
    to = torch.from_numpy(np.ascontiguousarray(offsets, dtype=np.int32)).to(DEV)
    tsa, tsb = dev_f32([sa]), dev_f32([sb])
    tsr = dev_f32([scale_result]) if scale_result is not None else None
    es = np.dtype(BITS_NP[d_type]).itemsize
    td = torch.full((max(batch_sum * N, 1) * es,), 0x5A, dtype=torch.uint8, device=DEV)
    st = mm.mm_scaled_gemm_grouped(batch_sum, N, K, G, ta.data_ptr(), a_fmt, K, tb.data_ptr(), b_fmt, K, N * K,
                                   ts.data_ptr(), to.data_ptr(), tsa.data_ptr(), tsb.data_ptr(),
                                   tsr.data_ptr() if tsr is not None else 0, td.data_ptr(), d_type, N, int(fast),
                                   stream())
    assert st == mm.MM_OK, (st, mm.mm_last_error())
    torch.cuda.synchronize()
    return np.ascontiguousarray(td.cpu().numpy().view(BITS_NP[d_type])[: batch_sum * N].reshape(batch_sum, N))


def debug_convert(x: np.ndarray, dtype: int) -> np.ndarray:
    tx = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    es = np.dtype(BITS_NP[dtype]).itemsize
    ty = torch.empty((x.size * es,), dtype=torch.uint8, device=DEV)
    st = mm.mm_debug_convert(tx.data_ptr(), ty.data_ptr(), dtype, x.size, stream())
    assert st == mm.MM_OK, (st, mm.mm_last_error())
    torch.cuda.synchronize()
    return ty.cpu().numpy().view(BITS_NP[dtype])


def scaled_gemm_bias(a, a_fmt, b, b_fmt, K, sa, sa_mode, sb, sb_mode, bias_bits, d_type, fast=False, ldd=None):
    """mm_scaled_gemm_bias; bias_bits [N] are the bit patterns of the bias in d_type."""
    M, lda = a.shape
    N, ldb = b.shape
    ldd = ldd or N
    ta, tb = dev_u8(a), dev_u8(b)
    tsa, tsb = dev_f32(sa), dev_f32(sb)
    es = np.dtype(BITS_NP[d_type]).itemsize
    tbias = torch.from_numpy(np.ascontiguousarray(bias_bits, dtype=BITS_NP[d_type]).view(np.uint8).copy()).to(DEV)
    td = torch.full((max(M, 1) * ldd * es,), 0x5A, dtype=torch.uint8, device=DEV)
    st = mm.mm_scaled_gemm_bias(M, N, K, ta.data_ptr(), a_fmt, lda, tb.data_ptr(), b_fmt, ldb, tsa.data_ptr(),
                                sa_mode, tsb.data_ptr(), sb_mode, tbias.data_ptr(), td.data_ptr(), d_type, ldd,
                                int(fast), stream())
    assert st == mm.MM_OK, (st, mm.mm_last_error())
    torch.cuda.synchronize()
    out = td.cpu().numpy().view(BITS_NP[d_type])[: M * ldd].reshape(M, ldd)[:, :N]
    return np.ascontiguousarray(out)


def scaled_gemm_batched(a, a_fmt, b, b_fmt, K, sa, sb, d_type, scale_result=None, fast=False, pad_a=0, pad_b=0,
                        pad_d=0):
    """mm_scaled_gemm_batched on a [L, M, lda], b [L, N, ldb] uint8 codes, items pad_* bytes / elements apart
    beyond their size (pad_a, pad_b multiples of 16). Returns the output bits [L, M, N]."""
    L, M, lda = a.shape
    N, ldb = b.shape[1], b.shape[2]
    sa_bytes, sb_bytes = M * lda + pad_a, N * ldb + pad_b
    abuf = np.zeros((L, sa_bytes), np.uint8); abuf[:, : M * lda] = a.reshape(L, -1)
    bbuf = np.zeros((L, sb_bytes), np.uint8); bbuf[:, : N * ldb] = b.reshape(L, -1)
    ta, tb = dev_u8(abuf), dev_u8(bbuf)
    tsa, tsb = dev_f32(sa), dev_f32(sb)
    tsr = dev_f32(scale_result) if scale_result is not None else None
    es = np.dtype(BITS_NP[d_type]).itemsize
    stride_d = M * N + pad_d
    td = torch.full((max(L * stride_d, 1) * es,), 0x5A, dtype=torch.uint8, device=DEV)
    st = mm.mm_scaled_gemm_batched(L, M, N, K, ta.data_ptr(), a_fmt, lda, sa_bytes, tb.data_ptr(), b_fmt, ldb,
                                   sb_bytes, tsa.data_ptr(), tsb.data_ptr(),
                                   tsr.data_ptr() if tsr is not None else 0, td.data_ptr(), d_type, N, stride_d,
                                   int(fast), stream())
    assert st == mm.MM_OK, (st, mm.mm_last_error())
    torch.cuda.synchronize()
    out = td.cpu().numpy().view(BITS_NP[d_type])[: L * stride_d].reshape(L, stride_d)[:, : M * N]
    return np.ascontiguousarray(out.reshape(L, M, N))


def transpose_u8(src, ld_src=None, ld_dst=None, fill=0x5A):
    """src [L, R, C] uint8 (numpy); rows padded to ld_src, dst rows of ld_dst; returns dst [L, C, ld_dst]."""
    L, R, C = src.shape
    ld_src = ld_src or C
    ld_dst = ld_dst or R
    s = np.full((L, R, ld_src), 0xA5, np.uint8)
    s[:, :, :C] = src
    ts = dev_u8(s)
    td = torch.full((max(L * C * ld_dst, 1),), fill, dtype=torch.uint8, device=DEV)
    st = mm.mm_transpose_u8(L, R, C, ts.data_ptr(), ld_src, R * ld_src, td.data_ptr(), ld_dst, C * ld_dst,
                            stream())
    assert st == mm.MM_OK, (st, mm.mm_last_error())
    torch.cuda.synchronize()
    return td.cpu().numpy()[: L * C * ld_dst].reshape(L, C, ld_dst)


def scaled_gemm_grouped_layout(a, a_fmt, b, b_fmt, sizes, offsets, sa, sb, d_type, transpose_a, transpose_b,
                               scale_result=None, fast=False, fill=0x5A):
    """Any of the four layouts on uint8 codes (numpy, contiguous rows); returns d bits ([batch_sum, N], or
    [G, N, K] with transpose_a; untouched elements keep the fill pattern)."""
    G = len(sizes)
    if transpose_a:
        batch_sum, N = a.shape
        K = b.shape[0] if transpose_b else b.shape[1]
        shape = (G, N, K)
    else:
        batch_sum, K = a.shape
        N = b.shape[1] if transpose_b else b.shape[2]
        shape = (batch_sum, N)
    ta, tb = dev_u8(a), dev_u8(b)
    ts = torch.from_numpy(np.ascontiguousarray(sizes, dtype=np.int32)).to(DEV)
    to = torch.from_numpy(np.ascontiguousarray(offsets, dtype=np.int32)).to(DEV)
    tsa, tsb = dev_f32([sa]), dev_f32([sb])
    tsr = dev_f32([scale_result]) if scale_result is not None else None
    es = np.dtype(BITS_NP[d_type]).itemsize
    n_out = int(np.prod(shape))
    td = torch.full((max(n_out, 1) * es,), fill, dtype=torch.uint8, device=DEV)
    st, nbytes = mm.mm_grouped_workspace_bytes(batch_sum, N, K, G, transpose_a, transpose_b)
    assert st == mm.MM_OK
    ws = torch.full((max(nbytes, 1),), 0xC3, dtype=torch.uint8, device=DEV)  # contents never matter
    ldb = b.shape[-1]
    stride_b = 0 if transpose_a else b.shape[1] * b.shape[2]
    st = mm.mm_scaled_gemm_grouped_layout(batch_sum, N, K, G, transpose_a, transpose_b, ta.data_ptr(), a_fmt,
                                          a.shape[1], tb.data_ptr(), b_fmt, ldb, stride_b, ts.data_ptr(),
                                          to.data_ptr(), tsa.data_ptr(), tsb.data_ptr(),
                                          tsr.data_ptr() if tsr is not None else 0, td.data_ptr(), d_type,
                                          shape[-1], N * K if transpose_a else 0, ws.data_ptr(), nbytes, int(fast),
                                          stream())
    assert st == mm.MM_OK, (st, mm.mm_last_error())
    torch.cuda.synchronize()
    return np.ascontiguousarray(td.cpu().numpy().view(BITS_NP[d_type])[:n_out].reshape(shape))
