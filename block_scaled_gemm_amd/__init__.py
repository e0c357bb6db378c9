"""Python binding of libmmfp8 (FP8 scaled GEMM and block-scaled GEMM + amax on MI355X).

Argument marshalling only: every step of the computation runs in the gfx950
kernels behind the C ABI declared in include/mm.h. torch is used for device
memory and the current stream. Importing the package loads libmmfp8.so from
this directory and raises if it is missing: there is no fallback path.

Raw C-ABI wrappers (same names as the C functions, integer pointers):
``mm_scaled_gemm``, ``mm_scaled_gemm_bias``, ``mm_scaled_gemm_batched``, ``mm_scaled_gemm_grouped``,
``mm_scaled_gemm_grouped_layout``, ``mm_grouped_workspace_bytes``, ``mm_transpose_u8``,
``mm_blockscaled_gemm_amax``, ``mm_blockscaled_gemm_amax_atom``,
``mm_debug_convert``, ``mm_last_error``, ``mm_version``. Tensor-level helpers:
``scaled_gemm`` (with an optional bias), ``scaled_bmm``, ``scaled_grouped_mm`` and
``blockscaled_gemm_amax`` (fp32 factors, or the page-native E8M0 bytes).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmmfp8.so")

MM_OK, MM_ERR_INVALID_ARGUMENT, MM_ERR_UNSUPPORTED, MM_ERR_MISALIGNED, MM_ERR_DEVICE = 0, 1, 2, 3, 4
MM_F8_E4M3FN, MM_F8_E5M2, MM_F32, MM_BF16, MM_F16, MM_F4_E2M1 = 0, 1, 2, 3, 4, 5
MM_SCALE_TENSOR, MM_SCALE_1x128, MM_SCALE_128x128 = 0, 1, 2
MM_SF_E8M0, MM_SF_E4M3FN = 0, 1
MM_NOALLOC_SCRATCH_BYTES = 160 << 20  # the scratch array of mm_scaled_gemm_grouped_layout_noalloc

# One HIP runtime per process. PyTorch ships its own HIP runtime with the same
# soname as the system one libmmfp8 is linked against; loaded first, it also
# serves libmmfp8. Loaded the other way round, the process ends up with two
# runtimes, and the one initialised second finds no GPU. So torch, when it is
# installed, is imported before the library.
try:
    import torch as _torch  # noqa: F401
except ImportError:
    _torch = None

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m block_scaled_gemm_amd.build` "
                      "(or __graft_entry__.build()); there is no CPU fallback")
_lib = ctypes.CDLL(LIB_PATH)

_P, _I64, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_lib.mm_scaled_gemm.argtypes = [_I64, _I64, _I64, _P, _I, _I64, _P, _I, _I64, _P, _I, _P, _I, _P, _P, _I, _I64, _I, _P]
_lib.mm_scaled_gemm.restype = _I
_lib.mm_scaled_gemm_bias.argtypes = [_I64, _I64, _I64, _P, _I, _I64, _P, _I, _I64, _P, _I, _P, _I, _P, _P, _I, _I64,
                                     _I, _P]
_lib.mm_scaled_gemm_bias.restype = _I
_lib.mm_scaled_gemm_batched.argtypes = [_I64, _I64, _I64, _I64, _P, _I, _I64, _I64, _P, _I, _I64, _I64, _P, _P, _P,
                                        _P, _I, _I64, _I64, _I, _P]
_lib.mm_scaled_gemm_batched.restype = _I
_lib.mm_scaled_gemm_grouped.argtypes = [_I64, _I64, _I64, _I64, _P, _I, _I64, _P, _I, _I64, _I64, _P, _P, _P, _P,
                                        _P, _P, _I, _I64, _I, _P]
_lib.mm_scaled_gemm_grouped.restype = _I
_lib.mm_blockscaled_gemm_amax.argtypes = [_I64, _I64, _I64, _I64, _P, _P, _I, _P, _P, _I, _P, _I, _P, _P, _P]
_lib.mm_blockscaled_gemm_amax.restype = _I
_lib.mm_blockscaled_gemm_amax_atom.argtypes = [_I64, _I64, _I64, _I64, _P, _P, _I, _P, _P, _I, _I, _P, _I, _P, _P,
                                               _P]
_lib.mm_blockscaled_gemm_amax_atom.restype = _I
_lib.mm_transpose_u8.argtypes = [_I64, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _P]
_lib.mm_transpose_u8.restype = _I
_lib.mm_grouped_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, _I, _I, ctypes.POINTER(ctypes.c_uint64)]
_lib.mm_grouped_workspace_bytes.restype = _I
_lib.mm_scaled_gemm_grouped_layout.argtypes = [_I64, _I64, _I64, _I64, _I, _I, _P, _I, _I64, _P, _I, _I64, _I64,
                                               _P, _P, _P, _P, _P, _P, _I, _I64, _I64, _P, ctypes.c_uint64, _I, _P]
_lib.mm_scaled_gemm_grouped_layout.restype = _I
_lib.mm_scaled_gemm_grouped_layout_noalloc.argtypes = [_I64, _I64, _I64, _I64, _I, _I, _P, _I, _I64, _P, _I, _I64,
                                                       _I64, _P, _P, _P, _P, _P, _P, _I, _I64, _I64, _I, _P]
_lib.mm_scaled_gemm_grouped_layout_noalloc.restype = _I
_lib.mm_debug_convert.argtypes = [_P, _P, _I, _I64, _P]
_lib.mm_debug_convert.restype = _I
_lib.mm_debug_mfma_gemm.argtypes = [_I64, _I64, _I64, _P, _P, _I, _P, _P, _P, _P]
_lib.mm_debug_mfma_gemm.restype = _I
_lib.mm_last_error.restype = ctypes.c_char_p
_lib.mm_version.restype = ctypes.c_char_p

EXPORTED = ("mm_scaled_gemm", "mm_scaled_gemm_bias", "mm_scaled_gemm_batched", "mm_scaled_gemm_grouped",
            "mm_scaled_gemm_grouped_layout", "mm_scaled_gemm_grouped_layout_noalloc", "mm_grouped_workspace_bytes",
            "mm_transpose_u8",
            "mm_blockscaled_gemm_amax",
            "mm_blockscaled_gemm_amax_atom", "mm_last_error", "mm_version", "mm_debug_convert", "mm_debug_mfma_gemm")


class MMError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


def mm_last_error() -> str:
    return _lib.mm_last_error().decode()


def mm_version() -> str:
    return _lib.mm_version().decode()


def mm_scaled_gemm(M, N, K, a, a_type, lda, b, b_type, ldb, scale_a, sa_mode, scale_b, sb_mode,
                   scale_result, d, d_type, ldd, use_fast_accum, stream) -> int:
    """Raw call of the C function; pointers and the stream are integers (0 = NULL). Returns the status."""
    return _lib.mm_scaled_gemm(M, N, K, a or None, a_type, lda, b or None, b_type, ldb, scale_a or None, sa_mode,
                               scale_b or None, sb_mode, scale_result or None, d or None, d_type, ldd,
                               int(use_fast_accum), stream or None)


def mm_scaled_gemm_bias(M, N, K, a, a_type, lda, b, b_type, ldb, scale_a, sa_mode, scale_b, sb_mode, bias,
                        d, d_type, ldd, use_fast_accum, stream) -> int:
    """Raw call of the C function; pointers and the stream are integers (0 = NULL). Returns the status."""
    return _lib.mm_scaled_gemm_bias(M, N, K, a or None, a_type, lda, b or None, b_type, ldb, scale_a or None,
                                    sa_mode, scale_b or None, sb_mode, bias or None, d or None, d_type, ldd,
                                    int(use_fast_accum), stream or None)


def mm_scaled_gemm_batched(L, M, N, K, a, a_type, lda, stride_a, b, b_type, ldb, stride_b, scale_a, scale_b,
                           scale_result, d, d_type, ldd, stride_d, use_fast_accum, stream) -> int:
    """Raw call of the C function; pointers and the stream are integers (0 = NULL). Returns the status."""
    return _lib.mm_scaled_gemm_batched(L, M, N, K, a or None, a_type, lda, stride_a, b or None, b_type, ldb,
                                       stride_b, scale_a or None, scale_b or None, scale_result or None,
                                       d or None, d_type, ldd, stride_d, int(use_fast_accum), stream or None)


def mm_scaled_gemm_grouped(batch_sum, N, K, G, a, a_type, lda, b, b_type, ldb, stride_b, batch_sizes,
                           batch_offsets, scale_a, scale_b, scale_result, d, d_type, ldd, use_fast_accum,
                           stream) -> int:
    """Raw call of the C function; pointers and the stream are integers (0 = NULL). Returns the status."""
    return _lib.mm_scaled_gemm_grouped(batch_sum, N, K, G, a or None, a_type, lda, b or None, b_type, ldb, stride_b,
                                       batch_sizes or None, batch_offsets or None, scale_a or None, scale_b or None,
                                       scale_result or None, d or None, d_type, ldd, int(use_fast_accum),
                                       stream or None)


def mm_transpose_u8(L, R, C, src, ld_src, stride_src, dst, ld_dst, stride_dst, stream) -> int:
    """Raw call of the C function; pointers and the stream are integers (0 = NULL). Returns the status."""
    return _lib.mm_transpose_u8(L, R, C, src or None, ld_src, stride_src, dst or None, ld_dst, stride_dst,
                                stream or None)


def mm_grouped_workspace_bytes(batch_sum, N, K, G, transpose_a, transpose_b):
    """Raw call of the C function. Returns (status, bytes)."""
    n = ctypes.c_uint64(0)
    st = _lib.mm_grouped_workspace_bytes(batch_sum, N, K, G, int(transpose_a), int(transpose_b), ctypes.byref(n))
    return st, n.value


def mm_scaled_gemm_grouped_layout(batch_sum, N, K, G, transpose_a, transpose_b, a, a_type, lda, b, b_type, ldb,
                                  stride_b, batch_sizes, batch_offsets, scale_a, scale_b, scale_result, d, d_type,
                                  ldd, stride_d, workspace, workspace_bytes, use_fast_accum, stream) -> int:
    """Raw call of the C function; pointers and the stream are integers (0 = NULL). Returns the status."""
    return _lib.mm_scaled_gemm_grouped_layout(batch_sum, N, K, G, int(transpose_a), int(transpose_b), a or None,
                                              a_type, lda, b or None, b_type, ldb, stride_b, batch_sizes or None,
                                              batch_offsets or None, scale_a or None, scale_b or None,
                                              scale_result or None, d or None, d_type, ldd, stride_d,
                                              workspace or None, workspace_bytes, int(use_fast_accum),
                                              stream or None)


def mm_scaled_gemm_grouped_layout_noalloc(batch_sum, N, K, G, transpose_a, transpose_b, a, a_type, lda, b, b_type,
                                          ldb, stride_b, batch_sizes, batch_offsets, scale_a, scale_b, scale_result, d,
                                          d_type, ldd, stride_d, use_fast_accum, stream) -> int:
    """Raw call of the C function (the library's own scratch array in place of a workspace); pointers and the
    stream are integers (0 = NULL). Returns the status."""
    return _lib.mm_scaled_gemm_grouped_layout_noalloc(batch_sum, N, K, G, int(transpose_a), int(transpose_b),
                                                      a or None, a_type, lda, b or None, b_type, ldb, stride_b,
                                                      batch_sizes or None, batch_offsets or None, scale_a or None,
                                                      scale_b or None, scale_result or None, d or None, d_type, ldd,
                                                      stride_d, int(use_fast_accum), stream or None)


def mm_debug_mfma_gemm(M, N, K, a, b, ab_type, sfa, sfb, d, stream) -> int:
    """Test hook (raw call): a GEMM summed by the scaled FP8 / FP4 MFMA, for measuring its precision."""
    return _lib.mm_debug_mfma_gemm(M, N, K, a or None, b or None, ab_type, sfa or None, sfb or None, d or None,
                                   stream or None)


def mm_blockscaled_gemm_amax(M, N, K, L, a, b, ab_type, sfa, sfb, sf_vec_size, c, c_type, amax, amax_index,
                             stream) -> int:
    """Raw call of the C function; pointers and the stream are integers (0 = NULL). Returns the status."""
    return _lib.mm_blockscaled_gemm_amax(M, N, K, L, a or None, b or None, ab_type, sfa or None, sfb or None,
                                         sf_vec_size, c or None, c_type, amax or None, amax_index or None,
                                         stream or None)


def mm_blockscaled_gemm_amax_atom(M, N, K, L, a, b, ab_type, sfa, sfb, sf_type, sf_vec_size, c, c_type, amax,
                                  amax_index, stream) -> int:
    """Raw call of the C function; pointers and the stream are integers (0 = NULL). Returns the status."""
    return _lib.mm_blockscaled_gemm_amax_atom(M, N, K, L, a or None, b or None, ab_type, sfa or None, sfb or None,
                                              sf_type, sf_vec_size, c or None, c_type, amax or None,
                                              amax_index or None, stream or None)


def mm_debug_convert(x, y, dtype, n, stream) -> int:
    return _lib.mm_debug_convert(x or None, y or None, dtype, n, stream or None)


def _check(status: int):
    if status != MM_OK:
        raise MMError(status, mm_last_error())


# ------------------------------------------------------------------ tensor helpers

def _torch():
    import torch
    return torch


def dtype_code(dt) -> int:
    torch = _torch()
    table = {torch.float8_e4m3fn: MM_F8_E4M3FN, torch.float8_e5m2: MM_F8_E5M2, torch.float32: MM_F32,
             torch.bfloat16: MM_BF16, torch.float16: MM_F16}
    if hasattr(torch, "float4_e2m1fn_x2"):
        table[torch.float4_e2m1fn_x2] = MM_F4_E2M1
    if dt not in table:
        raise TypeError(f"unsupported dtype {dt}")
    return table[dt]


def _fp8_code(t, fmt):
    torch = _torch()
    if t.dtype == torch.uint8:
        if fmt is None:
            raise TypeError("uint8 operands need an explicit format (MM_F8_E4M3FN, MM_F8_E5M2 or MM_F4_E2M1)")
        return fmt
    return dtype_code(t.dtype)


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _rows(t):
    """(row pitch in elements) of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D tensor with contiguous rows")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def scaled_gemm(a, b, scale_a, scale_b, out_dtype, scale_result=None, use_fast_accum=False, out=None,
                a_format=None, b_format=None, bias=None):
    """d = (a * scale_a) @ (b * scale_b)^T (+ bias) on the current stream.

    a: [M, K] FP8 (or uint8 codes with a_format) with contiguous rows.
    b: [N, K] FP8 with contiguous rows, or torch._scaled_mm's column-major
       mat2 [K, N] (detected by its strides and read as its [N, K] transpose).
    scale_a / scale_b: fp32 tensors, per-tensor (one element), 1x128 [M, ceil(K/128)],
       or for b 1x128 [N, ceil(K/128)] / 128x128 [ceil(N/128), ceil(K/128)].
    bias: optional contiguous [N] tensor of out_dtype (f32, bf16 or f16), added
       after the scales (mm_scaled_gemm_bias).
    """
    torch = _torch()
    if b.dim() == 2 and a.dim() == 2 and b.shape[0] == a.shape[1] and b.shape[1] > 1 and b.stride(0) == 1 and \
            b.stride(1) >= b.shape[0]:
        b = b.t()  # scaled_mm's column-major mat2 [K, N] (told by its strides alone) -> its [N, K] rows
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError(f"shape mismatch: a {tuple(a.shape)}, b {tuple(b.shape)}")
    kb = -(-K // 128)

    def mode_of(s, rows):
        if s.numel() == 1:
            return MM_SCALE_TENSOR
        if tuple(s.shape) == (rows, kb):
            return MM_SCALE_1x128
        if tuple(s.shape) == (-(-rows // 128), kb):
            return MM_SCALE_128x128
        raise ValueError(f"scale of shape {tuple(s.shape)} fits no scale mode")

    sa_mode = mode_of(scale_a, M)
    sb_mode = mode_of(scale_b, N)
    for s in (scale_a, scale_b):
        if s.dtype != torch.float32 or not s.is_contiguous():
            raise TypeError("scales must be contiguous float32 tensors")
    d_type = dtype_code(out_dtype)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    if bias is not None:
        if bias.dtype != out_dtype or tuple(bias.shape) != (N,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous [N] tensor of out_dtype")
        if scale_result is not None:
            raise ValueError("scale_result applies to FP8 outputs, which take no bias")
        st = mm_scaled_gemm_bias(M, N, K, a.data_ptr(), _fp8_code(a, a_format), _rows(a) if M else K,
                                 b.data_ptr(), _fp8_code(b, b_format), _rows(b) if N else K,
                                 scale_a.data_ptr(), sa_mode, scale_b.data_ptr(), sb_mode, bias.data_ptr(),
                                 out.data_ptr(), d_type, _rows(out) if M else N, use_fast_accum, _stream())
        _check(st)
        return out
    sr = 0 if scale_result is None else scale_result.data_ptr()
    st = mm_scaled_gemm(M, N, K, a.data_ptr(), _fp8_code(a, a_format), _rows(a) if M else K,
                        b.data_ptr(), _fp8_code(b, b_format), _rows(b) if N else K,
                        scale_a.data_ptr(), sa_mode, scale_b.data_ptr(), sb_mode, sr,
                        out.data_ptr(), d_type, _rows(out) if M else N, use_fast_accum, _stream())
    _check(st)
    return out


def scaled_bmm(a, b, scale_a, scale_b, out_dtype, scale_result=None, use_fast_accum=False, out=None,
               a_format=None, b_format=None, trans_b=True):
    """d[l] = (a[l] * scale_a) @ B[l] * scale_b for every l, on the current stream.

    a: [L, M, K] FP8 with K innermost. b: [L, N, K] (trans_b, B[l] = b[l]^T) or
    torch.bmm's [L, K, N] (trans_b False, B[l] = b[l]). As for BmmFP8FwdOp, b's
    strides decide whether it is copied: a b whose K axis is not innermost is
    first transposed into a new [L, N, K] buffer (mm_transpose_u8, one extra
    read and write of b). scale_a / scale_b: one fp32 element each, shared by
    the batch. Returns d [L, M, N] of out_dtype.
    """
    torch = _torch()
    if b.dim() == 3 and not trans_b:
        b = b.transpose(1, 2)  # the [L, N, K] view of b [L, K, N]
    if a.dim() != 3 or b.dim() != 3 or a.shape[0] != b.shape[0] or a.shape[2] != b.shape[2]:
        raise ValueError(f"expected a [L, M, K] and b [L, N, K] (or [L, K, N]), got {tuple(a.shape)} and "
                         f"{tuple(b.shape)}")
    L, M, K = a.shape
    N = b.shape[1]
    if a.shape[2] > 1 and a.stride(2) != 1:
        raise ValueError("a needs K innermost")
    if K > 1 and b.stride(2) != 1:
        if N > 1 and b.stride(1) != 1:
            raise ValueError("b needs K or N innermost")
        kp = -(-K // 16) * 16
        bt = torch.empty((L, N, kp), dtype=torch.uint8, device=b.device)
        _check(mm_transpose_u8(L, K, N, b.data_ptr(), b.stride(2), b.stride(0), bt.data_ptr(), kp, N * kp,
                               _stream()))
        b_format = _fp8_code(b, b_format)
        b = bt[:, :, :K]
    for s in (scale_a, scale_b):
        if s.dtype != torch.float32 or s.numel() != 1:
            raise TypeError("scale_a and scale_b must be one-element float32 tensors")
    if out is None:
        out = torch.empty((L, M, N), dtype=out_dtype, device=a.device)
    if out.dim() != 3 or (N > 1 and out.stride(2) != 1):
        raise ValueError("out must be [L, M, N] with contiguous rows")
    sr = 0 if scale_result is None else scale_result.data_ptr()
    lda = a.stride(1) if M > 1 else K
    ldb = b.stride(1) if N > 1 else K
    ldd = out.stride(1) if M > 1 else N
    st = mm_scaled_gemm_batched(L, M, N, K, a.data_ptr(), _fp8_code(a, a_format), lda, a.stride(0),
                                b.data_ptr(), _fp8_code(b, b_format), ldb, b.stride(0),
                                scale_a.data_ptr(), scale_b.data_ptr(), sr,
                                out.data_ptr(), dtype_code(out_dtype), ldd, out.stride(0), use_fast_accum, _stream())
    _check(st)
    return out


def scaled_grouped_mm(a, b, batch_sizes, batch_offsets, scale_a, scale_b, out_dtype, scale_result=None,
                      use_fast_accum=False, out=None, ab_formats=None, transpose_a=False, transpose_b=True):
    """Grouped FP8 GEMM in GroupedGemmFwdOp's four layouts, batch_sizes / batch_offsets int32 [G] on the device.

    NT (default): a [batch_sum, K], b [G, N, K]; NN: b [G, K, N]. Both return d [batch_sum, N] with group g's
    rows a[rows] @ B_g * scale_a * scale_b. TN (transpose_a): a [batch_sum, N], b [batch_sum, K]; TT: b
    [K, batch_sum]; both return d [G, N, K], group g's block A_g^T @ B_g over its rows. Layouts other than NT
    pack their operands into a workspace allocated here (mm_scaled_gemm_grouped_layout).
    """
    torch = _torch()
    for t in (batch_sizes, batch_offsets):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.dim() != 1 or t.numel() != batch_sizes.numel():
            raise ValueError("batch_sizes and batch_offsets must be contiguous int32 [G]")
    G = batch_sizes.numel()
    if a.dim() != 2 or b.dim() != (2 if transpose_a else 3) or (a.shape[1] > 1 and a.stride(1) != 1) or \
            (b.shape[-1] > 1 and b.stride(-1) != 1):
        raise ValueError("a must be 2-D and b 3-D (2-D with transpose_a), both with contiguous rows")
    if transpose_a:
        batch_sum, N = a.shape
        K = b.shape[0] if transpose_b else b.shape[1]
        if (b.shape[1] if transpose_b else b.shape[0]) != batch_sum:
            raise ValueError(f"b {tuple(b.shape)} does not match batch_sum {batch_sum}")
        shape = (G, N, K)
    else:
        batch_sum, K = a.shape
        if b.shape[0] != G:
            raise ValueError("b needs one operand per group")
        N = b.shape[1] if transpose_b else b.shape[2]
        if (b.shape[2] if transpose_b else b.shape[1]) != K:
            raise ValueError(f"b {tuple(b.shape)} does not match K {K}")
        shape = (batch_sum, N)
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=a.device)
    if tuple(out.shape) != shape or (out.shape[-1] > 1 and out.stride(-1) != 1):
        raise ValueError(f"out must be {shape} with contiguous rows")
    fa = _fp8_code(a, ab_formats[0] if ab_formats else None)
    fb = _fp8_code(b, ab_formats[1] if ab_formats else None)
    st, nbytes = mm_grouped_workspace_bytes(batch_sum, N, K, G, transpose_a, transpose_b)
    _check(st)
    ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=a.device)
    lda = a.stride(0) if a.shape[0] > 1 else a.shape[1]
    ldb = b.stride(-2) if b.shape[-2] > 1 else b.shape[-1]
    ldd = out.stride(-2) if out.shape[-2] > 1 else out.shape[-1]
    st = mm_scaled_gemm_grouped_layout(batch_sum, N, K, G, transpose_a, transpose_b, a.data_ptr(), fa, lda,
                                       b.data_ptr(), fb, ldb, b.stride(0) if not transpose_a else 0,
                                       batch_sizes.data_ptr(), batch_offsets.data_ptr(), scale_a.data_ptr(),
                                       scale_b.data_ptr(), scale_result.data_ptr() if scale_result is not None else 0,
                                       out.data_ptr(), dtype_code(out_dtype), ldd,
                                       out.stride(0) if transpose_a else 0, ws.data_ptr(), nbytes, use_fast_accum,
                                       _stream())
    _check(st)
    return out


def blockscaled_gemm_amax(a, b, sfa, sfb, c_dtype=None, sf_vec_size=32, with_index=False, ab_format=None):
    """C[l] = (A[l] * SFA[l]) @ (B[l] * SFB[l])^T and the global amax of C.

    a: [L, M, K] FP8, b: [L, N, K] FP8 (same format), or FP4 pairs
    (float4_e2m1fn_x2, or uint8 with ab_format=MM_F4_E2M1) [L, M, K/2] and
    [L, N, K/2]. The scale factors are either float32 powers of two (FP8
    only), sfa [L, M, ceil(K/32)] and sfb [L, N, ceil(K/32)], or the cuDNN
    page's own tensors: E8M0 bytes (float8_e8m0fnu, uint8 or int8) of storage
    shape (L, ceil(MN/128), ceil(K/(4 sf)), 32, 4, 4), or E4M3 bytes (float8_e4m3fn) of that shape with FP4
    operands and sf_vec_size=16. Returns
    (c [L, M, N], amax [1]) or (c, amax, amax_index [1]) with with_index; an FP4 C (c_dtype
    float4_e2m1fn_x2, FP4 operands only) is [L, M, ceil(N/2)], two values per byte, low nibble first.
    """
    torch = _torch()
    c_dtype = c_dtype or torch.float32
    L, M, K = a.shape
    N = b.shape[1]
    ab_type = _fp8_code(a, ab_format)
    if ab_type == MM_F4_E2M1:
        K *= 2
    for t in (a, b, sfa, sfb):
        if not t.is_contiguous():
            raise ValueError("operands must be contiguous")
    c_type = dtype_code(c_dtype)
    # FP4 C holds two values per byte: rows of ceil(N/2) bytes, the page's (M, ceil(N/2), L) n-major tensor
    c = torch.empty((L, M, -(-N // 2) if c_type == MM_F4_E2M1 else N), dtype=c_dtype, device=a.device)
    amax = torch.empty((1,), dtype=torch.float32, device=a.device)
    idx = torch.empty((1,), dtype=torch.int64, device=a.device) if with_index else None
    if sfa.element_size() == 1 and sfb.element_size() == 1:
        for t, rows in ((sfa, M), (sfb, N)):
            if t.numel() != L * -(-rows // 128) * -(-K // (4 * sf_vec_size)) * 512:
                raise ValueError("E8M0 scale factors must have the storage shape "
                                 "(L, ceil(MN/128), ceil(K/(4 sf)), 32, 4, 4)")
        sf_type = MM_SF_E4M3FN if sfa.dtype == torch.float8_e4m3fn else MM_SF_E8M0
        st = mm_blockscaled_gemm_amax_atom(M, N, K, L, a.data_ptr(), b.data_ptr(), ab_type,
                                           sfa.data_ptr(), sfb.data_ptr(), sf_type, sf_vec_size, c.data_ptr(),
                                           c_type, amax.data_ptr(), idx.data_ptr() if with_index else 0,
                                           _stream())
    else:
        if sfa.dtype != torch.float32 or sfb.dtype != torch.float32:
            raise ValueError("scale factors must be float32, or E8M0 bytes for both operands")
        st = mm_blockscaled_gemm_amax(M, N, K, L, a.data_ptr(), b.data_ptr(), ab_type,
                                      sfa.data_ptr(), sfb.data_ptr(), sf_vec_size, c.data_ptr(), c_type,
                                      amax.data_ptr(), idx.data_ptr() if with_index else 0, _stream())
    _check(st)
    return (c, amax, idx) if with_index else (c, amax)
