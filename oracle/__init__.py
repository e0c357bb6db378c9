"""CPU oracle for the FP8 scaled GEMM and the block-scaled GEMM + amax.

TEST INFRASTRUCTURE: only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The product path
(``block_scaled_gemm_amd``) never imports it and shares no code with it.

All arithmetic lives in ``oracle.cpp`` (plain C++, float64); this module only
marshals numpy arrays through ctypes. Its format numbers are its own:
E4M3FN = 0, E5M2 = 1, F32 = 2, BF16 = 3, F16 = 4, E2M1 = 5 (FP4, two per byte); scale modes TENSOR = 0,
1x128 = 1, 128x128 = 2; accumulation EXACT = 0, F32_CHUNKS = 1; scale-factor
element types SF_E8M0 = 0, SF_E4M3FN = 1.

Parity status of each function (what pins it is in tests/test_oracle_*.py):
decode_fp8, decode_fp4, round_to, scaled_gemm (exact and f32-chunk modes),
grouped_gemm, blockscaled_gemm_amax: pinned. sf_atom_unpack: element decoding, the
storage-to-logical permutation and the padding rule pinned; the order of the
rows and groups inside a 128 x 4 atom is a reading of the page's shapes
(parity unpinned for that order).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

E4M3FN, E5M2, F32, BF16, F16, E2M1 = 0, 1, 2, 3, 4, 5
SCALE_TENSOR, SCALE_1x128, SCALE_128x128 = 0, 1, 2
ACC_EXACT, ACC_F32_CHUNKS = 0, 1
SF_E8M0, SF_E4M3FN = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
# The mutation tests point this at a deliberately broken copy of the oracle.
_LIB_OVERRIDE = os.environ.get("ORACLE_LIB_PATH")
_lib = None

_BITS_DTYPE = {E4M3FN: np.uint8, E5M2: np.uint8, F32: np.uint32, BF16: np.uint16, F16: np.uint16, 5: np.uint8}


def build(force: bool = True) -> str:
    """Compile oracle.cpp into liboracle.so with g++ (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
               "-ffp-contract=off", "-fno-fast-math", "-o", _LIB + ".tmp", _SRC]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB
        if not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.orc_decode_fp8.argtypes = [P, I64, I, P]
        lib.orc_round.argtypes = [P, I64, I, P]
        lib.orc_scaled_gemm.argtypes = [I64, I64, I64, P, I, I64, P, I, I64, P, I, P, I, P, P, I, I,
                                        P, I64, P, P, P, I]
        lib.orc_blockscaled_gemm_amax.argtypes = [I64, I64, I64, I64, P, P, I, P, P, I, I, P, I64,
                                                  P, P, P, P, P, I]
        lib.orc_sf_atom_unpack.argtypes = [P, I, I64, I64, I64, I, P]
        lib.orc_decode_fp4.argtypes = [P, I64, P]
        lib.orc_grouped_gemm.argtypes = [I64, I64, I64, I64, P, I, I64, P, I, I64, I64, P, P, P, P, P, I, I, P, P, P,
                                         I]
        for f in (lib.orc_decode_fp8, lib.orc_round, lib.orc_scaled_gemm,
                  lib.orc_blockscaled_gemm_amax, lib.orc_sf_atom_unpack, lib.orc_decode_fp4,
                  lib.orc_grouped_gemm):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc == 2:
        raise RuntimeError("oracle refuses to run: the host FP environment flushes subnormals (FTZ/DAZ)")
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")


def _threads(threads):
    return int(threads) if threads else (os.cpu_count() or 1)


def bits_dtype(fmt: int):
    return _BITS_DTYPE[fmt]


def decode_fp8(codes: np.ndarray, fmt: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    _check(_load().orc_decode_fp8(_ptr(codes), codes.size, fmt, _ptr(out)))
    return out


def decode_fp4(codes: np.ndarray) -> np.ndarray:
    """E2M1 codes (0..15, one per array element) to float64."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    _check(_load().orc_decode_fp4(_ptr(codes), codes.size, _ptr(out)))
    return out


def round_to(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float64 values to dtype with the oracle's output rules; returns bit patterns (E2M1: one code per
    byte)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=_BITS_DTYPE[dtype])
    _check(_load().orc_round(_ptr(x), x.size, dtype, _ptr(out)))
    return out


def scaled_gemm(a, a_fmt, b, b_fmt, scale_a, sa_mode, scale_b, sb_mode, d_type,
                scale_result=None, accum=ACC_EXACT, rows=None, threads=None, bias=None):
    """d = (a*s_a) @ (b*s_b)^T (+ bias) for a [M, lda>=K] and b [N, ldb>=K] uint8 codes.

    ``bias``: optional [N] float64 values (the decoded bias), added after the
    scales; not allowed with FP8 outputs.

    ``a`` and ``b`` are 2-D uint8 arrays whose first K columns are used (pass K
    via ``a.shape[1]`` unless the arrays are wider, see ``K`` below). Returns
    (value float64 [R,N], sum_abs float64 [R,N], d_bits [R,N]) for the R rows in
    ``rows`` (all rows when None).
    """
    return scaled_gemm_k(a, a_fmt, b, b_fmt, a.shape[1], scale_a, sa_mode, scale_b, sb_mode,
                         d_type, scale_result, accum, rows, threads, bias)


def scaled_gemm_k(a, a_fmt, b, b_fmt, K, scale_a, sa_mode, scale_b, sb_mode, d_type,
                  scale_result=None, accum=ACC_EXACT, rows=None, threads=None, bias=None):
    """As scaled_gemm, with an explicit K <= row pitch of a and b."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    M, lda = a.shape
    N, ldb = b.shape
    sa = np.ascontiguousarray(scale_a, dtype=np.float32).reshape(-1)
    sb = np.ascontiguousarray(scale_b, dtype=np.float32).reshape(-1)
    sr = None if scale_result is None else np.asarray([scale_result], dtype=np.float32).reshape(-1)
    bi = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64).reshape(-1)
    if bi is not None and bi.size != N:
        raise ValueError("bias must have N values")
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = M if r is None else r.size
    value = np.empty((R, N), dtype=np.float64)
    sabs = np.empty((R, N), dtype=np.float64)
    bits = np.empty((R, N), dtype=_BITS_DTYPE[d_type])
    _check(_load().orc_scaled_gemm(M, N, K, _ptr(a), a_fmt, lda, _ptr(b), b_fmt, ldb,
                                   _ptr(sa), sa_mode, _ptr(sb), sb_mode, _ptr(sr), _ptr(bi), d_type, accum,
                                   _ptr(r), R, _ptr(value), _ptr(sabs), _ptr(bits),
                                   _threads(threads)))
    return value, sabs, bits


def grouped_gemm(a, a_fmt, b, b_fmt, sizes, offsets, scale_a, scale_b, d_type, scale_result=None,
                 accum=ACC_EXACT, threads=None):
    """Grouped GEMM (NT): a [batch_sum, K], b [G, N, K] uint8 codes, sizes / offsets int32 [G]; group g's rows
    offsets[g] .. +sizes[g] times b[g]^T, per-tensor scales. Returns (value, sum_abs, d_bits), each
    [batch_sum, N]; rows of no group hold NaN / NaN / 0."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    batch_sum, K = a.shape
    G, N, _ = b.shape
    sz = np.ascontiguousarray(sizes, dtype=np.int32)
    of = np.ascontiguousarray(offsets, dtype=np.int32)
    if sz.size != G or of.size != G:
        raise ValueError("sizes and offsets need one entry per group")
    sa = np.asarray([scale_a], dtype=np.float32).reshape(-1)
    sb = np.asarray([scale_b], dtype=np.float32).reshape(-1)
    sr = None if scale_result is None else np.asarray([scale_result], dtype=np.float32).reshape(-1)
    value = np.full((batch_sum, N), np.nan)
    sabs = np.full((batch_sum, N), np.nan)
    bits = np.zeros((batch_sum, N), dtype=_BITS_DTYPE[d_type])
    _check(_load().orc_grouped_gemm(batch_sum, N, K, G, _ptr(a), a_fmt, K, _ptr(b), b_fmt, K, N * K, _ptr(sz),
                                    _ptr(of), _ptr(sa), _ptr(sb), _ptr(sr), d_type, accum, _ptr(value), _ptr(sabs),
                                    _ptr(bits), _threads(threads)))
    return value, sabs, bits



def grouped_gemm_layout(a, a_fmt, b, b_fmt, sizes, offsets, scale_a, scale_b, d_type, transpose_a, transpose_b,
                        scale_result=None, accum=ACC_EXACT, threads=None):
    """TileOPs GroupedGemmFwdOp in all four (transpose_a, transpose_b) layouts ("Linear Algebra Operators",
    GroupedGemmFwdOp: the layout table and the forward's argument shapes), with FP8 codes and one scale per
    operand as the NT grouped_gemm.

    Without transpose_a the groups split the rows of a [batch_sum, K]: group g's rows times b[g]^T (NT, b
    [G, N, K]) or times b[g] (NN, b [G, K, N]); returns (value, sum_abs, d_bits), each [batch_sum, N].
    With transpose_a the groups split the contraction: a is [batch_sum, N], b is [batch_sum, K] (TN) or
    [K, batch_sum] (TT), and group g gives the [N, K] product A_g^T @ B_g of its rows (an empty group gives
    zeros); returns the three arrays, each [G, N, K]. Each group's product is the plain scaled GEMM over its
    own contraction (slow chunks of 128 counted from the group's first row).
    """
    a = np.asarray(a, dtype=np.uint8)
    b = np.asarray(b, dtype=np.uint8)
    sz = np.ascontiguousarray(sizes, dtype=np.int32).reshape(-1)
    of = np.ascontiguousarray(offsets, dtype=np.int32).reshape(-1)
    G = sz.size
    if of.size != G:
        raise ValueError("sizes and offsets need one entry per group")
    if (sz < 0).any() or (of != np.concatenate([[0], np.cumsum(sz)[:-1]]).astype(np.int64)[:G]).any():
        raise ValueError("sizes must be >= 0 and offsets their exclusive prefix sum")
    if not transpose_a:
        if a.shape[0] != int(sz.sum()):
            raise ValueError("sizes must add up to a's rows")
        # NN: group g's operand b[g] is [K, N]; its transpose is the NT operand
        bt = b if transpose_b else np.transpose(b, (0, 2, 1))
        return grouped_gemm(a, a_fmt, bt, b_fmt, sz, of, scale_a, scale_b, d_type, scale_result, accum, threads)
    batch_sum, N = a.shape
    # TN: b [batch_sum, K] -> the group's B_g is its rows; TT: b [K, batch_sum] -> B_g^T is its columns
    K = b.shape[0] if transpose_b else b.shape[1]
    if (b.shape[1] if transpose_b else b.shape[0]) != batch_sum or int(sz.sum()) != batch_sum:
        raise ValueError("sizes must add up to the packed contraction of a and b")
    value = np.zeros((G, N, K))
    sabs = np.zeros((G, N, K))
    bits = np.zeros((G, N, K), dtype=_BITS_DTYPE[d_type])
    for g in range(G):
        r0, s = int(of[g]), int(sz[g])
        if s == 0:
            # the product over an empty contraction: +0, whose code is 0 in every output type
            continue
        at = np.ascontiguousarray(a[r0:r0 + s, :].T)                       # A_g^T   [N, s]
        bt = np.ascontiguousarray(b[:, r0:r0 + s] if transpose_b else b[r0:r0 + s, :].T)  # B_g^T [K, s]
        value[g], sabs[g], bits[g] = scaled_gemm(at, a_fmt, bt, b_fmt, scale_a, SCALE_TENSOR, scale_b,
                                                 SCALE_TENSOR, d_type, scale_result, accum, threads=threads)
    return value, sabs, bits

def blockscaled_gemm_amax(a, b, ab_fmt, sfa, sfb, sf_vec, c_type, rows=None, threads=None):
    """C[l,m,n] = sum_k A^ B^ with A^ = A*SFA[l,m,k//sf]; a [L,M,K], b [L,N,K] uint8
    (E2M1: [L,M,K/2] and [L,N,K/2] bytes, two elements each).

    Returns (value [L,R,N], sum_abs [L,R,N], c_bits [L,R,N], amax float32, amax_index int).
    """
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    L, M, K = a.shape
    if ab_fmt == E2M1:
        K *= 2
    N = b.shape[1]
    sfa = np.ascontiguousarray(sfa, dtype=np.float32)
    sfb = np.ascontiguousarray(sfb, dtype=np.float32)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = M if r is None else r.size
    value = np.empty((L, R, N), dtype=np.float64)
    sabs = np.empty((L, R, N), dtype=np.float64)
    # E2M1 C: packed, [L, R, ceil(N/2)] bytes
    bits = np.empty((L, R, (N + 1) // 2 if c_type == E2M1 else N), dtype=_BITS_DTYPE[c_type])
    amax = np.zeros(1, dtype=np.float32)
    idx = np.zeros(1, dtype=np.int64)
    _check(_load().orc_blockscaled_gemm_amax(M, N, K, L, _ptr(a), _ptr(b), ab_fmt, _ptr(sfa),
                                             _ptr(sfb), sf_vec, c_type, _ptr(r), R, _ptr(value),
                                             _ptr(sabs), _ptr(bits), _ptr(amax), _ptr(idx),
                                             _threads(threads)))
    return value, sabs, bits, float(amax[0]), int(idx[0])


def sf_atom_shape(MN: int, K: int, L: int, sf_vec: int):
    """Storage shape (L, ceil(MN/128), ceil(K/(4 sf)), 32, 4, 4) of a page-native scale tensor."""
    return (L, -(-MN // 128), -(-K // (4 * sf_vec)), 32, 4, 4)


def sf_atom_unpack(sf, sf_type: int, MN: int, K: int, L: int, sf_vec: int) -> np.ndarray:
    """Page-native scale bytes (storage order, any shape of the right size) -> float32 [L, MN, ceil(K/sf)]."""
    sf = np.ascontiguousarray(sf, dtype=np.uint8).reshape(-1)
    if sf.size != int(np.prod(sf_atom_shape(MN, K, L, sf_vec))):
        raise ValueError("scale tensor size does not match the atom shape")
    G = -(-K // sf_vec)
    out = np.full((L, MN, G), np.nan, dtype=np.float32)
    _check(_load().orc_sf_atom_unpack(_ptr(sf), sf_type, MN, K, L, sf_vec, _ptr(out)))
    return out


def blockscaled_gemm_amax_atom(a, b, ab_fmt, sfa, sfb, sf_type, sf_vec, c_type, rows=None, threads=None):
    """blockscaled_gemm_amax with page-native scale tensors (storage bytes, see sf_atom_unpack)."""
    L, M, K = np.shape(a)
    N = np.shape(b)[1]
    if ab_fmt == E2M1:
        K *= 2
    fa = sf_atom_unpack(sfa, sf_type, M, K, L, sf_vec)
    fb = sf_atom_unpack(sfb, sf_type, N, K, L, sf_vec)
    return blockscaled_gemm_amax(a, b, ab_fmt, fa, fb, sf_vec, c_type, rows=rows, threads=threads)
