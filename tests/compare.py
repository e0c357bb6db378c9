"""Comparators for GPU results against the oracle.

Tolerances (one floating-point rule per output type):
 - fp32 output: |gpu - exact| <= 2^-20 * sum_k |a_k b_k s| per element.
 - bf16 / f16 / FP8 output: within 1 ulp after rounding: the ordered-integer
   distance between the GPU's bits and the oracle's rounded bits is <= 1, or
   |gpu - exact| <= 2^-20 * sum|t| + ulp_out(exact) / 2 (the second form covers
   heavy cancellation, where the fp32 accumulator's own error already exceeds
   an output ulp of a tiny result).
 - NaN must be NaN in both and carry the canonical encoding; +0 and -0 are at
   distance 0 and +-Inf one step past the largest finite value in the ulp rule;
   fp32 infinities must match exactly.
"""
from __future__ import annotations

import numpy as np

E4M3FN, E5M2, F32, BF16, F16, E2M1 = 0, 1, 2, 3, 4, 5
CANON_NAN = {F32: 0x7FFFFFFF, BF16: 0x7FFF, F16: 0x7FFF, E4M3FN: 0x7F, E5M2: 0x7F}
WIDTH = {F32: 32, BF16: 16, F16: 16, E4M3FN: 8, E5M2: 8, E2M1: 4}
MANT = {F32: 23, BF16: 7, F16: 10, E4M3FN: 3, E5M2: 2, E2M1: 1}
EMIN = {F32: -126, BF16: -126, F16: -14, E4M3FN: -6, E5M2: -14, E2M1: 0}
# E2M1 (FP4) codes, one per array element: sign bit 3, magnitudes of the OCP format
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
# E2M1 has no NaN: a NaN output is written as the code of +6 (the library's and the oracle's reading)
E2M1_NAN_CODE = 0x7
TOL = 2.0 ** -20


def bits_to_float(bits: np.ndarray, fmt: int) -> np.ndarray:
    """Values of bit patterns (independent of the oracle: numpy/torch views)."""
    import torch
    bits = np.asarray(bits)
    if fmt == F32:
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if fmt == F16:
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if fmt == BF16:
        t = torch.from_numpy(np.ascontiguousarray(bits.astype(np.uint16)).view(np.int16))
        return t.view(torch.bfloat16).to(torch.float64).numpy()
    if fmt == E2M1:
        b = bits.astype(np.int64) & 15
        return np.where(b & 8, -1.0, 1.0) * E2M1_MAG[b & 7]
    t = torch.from_numpy(np.ascontiguousarray(bits.astype(np.uint8)))
    if fmt == E4M3FN:
        return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return t.view(torch.float8_e5m2).to(torch.float64).numpy()


def is_nan_bits(bits: np.ndarray, fmt: int) -> np.ndarray:
    return np.isnan(bits_to_float(bits, fmt))


def ordered_int(bits: np.ndarray, fmt: int) -> np.ndarray:
    """Map sign-magnitude bit patterns to integers ordered like the values (+0 == -0)."""
    w = WIDTH[fmt]
    b = np.asarray(bits).astype(np.int64) & ((1 << w) - 1)
    sign = (b >> (w - 1)) & 1
    mag = b & ((1 << (w - 1)) - 1)
    return np.where(sign == 1, -mag, mag)


def ulp_of(x: np.ndarray, fmt: int) -> np.ndarray:
    """Spacing of the output format at |x| (subnormal spacing below the normal range)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, EMIN[fmt])
    return np.ldexp(1.0, (e - MANT[fmt]).astype(np.int64))


def check(gpu_bits: np.ndarray, value: np.ndarray, sum_abs: np.ndarray, oracle_bits: np.ndarray,
          fmt: int, what: str = "") -> dict:
    """Compare element by element; raise AssertionError listing the first mismatches."""
    gpu_bits = np.asarray(gpu_bits)
    assert gpu_bits.shape == value.shape, (gpu_bits.shape, value.shape)
    g = bits_to_float(gpu_bits, fmt)
    v = np.asarray(value, dtype=np.float64)
    sa = np.asarray(sum_abs, dtype=np.float64)
    w = WIDTH[fmt]
    mask = (1 << w) - 1
    gb = gpu_bits.astype(np.int64) & mask
    ob = np.asarray(oracle_bits).astype(np.int64) & mask

    v_nan = np.isnan(v)
    g_nan = np.isnan(g)
    ok = np.zeros(v.shape, dtype=bool)
    if fmt == E2M1:
        ok |= v_nan & (gb == E2M1_NAN_CODE)
    else:
        # NaN: both NaN and the GPU's encoding canonical
        ok |= v_nan & g_nan & (gb == CANON_NAN[fmt])
    # infinities and saturated values: exact bit match of the rounded result
    fin = ~v_nan & ~g_nan
    exact_bits = fin & (gb == ob)
    ok |= exact_bits
    if fmt == F32:
        with np.errstate(invalid="ignore"):
            err = np.abs(g - v)
            ok |= fin & np.isfinite(g) & np.isfinite(v) & (err <= TOL * sa)
    else:
        # +-Inf sits one step past the largest finite value in the ordered-integer map
        dist = np.abs(ordered_int(gb, fmt) - ordered_int(ob, fmt))
        ok |= fin & (dist <= 1)
        o_val = bits_to_float(ob, fmt)
        both_finite = fin & np.isfinite(g) & np.isfinite(o_val)
        with np.errstate(invalid="ignore"):
            err = np.abs(g - v)
            ok |= both_finite & np.isfinite(v) & (err <= TOL * sa + 0.5 * ulp_of(v, fmt))
    bad = np.argwhere(~ok)
    stats = {"n": int(v.size), "bad": int(bad.shape[0])}
    if bad.shape[0]:
        lines = []
        for idx in bad[:10]:
            t = tuple(int(i) for i in idx)
            lines.append(f"  at {t}: gpu bits {int(gb[t]):#x} ({g[t]!r}), oracle bits {int(ob[t]):#x}, "
                         f"exact {v[t]!r}, sum|t| {sa[t]!r}")
        raise AssertionError(f"{what}: {bad.shape[0]} of {v.size} outputs out of tolerance\n" + "\n".join(lines))
    return stats


def assert_bitwise_equal(actual: np.ndarray, expected: np.ndarray, what: str = ""):
    """Equal integer views (so +0 != -0 and NaN payloads must match)."""
    a = np.asarray(actual)
    e = np.asarray(expected)
    assert a.shape == e.shape, (what, a.shape, e.shape)
    ai = a.view(np.dtype(f"u{a.dtype.itemsize}"))
    ei = e.view(np.dtype(f"u{e.dtype.itemsize}"))
    bad = np.argwhere(ai != ei)
    if bad.shape[0]:
        first = [f"{tuple(int(i) for i in b)}: {int(ai[tuple(b)]):#x} != {int(ei[tuple(b)]):#x}" for b in bad[:10]]
        raise AssertionError(f"{what}: {bad.shape[0]} of {a.size} differ\n  " + "\n  ".join(first))
