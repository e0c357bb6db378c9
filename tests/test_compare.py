"""Self-tests of the GPU-vs-oracle comparator (CPU)."""
import numpy as np
import pytest

import compare
from compare import F32, BF16, F16, E4M3FN


def _f32bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def test_fp32_tolerance_bound():
    v = np.array([1.0, 1.0, -3.0, 0.0])
    sa = np.array([2.0 ** 10, 2.0 ** 10, 1.0, 0.0])
    ok = _f32bits([1.0 + 2.0 ** -11, 1.0 - 2.0 ** -10, -3.0, 0.0])
    compare.check(ok, v, sa, ok, F32)
    bad = _f32bits([1.0 + 2.0 ** -9, 1.0, -3.0, 0.0])
    with pytest.raises(AssertionError):
        compare.check(bad, v, sa, ok, F32)


def test_nan_must_be_canonical_and_matched():
    v = np.array([np.nan, 1.0])
    sa = np.array([1.0, 1.0])
    ob = np.array([0x7FFFFFFF, 0x3F800000], np.uint32)
    compare.check(ob, v, sa, ob, F32)
    with pytest.raises(AssertionError):   # non-canonical payload
        compare.check(np.array([0x7FC00000, 0x3F800000], np.uint32), v, sa, ob, F32)
    with pytest.raises(AssertionError):   # NaN where a number is due
        compare.check(np.array([0x7FFFFFFF, 0x7FFFFFFF], np.uint32), v, sa, ob, F32)


def test_one_ulp_rule_bf16():
    v = np.array([1.0, 1.0, 1.0])
    sa = np.array([1e-30, 1e-30, 1e-30])
    ob = np.array([0x3F80, 0x3F80, 0x3F80], np.uint16)
    compare.check(np.array([0x3F80, 0x3F81, 0x3F7F], np.uint16), v, sa, ob, BF16)
    with pytest.raises(AssertionError):
        compare.check(np.array([0x3F80, 0x3F82, 0x3F80], np.uint16), v, sa, ob, BF16)


def test_ulp_rule_across_zero_and_inf():
    # +0 and -0 are at distance 0; +-smallest subnormal is one step from zero
    v = np.array([0.0, 0.0, np.inf])
    sa = np.array([0.0, 0.0, 1.0])
    ob = np.array([0x0000, 0x0000, 0x7C00], np.uint16)
    compare.check(np.array([0x8000, 0x0001, 0x7C00], np.uint16), v, sa, ob, F16)
    # the largest finite value is one step from +Inf; two steps is out
    compare.check(np.array([0x0000, 0x0000, 0x7BFF], np.uint16), v, sa, ob, F16)
    with pytest.raises(AssertionError):
        compare.check(np.array([0x0000, 0x0000, 0x7BFE], np.uint16), v, sa, ob, F16)
    with pytest.raises(AssertionError):   # fp32 infinities must match exactly
        compare.check(np.array([0x7F7FFFFF], np.uint32), np.array([np.inf]), np.array([1.0]),
                      np.array([0x7F800000], np.uint32), F32)


def test_cancellation_branch_fp8():
    # exact value tiny after cancellation; a GPU value within 2^-20 sum|t| + ulp/2 passes
    v = np.array([2.0 ** -12])
    sa = np.array([2.0 ** 12])
    ob = np.array([0x00], np.uint8)  # oracle rounds 2^-12 to +0 in E4M3
    gpu = np.array([0x02], np.uint8)  # 2 * 2^-9, off by two steps but within 2^-8 + ulp/2
    compare.check(gpu, v, sa, ob, E4M3FN)


def test_bitwise_helper():
    compare.assert_bitwise_equal(np.array([0.0], np.float32), np.array([0.0], np.float32))
    with pytest.raises(AssertionError):
        compare.assert_bitwise_equal(np.array([-0.0], np.float32), np.array([0.0], np.float32))
