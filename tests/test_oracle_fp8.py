"""Pins of the oracle's FP8 decode and output rounding (CPU).

Each check compares the oracle with something other than itself: the OCP
anchor values in tests/golden/, torch's and numpy's own casts, or invariants of
the formats.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3FN, E5M2, F32, BF16, F16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FMT = {"e4m3fn": E4M3FN, "e5m2": E5M2, "f32": F32, "bf16": BF16, "f16": F16}
ALL = np.arange(256, dtype=np.uint8)


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ------------------------------------------------------------------ decode

def test_decode_anchor_values():
    for fmt, code, val in _read_golden("fp8_anchors.txt"):
        got = oracle.decode_fp8(np.array([int(code, 16)], dtype=np.uint8), FMT[fmt])[0]
        if val == "nan":
            assert math.isnan(got), (fmt, code)
        else:
            want = float(val)
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (fmt, code, got, want)


@pytest.mark.parametrize("fmt,tdt", [(E4M3FN, torch.float8_e4m3fn), (E5M2, torch.float8_e5m2)])
def test_decode_matches_torch_cast(fmt, tdt):
    got = oracle.decode_fp8(ALL, fmt)
    want = torch.from_numpy(ALL.copy()).view(tdt).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint64), want[~nan].view(np.uint64))


@pytest.mark.parametrize("fmt,n_nan,n_inf,vmax,vmin_sub,last_pos", [
    (E4M3FN, 2, 0, 448.0, 2.0 ** -9, 0x7E),
    (E5M2, 6, 2, 57344.0, 2.0 ** -16, 0x7B),
])
def test_decode_invariants(fmt, n_nan, n_inf, vmax, vmin_sub, last_pos):
    v = oracle.decode_fp8(ALL, fmt)
    assert int(np.isnan(v).sum()) == n_nan
    assert int(np.isinf(v).sum()) == n_inf
    fin = v[np.isfinite(v)]
    assert fin.max() == vmax and fin.min() == -vmax
    assert np.min(fin[fin > 0]) == vmin_sub
    # sign symmetry: dec(c ^ 0x80) == -dec(c), including the zero sign
    for c in range(256):
        x, y = v[c], v[c ^ 0x80]
        if math.isnan(x):
            assert math.isnan(y)
        else:
            assert y == -x and math.copysign(1, y) == -math.copysign(1, x)
    # strictly increasing over the positive finite codes
    pos = v[: last_pos + 1]
    assert np.all(np.diff(pos) > 0)
    # every finite value is an integer multiple of the smallest subnormal
    assert np.all(np.mod(fin / vmin_sub, 1.0) == 0)


# ------------------------------------------------------------------ rounding

def _special_doubles(rng, n):
    """Random doubles of every magnitude, plus values exactly halfway between floats."""
    x = rng.standard_normal(n) * np.exp2(rng.integers(-160, 140, n).astype(np.float64))
    f = x.astype(np.float32)
    # midpoints between adjacent fp32 values (ties) and just off them
    nxt = np.nextafter(f, np.float32(np.inf))
    mid = (f.astype(np.float64) + nxt.astype(np.float64)) / 2
    return np.concatenate([x, mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf),
                           [0.0, -0.0, np.inf, -np.inf, 3.4028235677973366e38, 3.4028235e38 * 1.0000001,
                            1e-46, 7e-46, 1.4e-45, -1.4e-45]])


def test_round_f32_matches_ieee_cast():
    x = _special_doubles(np.random.default_rng(11), 20000)
    got = oracle.round_to(x, F32)
    with np.errstate(over="ignore"):
        want = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, want)


def test_round_f16_matches_numpy_cast():
    rng = np.random.default_rng(12)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-30, 20, 20000).astype(np.float64))
    h = x.astype(np.float16)
    nxt = np.nextafter(h, np.float16(np.inf))
    mid = (h.astype(np.float64) + nxt.astype(np.float64)) / 2
    x = np.concatenate([x, mid, [65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -25, 2.0 ** -25 * 1.5, 0.0, -0.0]])
    got = oracle.round_to(x, F16)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    finite = np.isfinite(x)
    assert np.array_equal(got[finite], want[finite])


def test_round_bf16_matches_torch_cast():
    # fp32-representable inputs (torch rounds fp32 -> bf16 with RNE), ties included
    rng = np.random.default_rng(13)
    bits = rng.integers(0, 2 ** 32, 50000, dtype=np.uint64).astype(np.uint32)
    bits[:2000] = (bits[:2000] & 0xFFFF0000) | 0x8000          # exact ties
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    got = oracle.round_to(f.astype(np.float64), BF16)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], want[~nan])


@pytest.mark.parametrize("fmt,tdt,vmax", [(E4M3FN, torch.float8_e4m3fn, 448.0), (E5M2, torch.float8_e5m2, 57344.0)])
def test_round_fp8_matches_torch_cast_in_range(fmt, tdt, vmax):
    rng = np.random.default_rng(14)
    x = (rng.standard_normal(50000) * np.exp2(rng.integers(-20, 16, 50000))).astype(np.float32)
    x = x[np.abs(x) <= vmax]
    # every midpoint between adjacent finite codes (ties) and the codes themselves
    vals = torch.from_numpy(ALL.copy()).view(tdt).to(torch.float64).numpy()
    fin = np.sort(np.unique(vals[np.isfinite(vals)]))
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, fin.astype(np.float32), mids])
    got = oracle.round_to(x.astype(np.float64), fmt)
    want = torch.from_numpy(x.copy()).to(tdt).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt,maxc", [(E4M3FN, 0x7E), (E5M2, 0x7B)])
def test_round_fp8_saturates(fmt, maxc):
    big = np.array([1e3, 1e9, np.inf, 464.0, 480.0, 61440.0, 1e30])
    got = oracle.round_to(big, fmt)
    vmax = 448.0 if fmt == E4M3FN else 57344.0
    for x, c in zip(big, got):
        assert c == (maxc if x > vmax else c), (x, c)
    assert np.all(got[big > vmax] == maxc)
    assert np.all(oracle.round_to(-big, fmt)[big > vmax] == (maxc | 0x80))


def test_round_canonical_nan_and_zero_sign():
    for dt, bits in _read_golden("canonical_nan.txt"):
        got = oracle.round_to(np.array([np.nan, -np.nan]), FMT[dt])
        assert int(got[0]) == int(bits, 16) and int(got[1]) == int(bits, 16), dt
    for dt in (E4M3FN, E5M2, F32, BF16, F16):
        z = oracle.round_to(np.array([0.0, -0.0]), dt)
        w = {E4M3FN: 8, E5M2: 8, F32: 32, BF16: 16, F16: 16}[dt]
        assert int(z[0]) == 0 and int(z[1]) == 1 << (w - 1), dt


def test_round_ieee_overflow_to_inf():
    # bf16 / f16 / f32 overflow follow IEEE RNE: to +-Inf
    assert int(oracle.round_to(np.array([1e39]), F32)[0]) == 0x7F800000
    assert int(oracle.round_to(np.array([-1e39]), BF16)[0]) == 0xFF80
    assert int(oracle.round_to(np.array([65520.0]), F16)[0]) == 0x7C00
    assert int(oracle.round_to(np.array([65519.0]), F16)[0]) == 0x7BFF
