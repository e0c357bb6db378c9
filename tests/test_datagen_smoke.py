"""CPU checks that the smoke-gate input sets hold what "mmaemu backends" (Gates and the verdict cache) lists:
every finite code, one exponent per 16-element block, cancellation inside blocks, subnormals and +-0, +-max and
-0 everywhere. Values are decoded with torch's float8 dtypes, independently of the oracle."""
import numpy as np
import pytest
import torch

import datagen
from datagen import E4M3FN, E5M2

TORCH = {E4M3FN: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def decode(codes, fmt):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(TORCH[fmt]).to(torch.float64).numpy()


@pytest.mark.parametrize("fmt", [E4M3FN, E5M2])
def test_smoke_adversarial_set_properties(fmt):
    d = datagen.set_smoke_adversarial_64x64x256(fmt)
    for x in (d["a"], d["b"]):
        assert x.shape == (64, 256)
        v = decode(x, fmt)
        assert np.isfinite(v).all()                         # no NaN or Inf code
        assert set(np.unique(x)) == set(datagen.finite_codes(fmt))  # every finite code, nothing else
        mbits = 3 if fmt == E4M3FN else 2
        for r in range(64):
            kind = datagen.SMOKE_KINDS[r % 8]
            row = x[r]
            if kind == "every_finite":
                assert set(row[: datagen.finite_codes(fmt).size]) == set(datagen.finite_codes(fmt))
            elif kind == "one_exponent":
                e = (row.reshape(16, 16).astype(np.int64) >> mbits) & ((1 << (7 - mbits)) - 1)
                assert (e == e[:, :1]).all()
            elif kind == "cancel":
                assert (decode(row, fmt).reshape(16, 16).sum(axis=1) == 0).all()
                assert (np.abs(decode(row, fmt)).reshape(16, 16).sum(axis=1) > 0).any()
            elif kind == "subnormal_zero":
                assert (((row >> mbits) & ((1 << (7 - mbits)) - 1)) == 0).all()
            elif kind == "max":
                assert (np.abs(decode(row, fmt)) == datagen.FMT_MAX[fmt]).all()
            elif kind == "minus_zero":
                assert (row == 0x80).all()


@pytest.mark.parametrize("fmt", [E4M3FN, E5M2])
def test_smoke_random_set_covers_special_codes(fmt):
    d = datagen.set_smoke_random_16x8x64(fmt)
    assert d["a"].shape == (16, 64) and d["b"].shape == (8, 64)
    v = np.concatenate([decode(d["a"], fmt).ravel(), decode(d["b"], fmt).ravel()])
    assert np.isnan(v).any() and (v == 0).any()
