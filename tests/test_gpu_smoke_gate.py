"""GPU parity on the two cases of the smoke gate of "mmaemu backends" (Gates and the verdict cache).

 - 16 x 8 x 64 uniformly random codes (NaN and Inf codes included);
 - 64 x 64 x 256 adversarial codes: every finite code, one exponent per 16-element
   block, cancellation inside blocks, subnormals and +-0, +-max, -0 everywhere
   (tests/datagen.py set_smoke_adversarial_64x64x256).

Each runs through mm_scaled_gemm in both formats, fast and slow accumulation and
every output type, compared element by element with the exact oracle (fp32 out:
2^-20 * sum|t|; narrower outputs: 1 ulp after rounding), NaN canonical. Outputs
that are exact by construction are checked bit for bit: a -0 row against
anything finite gives +0.
"""
import numpy as np
import pytest

import compare
import datagen
import oracle
from oracle import E4M3FN, E5M2, F32, BF16, F16

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")
DTYPES = (F32, BF16, F16, E4M3FN, E5M2)
DT_NAME = {F32: "f32", BF16: "bf16", F16: "f16", E4M3FN: "e4m3", E5M2: "e5m2"}
FMT_NAME = {E4M3FN: "e4m3", E5M2: "e5m2"}


def run_case(d, d_type, fast):
    sr = np.float32(1.0 / 1024) if d_type in (E4M3FN, E5M2) else None
    gpu = gu.scaled_gemm(d["a"], d["a_fmt"], d["b"], d["b_fmt"], d["K"], d["scale_a"], 0, d["scale_b"], 0, d_type,
                         scale_result=sr, fast=fast)
    value, sabs, bits = oracle.scaled_gemm_k(d["a"], d["a_fmt"], d["b"], d["b_fmt"], d["K"], d["scale_a"], 0,
                                             d["scale_b"], 0, d_type, scale_result=sr, accum=oracle.ACC_EXACT)
    compare.check(gpu, value, sabs, bits, d_type, f"smoke {FMT_NAME[d['a_fmt']]} -> {DT_NAME[d_type]} fast={fast}")
    return gpu, value


@pytest.mark.parametrize("fast", [False, True], ids=["slow", "fast"])
@pytest.mark.parametrize("d_type", DTYPES, ids=[DT_NAME[t] for t in DTYPES])
@pytest.mark.parametrize("fmt", [E4M3FN, E5M2], ids=["e4m3", "e5m2"])
def test_smoke_random_codes_16x8x64(fmt, d_type, fast):
    d = datagen.set_smoke_random_16x8x64(fmt)
    gpu, value = run_case(d, d_type, fast)
    assert np.isnan(value).any()  # the random codes include NaN codes: those rows and columns are NaN


@pytest.mark.parametrize("fast", [False, True], ids=["slow", "fast"])
@pytest.mark.parametrize("d_type", DTYPES, ids=[DT_NAME[t] for t in DTYPES])
@pytest.mark.parametrize("fmt", [E4M3FN, E5M2], ids=["e4m3", "e5m2"])
def test_smoke_adversarial_codes_64x64x256(fmt, d_type, fast):
    d = datagen.set_smoke_adversarial_64x64x256(fmt)
    gpu, value = run_case(d, d_type, fast)
    kinds = np.array([datagen.SMOKE_KINDS[r % 8] for r in range(64)])
    mz = kinds == "minus_zero"
    # -0 rows of A (and of B) against finite codes: every product is a zero, the sum +0
    assert (gpu[mz, :] == 0).all() and (gpu[:, mz] == 0).all()
