"""GPU parity of the layouts that need operand packing, against the oracle.

"TileOPs: Linear Algebra Operators": BmmFP8FwdOp takes b as [B, K, N] as well
as [B, N, K], and GroupedGemmFwdOp has the NN, TN and TT layouts besides NT.
The library packs such operands with the contraction innermost (one extra read
and write) and runs the same GEMM kernels. What is checked here:

- the byte transpose bit for bit (integer work), pitches and ragged edges
  included, and that bytes past a row's extent are not written;
- BMM with b as [L, K, N] against the oracle, and the zero-copy case (a
  [L, K, N] view whose K axis is innermost) against the plain call;
- the grouped GEMM in NN, TN and TT against the oracle's four-layout grouped
  GEMM, element by element at sizes spanning several tiles with ragged and
  empty groups, fast and slow accumulation, every output type, and on
  sampled rows at the grouped workload's full size.
"""
import numpy as np
import pytest

import compare
import datagen
import oracle
from oracle import E4M3FN, E5M2, F32, BF16, F16

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")
torch = gu.torch
mm = gu.mm
DEV = gu.DEV


# ------------------------------------------------------------------ byte transpose

@pytest.mark.parametrize("L,R,C,ld_src,ld_dst", [(3, 100, 200, 208, 112), (1, 1, 1, 1, 1), (2, 64, 64, 64, 64),
                                                 (1, 300, 7, 9, 300), (4, 129, 65, 65, 144)])
def test_transpose_is_exact(L, R, C, ld_src, ld_dst):
    src = datagen.rng(60, R * C).integers(0, 256, size=(L, R, C), dtype=np.uint8)
    got = gu.transpose_u8(src, ld_src, ld_dst)
    np.testing.assert_array_equal(got[:, :, :R], np.transpose(src, (0, 2, 1)))
    assert (got[:, :, R:] == 0x5A).all()  # bytes past R are not written


# ------------------------------------------------------------------ BMM with b as [L, K, N]

def fp8(codes, fmt=E4M3FN):
    t = torch.from_numpy(np.ascontiguousarray(codes)).to(DEV)
    return t.view(torch.float8_e4m3fn if fmt == E4M3FN else torch.float8_e5m2)


def bits(t):
    t = t.contiguous()
    view = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()]
    return t.view(view).cpu().numpy().view({1: np.uint8, 2: np.uint16, 4: np.uint32}[t.element_size()])


@pytest.mark.parametrize("L,M,N,K,d_type,fast", [(3, 130, 96, 384, BF16, False), (2, 64, 200, 1000, F32, True),
                                                 (1, 300, 136, 40, F16, False), (2, 100, 72, 256, E4M3FN, False)])
def test_bmm_with_b_as_k_by_n(L, M, N, K, d_type, fast):
    g = datagen.rng(61, M + K)
    a = datagen.gauss_codes(g, (L, M, K), 64.0)
    b_kn = datagen.gauss_codes(g, (L, K, N), 64.0, E5M2)
    torch_dt = {BF16: torch.bfloat16, F32: torch.float32, F16: torch.float16, E4M3FN: torch.float8_e4m3fn}[d_type]
    sr = 1.0 / 8 if d_type == E4M3FN else None
    t_sr = torch.tensor([sr], dtype=torch.float32, device=DEV) if sr else None
    sa = torch.tensor([0.5], dtype=torch.float32, device=DEV)
    sb = torch.tensor([0.125], dtype=torch.float32, device=DEV)
    out = mm.scaled_bmm(fp8(a), fp8(b_kn, E5M2), sa, sb, torch_dt, scale_result=t_sr, use_fast_accum=fast,
                        trans_b=False)
    got = bits(out).reshape(L, M, N)
    for l in range(L):
        value, sabs, obits = oracle.scaled_gemm(a[l], E4M3FN, np.ascontiguousarray(b_kn[l].T), E5M2, 0.5, 0, 0.125,
                                                0, d_type, scale_result=sr,
                                                accum=oracle.ACC_EXACT)
        compare.check(got[l], value, sabs, obits, d_type, f"bmm item {l}")


def test_bmm_k_innermost_view_is_not_copied_and_agrees():
    L, M, N, K = 2, 96, 80, 256
    g = datagen.rng(62, 0)
    a = datagen.gauss_codes(g, (L, M, K), 64.0)
    b_nk = datagen.gauss_codes(g, (L, N, K), 64.0)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    plain = mm.scaled_bmm(fp8(a), fp8(b_nk), one, one, torch.float32)
    # the [L, K, N] view of a [L, N, K] tensor has K innermost: trans_b=False takes it without a copy
    view = mm.scaled_bmm(fp8(a), fp8(b_nk).transpose(1, 2), one, one, torch.float32, trans_b=False)
    np.testing.assert_array_equal(bits(view), bits(plain))


# ------------------------------------------------------------------ grouped NN / TN / TT

def check_layout(w, d_type, ta, tb, fast=False, scale_result=None, fmt=(E4M3FN, E4M3FN)):
    gpu = gu.scaled_gemm_grouped_layout(w["a"], fmt[0], w["b"], fmt[1], w["sizes"], w["offsets"], w["scale_a"],
                                        w["scale_b"], d_type, ta, tb, scale_result=scale_result, fast=fast)
    value, sabs, obits = oracle.grouped_gemm_layout(w["a"], fmt[0], w["b"], fmt[1], w["sizes"], w["offsets"],
                                                    w["scale_a"], w["scale_b"], d_type, ta, tb,
                                                    scale_result=scale_result,
                                                    accum=oracle.ACC_EXACT)
    if ta:
        compare.check(gpu.reshape(-1, gpu.shape[-1]), value.reshape(-1, value.shape[-1]),
                      sabs.reshape(-1, sabs.shape[-1]), obits.reshape(-1, obits.shape[-1]), d_type, "grouped TN/TT")
    else:
        compare.check(gpu, value, sabs, obits, d_type, "grouped NN")
    return gpu


@pytest.mark.parametrize("G,batch_sum,N,K,empty,fast,d_type", [
    (5, 300, 136, 256, 1, False, BF16),     # ragged groups, one empty, partial tiles
    (3, 1000, 200, 1040, 0, True, F32),     # K tail
    (100, 1500, 64, 128, 20, False, F16),   # many groups, many empty
    (4, 600, 72, 88, 0, False, E4M3FN),     # K not a multiple of 16: the packed pitch is padded
])
def test_grouped_nn(G, batch_sum, N, K, empty, fast, d_type):
    w = datagen.set_grouped_layout(G, batch_sum, N, K, empty, False, False, config=70 + G)
    sr = 1.0 / 16 if d_type == E4M3FN else None
    check_layout(w, d_type, False, False, fast=fast, scale_result=sr)


@pytest.mark.parametrize("tb", [False, True], ids=["TN", "TT"])
@pytest.mark.parametrize("G,batch_sum,N,K,empty,fast,d_type", [
    (5, 300, 136, 200, 1, False, BF16),     # ragged contraction per group, one empty group (a zero block)
    (3, 1000, 64, 96, 0, True, F32),
    (70, 2000, 128, 128, 10, False, E4M3FN),  # more than 64 groups (two rounds of the start scan)
    (4, 5000, 256, 256, 0, False, BF16),    # groups spanning many 128-element slow chunks
    (6, 777, 40, 300, 2, True, F16),        # thin blocks
    (2, 37, 100, 70, 0, False, E5M2),       # contractions shorter than one step
    (8, 3000, 1024, 2048, 2, False, BF16),  # slow on 256x256 row-chunk tiles, ragged contractions, empty groups
])
def test_grouped_contraction_split(tb, G, batch_sum, N, K, empty, fast, d_type):
    w = datagen.set_grouped_layout(G, batch_sum, N, K, empty, True, tb, config=80 + G)
    sr = 1.0 / 16 if d_type in (E4M3FN, E5M2) else None
    gpu = check_layout(w, d_type, True, tb, fast=fast, scale_result=sr)
    for g in np.flatnonzero(w["sizes"] == 0):
        assert (gpu[g] == 0).all()  # an empty group's block is +0


def test_grouped_contraction_split_e5m2_operands():
    w = datagen.set_grouped_layout(3, 400, 96, 160, 0, True, False, config=90)
    w["a"] = datagen.gauss_codes(datagen.rng(90, 5), w["a"].shape, 64.0, E5M2)
    check_layout(w, F32, True, False, fmt=(E5M2, E4M3FN))


def test_grouped_contraction_split_full_size():
    """The grouped workload's shapes with the groups splitting the contraction: 8 groups over 8192 packed rows,
    a [8192, 4096], b [8192, 4096] (TN), blocks [8, 4096, 4096] bf16, slow; sampled rows of every block."""
    G, S, N, K = 8, 8192, 4096, 4096
    w = datagen.set_grouped_layout(G, S, N, K, 0, True, False, config=9)
    gpu = gu.scaled_gemm_grouped_layout(w["a"], E4M3FN, w["b"], E4M3FN, w["sizes"], w["offsets"], w["scale_a"],
                                        w["scale_b"], BF16, True, False)
    rows = np.unique(np.concatenate([np.arange(16), np.arange(0, N, 64) + datagen.rng(91, 0).integers(0, 64, N // 64),
                                     np.arange(N - 16, N)]))  # a row in every 64-row band of the block
    for g in range(G):
        r0, s = int(w["offsets"][g]), int(w["sizes"][g])
        at = np.ascontiguousarray(w["a"][r0:r0 + s].T)
        bt = np.ascontiguousarray(w["b"][r0:r0 + s].T)
        value, sabs, obits = oracle.scaled_gemm(at, E4M3FN, bt, E4M3FN, w["scale_a"], 0, w["scale_b"], 0, BF16,
                                                accum=oracle.ACC_EXACT, rows=rows)
        compare.check(gpu[g][rows], value, sabs, obits, BF16, f"group {g}")


@pytest.mark.parametrize("tb", [False, True], ids=["TN", "TT"])
def test_contraction_split_uses_exactly_the_listed_rows(tb):
    # metadata the page makes the caller's error (sizes not adding up, a gap between groups): every group's
    # block is still the product over exactly its listed rows, within the buffers
    S, N, K = 400, 72, 96
    w = datagen.set_grouped_layout(4, S, N, K, 0, True, tb, config=92)
    sizes = np.array([50, 0, 30, 100], np.int32)
    offsets = np.array([0, 60, 60, 250], np.int32)
    gpu = gu.scaled_gemm_grouped_layout(w["a"], E4M3FN, w["b"], E4M3FN, sizes, offsets, w["scale_a"], w["scale_b"],
                                        F32, True, tb)
    bt_all = w["b"] if tb else np.ascontiguousarray(w["b"].T)  # [K, S]
    for g, (sz, of) in enumerate(zip(sizes, offsets)):
        if sz == 0:
            assert (gpu[g] == 0).all()
            continue
        value, sabs, obits = oracle.scaled_gemm(np.ascontiguousarray(w["a"][of:of + sz].T), E4M3FN,
                                                np.ascontiguousarray(bt_all[:, of:of + sz]), E4M3FN, w["scale_a"],
                                                0, w["scale_b"], 0, F32, accum=oracle.ACC_EXACT)
        compare.check(gpu[g], value, sabs, obits, F32, f"group {g}")


def test_grouped_nn_e5m2_fast():
    w = datagen.set_grouped_layout(6, 900, 136, 320, 1, False, False, config=93)
    w["b"] = datagen.gauss_codes(datagen.rng(93, 7), w["b"].shape, 64.0, E5M2)
    check_layout(w, BF16, False, False, fast=True, fmt=(E4M3FN, E5M2))
