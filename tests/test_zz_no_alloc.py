"""mm_scaled_gemm_grouped_layout_noalloc (the library's scratch array in place of the caller's workspace) against
mm_scaled_gemm_grouped_layout with a workspace, bitwise, on two calls in a row, the second with a smaller input,
for a layout that packs b (NN) and one that packs both operands (TN)."""
import numpy as np
import pytest

import datagen
from oracle import E4M3FN, BF16, F32

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")
torch = gu.torch
mm = gu.mm
DEV = gu.DEV


def run_noalloc(w, d_type, transpose_a, transpose_b, fast=False):
    """The no-allocation entry on the same inputs as gu.scaled_gemm_grouped_layout; returns d bits."""
    a, b, sizes = w["a"], w["b"], w["sizes"]
    G = len(sizes)
    if transpose_a:
        batch_sum, N = a.shape
        K = b.shape[0] if transpose_b else b.shape[1]
        shape = (G, N, K)
    else:
        batch_sum, K = a.shape
        N = b.shape[1] if transpose_b else b.shape[2]
        shape = (batch_sum, N)
    ta, tb = gu.dev_u8(a), gu.dev_u8(b)
    ts = torch.from_numpy(np.ascontiguousarray(sizes, dtype=np.int32)).to(DEV)
    to = torch.from_numpy(np.ascontiguousarray(w["offsets"], dtype=np.int32)).to(DEV)
    tsa, tsb = gu.dev_f32([w["scale_a"]]), gu.dev_f32([w["scale_b"]])
    es = np.dtype(gu.BITS_NP[d_type]).itemsize
    n_out = int(np.prod(shape))
    td = torch.full((max(n_out, 1) * es,), 0x5A, dtype=torch.uint8, device=DEV)
    st = mm.mm_scaled_gemm_grouped_layout_noalloc(batch_sum, N, K, G, transpose_a, transpose_b, ta.data_ptr(), E4M3FN,
                                                  a.shape[1], tb.data_ptr(), E4M3FN, b.shape[-1],
                                                  0 if transpose_a else b.shape[1] * b.shape[2], ts.data_ptr(),
                                                  to.data_ptr(), tsa.data_ptr(), tsb.data_ptr(), 0, td.data_ptr(),
                                                  d_type, shape[-1], N * K if transpose_a else 0, int(fast),
                                                  gu.stream())
    assert st == mm.MM_OK, (st, mm.mm_last_error())
    torch.cuda.synchronize()
    return np.ascontiguousarray(td.cpu().numpy().view(gu.BITS_NP[d_type])[:n_out].reshape(shape))


@pytest.mark.parametrize("transpose_a,transpose_b", [(0, 0), (1, 0)], ids=["NN", "TN"])
def test_noalloc_equals_workspace_entry_on_two_calls(transpose_a, transpose_b):
    big = datagen.set_grouped_layout(5, 900, 136, 520, 1, bool(transpose_a), bool(transpose_b), config=95)
    small = datagen.set_grouped_layout(3, 200, 72, 256, 0, bool(transpose_a), bool(transpose_b), config=96)
    for w, d_type, fast in ((big, BF16, False), (small, F32, True)):
        got = run_noalloc(w, d_type, transpose_a, transpose_b, fast)
        want = gu.scaled_gemm_grouped_layout(w["a"], E4M3FN, w["b"], E4M3FN, w["sizes"], w["offsets"],
                                             w["scale_a"], w["scale_b"], d_type, transpose_a, transpose_b, fast=fast)
        np.testing.assert_array_equal(got, want)


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    G, N, K = 64, 2048, 2048  # NN packs G N K bytes = 256 MiB
    st = mm.mm_scaled_gemm_grouped_layout_noalloc(1024, N, K, G, 0, 0, 0x10000, E4M3FN, K, 0x10000, E4M3FN, N, N * K,
                                                  0x10000, 0x10000, 0x10000, 0x10000, 0, 0x10000, BF16, N, 0, 0,
                                                  gu.stream())
    assert st == mm.MM_ERR_UNSUPPORTED and "scratch array" in mm.mm_last_error()
