"""HIP graph capture through the C ABI: a sequence of calls (the split tile plan, a skinny GEMM, block scaling with a
bias on the row-chunk tiles, the batched block-scaled GEMM with amax and its index) captured into one graph
replays bit for bit like the same calls run eagerly, with eager work on the outputs between the replays. The
library promises capturable calls that record no memset nodes (outputs it must clear are cleared by its own
kernels), and the amax entry clears its amax itself."""
import numpy as np
import pytest

import datagen
from oracle import E4M3FN, F32, BF16, F16

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")
torch = gu.torch
mm = gu.mm


def _inputs():
    g = np.random.default_rng(2024)
    t = {}
    # the split plan: 256x256 row-chunk tiles on 12288 columns, 128x128 tiles on the last 2048
    t["a1"] = gu.dev_u8(datagen.gauss_codes(g, (4096, 264), 64.0))
    t["b1"] = gu.dev_u8(datagen.gauss_codes(g, (14336, 264), 64.0))
    # the skinny kernel
    t["a2"] = gu.dev_u8(datagen.gauss_codes(g, (16, 1024), 64.0))
    t["b2"] = gu.dev_u8(datagen.gauss_codes(g, (4096, 1024), 64.0))
    # block scaling (1x128 scale_a, 128x128 scale_b) with a bias on 256x256 row-chunk tiles
    t["a3"] = gu.dev_u8(datagen.gauss_codes(g, (4096, 520), 64.0))
    t["b3"] = gu.dev_u8(datagen.gauss_codes(g, (4096, 520), 64.0))
    t["sa3"] = gu.dev_f32(datagen.log_uniform_scales(g, (4096, 5)))
    t["sb3"] = gu.dev_f32(datagen.log_uniform_scales(g, (32, 5)))
    t["bias3"] = torch.from_numpy(np.float16(g.standard_normal(4096)).view(np.uint16).view(np.uint8).copy()).to(gu.DEV)
    # the batched block-scaled GEMM with amax and index: L = 2, 256 x 256 x 512, factors per 32
    t["a4"] = gu.dev_u8(datagen.gauss_codes(g, (2, 256, 512), 64.0))
    t["b4"] = gu.dev_u8(datagen.gauss_codes(g, (2, 256, 512), 64.0))
    t["sa4"] = gu.dev_f32(np.exp2(g.integers(-4, 5, size=(2, 256, 16))).astype(np.float32))
    t["sb4"] = gu.dev_f32(np.exp2(g.integers(-4, 5, size=(2, 256, 16))).astype(np.float32))
    t["s"] = gu.dev_f32([0.5, 0.25])
    return t


def _outputs():
    def buf(nbytes):
        return torch.full((nbytes,), 0x5A, dtype=torch.uint8, device=gu.DEV)
    return {"d1": buf(4096 * 14336 * 2), "d2": buf(16 * 4096 * 2), "d3": buf(4096 * 4096 * 2),
            "c4": buf(2 * 256 * 256 * 4), "amax4": torch.full((1,), 123.0, dtype=torch.float32, device=gu.DEV),
            "idx4": torch.full((1,), 777, dtype=torch.int64, device=gu.DEV)}


def _enqueue(t, o):
    s = gu.stream()
    sa, sb = t["s"].data_ptr(), t["s"].data_ptr() + 4
    calls = [
        mm.mm_scaled_gemm(4096, 14336, 264, t["a1"].data_ptr(), E4M3FN, 264, t["b1"].data_ptr(), E4M3FN, 264, sa, 0,
                          sb, 0, 0, o["d1"].data_ptr(), BF16, 14336, 0, s),
        mm.mm_scaled_gemm(16, 4096, 1024, t["a2"].data_ptr(), E4M3FN, 1024, t["b2"].data_ptr(), E4M3FN, 1024, sa, 0,
                          sb, 0, 0, o["d2"].data_ptr(), BF16, 4096, 0, s),
        mm.mm_scaled_gemm_bias(4096, 4096, 520, t["a3"].data_ptr(), E4M3FN, 520, t["b3"].data_ptr(), E4M3FN, 520,
                               t["sa3"].data_ptr(), 1, t["sb3"].data_ptr(), 2, t["bias3"].data_ptr(),
                               o["d3"].data_ptr(), F16, 4096, 0, s),
        mm.mm_blockscaled_gemm_amax(256, 256, 512, 2, t["a4"].data_ptr(), t["b4"].data_ptr(), E4M3FN,
                                    t["sa4"].data_ptr(), t["sb4"].data_ptr(), 32, o["c4"].data_ptr(), F32,
                                    o["amax4"].data_ptr(), o["idx4"].data_ptr(), s),
    ]
    for st in calls:
        assert st == mm.MM_OK, (st, mm.mm_last_error())


def test_graph_replays_match_eager():
    t = _inputs()
    eager = _outputs()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        _enqueue(t, eager)
    torch.cuda.synchronize()

    captured = _outputs()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _enqueue(t, captured)
    torch.cuda.synchronize()
    for rep in range(3):
        for k, v in captured.items():  # eager work on the outputs between replays
            v.fill_(0x3C if v.dtype == torch.uint8 else -1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(captured[k], eager[k]), f"replay {rep}: {k} differs from the eager call"
    assert float(eager["amax4"].item()) > 0 and 0 <= int(eager["idx4"].item()) < 2 * 256 * 256
