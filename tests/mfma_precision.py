"""How exactly the gfx950 scaled FP8 / FP4 MFMA sums its products, against the exact oracle.

Runs the test hook mm_debug_mfma_gemm (every 128 K one v_mfma_scale_f32_16x16x128_f8f6f4 into a single fp32
chain) and, for the FP8 cases, the library's own contraction (FP8 converted exactly to bf16, bf16 MFMA, one fp32
chain: mm_scaled_gemm with fast accumulation, mm_blockscaled_gemm_amax for factors per 32) on seeded 256 x 256
problems, and prints one markdown table line per case and K: the largest |gpu - exact| / sum_k|a_k b_k s_k|
(log2), its 99.9th percentile, and the share of outputs above the 2^-20 bound the library guarantees.
FP4 operands are laid out as the instruction takes them with factors per 32 values (lane (r, g) holds the
32 values k = 32 g .. 32 g + 31 of row r and that group's E8M0 factor); FP8 runs with unit factors only (its
own sums already miss the bound).

    python tests/mfma_precision.py > profiles/mfma_precision_fp8_fp4.md

Needs a GPU. Not a pytest module (it asserts nothing): the decision it informs is recorded with its output.
"""
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import block_scaled_gemm_amd as mm  # noqa: E402
import datagen  # noqa: E402
import oracle  # noqa: E402

DEV = torch.device("cuda:0")
M = N = 256
TOL = 2.0 ** -20


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def e8m0_bytes(f):
    """E8M0 codes of fp32 powers of two (their exponent fields)."""
    return ((np.ascontiguousarray(f, np.float32).view(np.uint32) >> 23) & 0xFF).astype(np.uint8)


def hook(a, b, fmt, K, fa=None, fb=None):
    d = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ta, tb = dev(a), dev(b)
    tfa = dev(e8m0_bytes(fa)) if fa is not None else None
    tfb = dev(e8m0_bytes(fb)) if fb is not None else None
    st = mm.mm_debug_mfma_gemm(M, N, K, ta.data_ptr(), tb.data_ptr(), fmt, tfa.data_ptr() if tfa is not None else 0,
                               tfb.data_ptr() if tfb is not None else 0, d.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert st == mm.MM_OK, mm.mm_last_error()
    torch.cuda.synchronize()
    return d.cpu().numpy().astype(np.float64)


def product_path(a, b, fmt, K, fa=None, fb=None):
    """The library's own contraction on the same data (f32 out)."""
    out = torch.empty((M, N), dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    ta, tb = dev(a), dev(b)
    if fa is None:
        one = torch.ones(1, dtype=torch.float32, device=DEV)
        st = mm.mm_scaled_gemm(M, N, K, ta.data_ptr(), fmt, K, tb.data_ptr(), fmt, K, one.data_ptr(), 0,
                               one.data_ptr(), 0, 0, out.data_ptr(), mm.MM_F32, N, 1, stream)
    else:
        tfa, tfb = dev(fa), dev(fb)
        st = mm.mm_blockscaled_gemm_amax(M, N, K, 1, ta.data_ptr(), tb.data_ptr(), fmt, tfa.data_ptr(),
                                         tfb.data_ptr(), 32, out.data_ptr(), mm.MM_F32, 0, 0, stream)
    assert st == mm.MM_OK, mm.mm_last_error()
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def exact(a, b, fmt, fa=None, fb=None):
    if fa is None:
        value, sabs, _ = oracle.scaled_gemm(a, fmt, b, fmt, np.float32(1), 0, np.float32(1), 0, oracle.F32)
        return value, sabs
    value, sabs, _, _, _ = oracle.blockscaled_gemm_amax(a[None], b[None], fmt, fa[None], fb[None], 32, oracle.F32)
    return value[0], sabs[0]


def stats(got, value, sabs):
    ok = sabs > 0
    rel = np.abs(got - value)[ok] / sabs[ok]
    mx = rel.max()
    p = np.quantile(rel, 0.999)
    lg = lambda x: "-inf" if x == 0 else f"{np.log2(x):.1f}"
    return lg(mx), lg(p), f"{100.0 * np.mean(rel > TOL):.2f}%"


def cases():
    g = np.random.default_rng(2024)
    for K in (128, 1024, 4096, 8192):
        a = datagen.gauss_codes(g, (M, K), 64.0)
        b = datagen.gauss_codes(g, (N, K), 64.0)
        yield "E4M3, N(0,1)*64 clamped, scales 1", mm.MM_F8_E4M3FN, K, a, b, None, None
    for K in (128, 4096):
        a = datagen.gauss_codes(g, (M, K), 64.0, datagen.E5M2)
        b = datagen.gauss_codes(g, (N, K), 64.0, datagen.E5M2)
        yield "E5M2, N(0,1)*64, scales 1", mm.MM_F8_E5M2, K, a, b, None, None
    for K in (128, 1024, 8192):
        a = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
        b = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        yield "E2M1 uniform codes, factors 1", mm.MM_F4_E2M1, K, a, b, np.ones((M, K // 32), np.float32), \
            np.ones((N, K // 32), np.float32)
    for K in (128, 1024, 8192):
        a = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
        b = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        fa, fb = datagen.pow2_scales(g, (M, K // 32)), datagen.pow2_scales(g, (N, K // 32))
        yield "E2M1 uniform codes, factors 2^U{-8..4} per 32", mm.MM_F4_E2M1, K, a, b, fa, fb
    for K in (128, 1024, 8192):
        a = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
        b = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        f = np.where(np.arange(K // 32) % 2 == 0, 2.0 ** -8, 2.0 ** 4).astype(np.float32)
        yield "E2M1, factors 2^-8 / 2^4 alternating per 32", mm.MM_F4_E2M1, K, a, b, \
            np.tile(f, (M, 1)), np.tile(f, (N, 1))


def main():
    print("# Summation precision of the gfx950 scaled FP8 / FP4 MFMA\n")
    print("Command: `python tests/mfma_precision.py` on one MI355X (" + mm.mm_version() + "), "
          f"{M} x {N} outputs per line; err = |gpu - exact| / sum|a b s|, exact = the oracle's float64 sum.\n")
    print("| data | K | path | max err (log2) | 99.9% err (log2) | outputs over 2^-20 |")
    print("|---|---|---|---|---|---|")
    for name, fmt, K, a, b, fa, fb in cases():
        value, sabs = exact(a, b, fmt, fa, fb)
        h = stats(hook(a, b, fmt, K, fa, fb), value, sabs)
        print(f"| {name} | {K} | scaled FP8/FP4 MFMA | {h[0]} | {h[1]} | {h[2]} |", flush=True)
        if fmt != mm.MM_F4_E2M1:
            p = stats(product_path(a, b, fmt, K, fa, fb), value, sabs)
            print(f"| {name} | {K} | bf16 MFMA after exact conversion | {p[0]} | {p[1]} | {p[2]} |", flush=True)


if __name__ == "__main__":
    main()
