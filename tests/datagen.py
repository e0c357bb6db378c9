"""Seeded synthetic inputs for the FP8 scaled GEMM sets.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark. It holds none of the GEMM's arithmetic: it draws random numbers
(numpy PCG64, seed = 1000 * set id + stream, stream 0 = A, 1 = B,
2 = scales, 3 = adversarial codes; the set ids are fixed integers) and turns
synthetic real values into FP8 codes with torch's CPU float8 casts after
clamping to the format's range.

Sets (the shapes and value recipes of the pages' LLM-layer GEMMs; where the
pages leave a value open, the recipe below is this repository's choice):

 - 256^3 (set id 1): E4M3 from N(0,1)*64 clamped to +-448, per-tensor scales
   0.5 / 0.25, fast accumulation, fp32 output.
 - per-tensor, N = K = 4096 (set id 2), M in {16, 64, 256, 1024, 2048, 8192},
   slow accumulation, bf16 output. Gaussian set: z ~ N(0,1) per tensor,
   x = z * 240 / max|z|, scale = max|z| / 240. Adversarial set: i.i.d. codes
   (25% +-448, 25% random-sign subnormals, 10% +-0, 40% uniform finite codes)
   with structured rows, scales 1.
 - block-scaled 4096 x 14336 x 4096 (set id 3): E4M3 from N(0,1)*64, scale_a
   per 1x128 [M, K/128], scale_b per 128x128 [N/128, K/128], fp32 values 2^u
   with u ~ U(-8, 4) (log-uniform in [2^-8, 2^4]), bf16 output.
 - MX, L = 8, 2048 x 2048 x 8192 (set id 4): E4M3 from N(0,1)*64, power-of-two
   scale factors 2^e, e ~ U{-8..4}, per 32 K elements per row; fp32 C and amax.
 - K tail, 8192 x 28672 x 8200 (set id 5): (a) E4M3 from N(0,1)*32 with 1%
   outliers at +-448, scales 2^-3, scale_result 1/16, E4M3 output, slow
   accumulation; (b) E5M2 from N(0,1)*32 with 1% outliers at +-57344, scales
   2^-10, f16 output, slow accumulation.
 - batched, page-native MX factors, FP4, grouped, FP4 with E4M3 factors: see
   their functions below.
"""
from __future__ import annotations

import numpy as np
import torch

E4M3FN, E5M2 = 0, 1
FMT_MAX = {E4M3FN: 448.0, E5M2: 57344.0}
_TORCH_FP8 = {E4M3FN: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}

BENCH_MS = (16, 64, 256, 1024, 2048, 8192)


def rng(set_id: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * set_id + stream))


def to_codes(x: np.ndarray, fmt: int) -> np.ndarray:
    """FP8 codes of float values already inside the format's finite range."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(_TORCH_FP8[fmt]).view(torch.uint8).numpy()


def gauss_codes(g: np.random.Generator, shape, sigma: float, fmt: int = E4M3FN,
                outlier_frac: float = 0.0) -> np.ndarray:
    """clip(N(0,1)*sigma, +-max) as FP8 codes, with a fraction of entries set to +-max."""
    mx = FMT_MAX[fmt]
    x = g.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(sigma)
    np.clip(x, -mx, mx, out=x)
    if outlier_frac > 0:
        mask = g.random(size=shape, dtype=np.float32) < outlier_frac
        sign = np.where(g.random(size=shape, dtype=np.float32) < 0.5, -mx, mx).astype(np.float32)
        x[mask] = sign[mask]
    return to_codes(x, fmt)


def normalized_codes(g: np.random.Generator, shape, target: float = 240.0, fmt: int = E4M3FN):
    """x = z * target / max|z| as FP8 codes; returns (codes, scale = max|z| / target)."""
    z = g.standard_normal(size=shape, dtype=np.float32)
    zmax = float(np.max(np.abs(z))) if z.size else 1.0
    x = z * np.float32(target / zmax)
    return to_codes(x, fmt), np.float32(zmax / target)


def finite_codes(fmt: int) -> np.ndarray:
    """Every code of the format that encodes a finite value."""
    c = np.arange(256, dtype=np.uint8)
    if fmt == E4M3FN:
        return c[(c & 0x7F) != 0x7F]
    return c[((c >> 2) & 31) != 31]


def adversarial_codes(g: np.random.Generator, shape, fmt: int = E4M3FN) -> np.ndarray:
    """i.i.d. codes: 25% +-max, 25% random-sign subnormals, 10% +-0, 40% uniform finite."""
    n = int(np.prod(shape))
    u = g.random(n)
    sign = (g.random(n) < 0.5).astype(np.uint8) << 7
    maxcode = 0x7E if fmt == E4M3FN else 0x7B
    sub_hi = 7 if fmt == E4M3FN else 3
    sub = g.integers(1, sub_hi + 1, size=n).astype(np.uint8)
    fin = finite_codes(fmt)
    uni = fin[g.integers(0, fin.size, size=n)]
    out = np.where(u < 0.25, maxcode | sign,
          np.where(u < 0.50, sub | sign,
          np.where(u < 0.60, sign, uni))).astype(np.uint8)
    return out.reshape(shape)


def adversarial_pair(M: int, N: int, K: int, set_id: int = 2, fmt: int = E4M3FN):
    """Adversarial A [M,K], B [N,K] with structured rows.

    Row 0 of A and of B is all +max; row 1 of A alternates +max / -max against
    B row 1 all +max (the sum cancels to 0); row 2 of A and B is all the
    smallest subnormal; row 3 of A is all -0.
    """
    g = rng(set_id, 3)
    a = adversarial_codes(g, (M, K), fmt)
    b = adversarial_codes(g, (N, K), fmt)
    maxcode = 0x7E if fmt == E4M3FN else 0x7B
    if M > 0 and N > 0:
        a[0, :] = maxcode
        b[0, :] = maxcode
    if M > 1 and N > 1:
        a[1, :] = maxcode
        a[1, 1::2] = maxcode | 0x80
        b[1, :] = maxcode
    if M > 2 and N > 2:
        a[2, :] = 0x01
        b[2, :] = 0x01
    if M > 3:
        a[3, :] = 0x80
    return a, b


def log_uniform_scales(g: np.random.Generator, shape, lo: float = -8.0, hi: float = 4.0):
    """fp32 values 2^u with u ~ U(lo, hi)."""
    u = g.uniform(lo, hi, size=shape)
    return np.exp2(u).astype(np.float32)


def pow2_scales(g: np.random.Generator, shape, lo: int = -8, hi: int = 4):
    """fp32 powers of two 2^e with e ~ U{lo..hi}."""
    e = g.integers(lo, hi + 1, size=shape)
    return np.ldexp(np.ones(shape, dtype=np.float32), e).astype(np.float32)


def set_smoke_random_16x8x64(fmt: int = E4M3FN, set_id: int = 40):
    """The first case of the "mmaemu backends" smoke gate: 16 x 8 x 64 uniformly random codes (all 256 codes,
    NaN and Inf codes included), scales 1."""
    g = rng(set_id, fmt)
    a = g.integers(0, 256, size=(16, 64)).astype(np.uint8)
    b = g.integers(0, 256, size=(8, 64)).astype(np.uint8)
    return dict(a=a, b=b, K=64, a_fmt=fmt, b_fmt=fmt, scale_a=np.float32(1.0), scale_b=np.float32(1.0))


# the row kinds of the 64 x 64 x 256 adversarial smoke case, row r of A and of B taking kind r % 8
SMOKE_KINDS = ("every_finite", "one_exponent", "cancel", "subnormal_zero", "max", "minus_zero", "mixed",
               "one_exponent")


def set_smoke_adversarial_64x64x256(fmt: int = E4M3FN, set_id: int = 41):
    """The second case of the "mmaemu backends" smoke gate: 64 x 64 x 256 adversarial codes. Row r of A and of
    B is of kind SMOKE_KINDS[r % 8]:

     - every_finite: every finite code of the format once, in a seeded order (the rest of the row +0);
     - one_exponent: each 16-element block draws its codes from one exponent field (random per block; random
       sign and mantissa);
     - cancel: each 16-element block holds 8 random finite codes and their negations, in a shuffled order
       (the block's values sum to zero);
     - subnormal_zero: subnormal codes of random sign and +-0;
     - max: +-max (random sign);
     - minus_zero: -0 everywhere;
     - mixed: i.i.d. adversarial codes (adversarial_codes).
    Scales 1.
    """
    g = rng(set_id, fmt)
    K = 256
    fin = finite_codes(fmt)
    mbits = 3 if fmt == E4M3FN else 2
    top_exp = 15 if fmt == E4M3FN else 30       # largest exponent field of a finite code
    sub_hi = 7 if fmt == E4M3FN else 3
    maxcode = 0x7E if fmt == E4M3FN else 0x7B

    def row(kind):
        if kind == "every_finite":
            r = np.zeros(K, np.uint8)
            r[: fin.size] = g.permutation(fin)
            return r
        if kind == "one_exponent":
            blocks = []
            for _ in range(K // 16):
                e = int(g.integers(0, top_exp + 1))
                m = g.integers(0, 1 << mbits, size=16)
                if fmt == E4M3FN and e == 15:
                    m = np.minimum(m, 6)          # mantissa 7 with exponent 15 is the NaN code
                sign = (g.random(16) < 0.5).astype(np.int64) << 7
                blocks.append(((e << mbits) | m | sign).astype(np.uint8))
            return np.concatenate(blocks)
        if kind == "cancel":
            blocks = []
            for _ in range(K // 16):
                half = fin[g.integers(0, fin.size, size=8)]
                blocks.append(g.permutation(np.concatenate([half, half ^ 0x80])).astype(np.uint8))
            return np.concatenate(blocks)
        if kind == "subnormal_zero":
            code = g.integers(0, sub_hi + 1, size=K)
            return (code | ((g.random(K) < 0.5).astype(np.int64) << 7)).astype(np.uint8)
        if kind == "max":
            return (maxcode | ((g.random(K) < 0.5).astype(np.int64) << 7)).astype(np.uint8)
        if kind == "minus_zero":
            return np.full(K, 0x80, np.uint8)
        return adversarial_codes(g, (K,), fmt)

    a = np.stack([row(SMOKE_KINDS[r % 8]) for r in range(64)])
    b = np.stack([row(SMOKE_KINDS[r % 8]) for r in range(64)])
    return dict(a=a, b=b, K=K, a_fmt=fmt, b_fmt=fmt, scale_a=np.float32(1.0), scale_b=np.float32(1.0))


# ----------------------------------------------------------------- sets

def set_256_cubed(M=256, N=256, K=256):
    a = gauss_codes(rng(1, 0), (M, K), 64.0)
    b = gauss_codes(rng(1, 1), (N, K), 64.0)
    return dict(a=a, b=b, K=K, a_fmt=E4M3FN, b_fmt=E4M3FN,
                scale_a=np.float32(0.5), scale_b=np.float32(0.25))


def set_gauss_n4096(M: int, N: int = 4096, K: int = 4096, seed_offset: int = 0):
    """Per-tensor Gaussian set (M x 4096 x 4096 by default); seed_offset selects an independent copy."""
    ga = rng(2, 0 + 10 * seed_offset)
    gb = rng(2, 1 + 10 * seed_offset)
    a, sa = normalized_codes(ga, (M, K))
    b, sb = normalized_codes(gb, (N, K))
    return dict(a=a, b=b, K=K, a_fmt=E4M3FN, b_fmt=E4M3FN, scale_a=sa, scale_b=sb)


def set_adversarial_n4096(M: int, N: int = 4096, K: int = 4096):
    a, b = adversarial_pair(M, N, K, 2)
    return dict(a=a, b=b, K=K, a_fmt=E4M3FN, b_fmt=E4M3FN,
                scale_a=np.float32(1.0), scale_b=np.float32(1.0))


def set_block_scaled_4096x14336x4096(M=4096, N=14336, K=4096):
    a = gauss_codes(rng(3, 0), (M, K), 64.0)
    b = gauss_codes(rng(3, 1), (N, K), 64.0)
    kb = -(-K // 128)
    g = rng(3, 2)
    sa = log_uniform_scales(g, (M, kb))
    sb = log_uniform_scales(g, (-(-N // 128), kb))
    return dict(a=a, b=b, K=K, a_fmt=E4M3FN, b_fmt=E4M3FN, scale_a=sa, scale_b=sb)


def set_mx_l8_2048x2048x8192(L=8, M=2048, N=2048, K=8192, sf=32):
    a = gauss_codes(rng(4, 0), (L, M, K), 64.0)
    b = gauss_codes(rng(4, 1), (L, N, K), 64.0)
    ks = -(-K // sf)
    g = rng(4, 2)
    sfa = pow2_scales(g, (L, M, ks))
    sfb = pow2_scales(g, (L, N, ks))
    return dict(a=a, b=b, ab_fmt=E4M3FN, sfa=sfa, sfb=sfb, sf_vec=sf)


def set_e4m3_out_8192x28672x8200(M=8192, N=28672, K=8200):
    a = gauss_codes(rng(5, 0), (M, K), 32.0, E4M3FN, 0.01)
    b = gauss_codes(rng(5, 1), (N, K), 32.0, E4M3FN, 0.01)
    return dict(a=a, b=b, K=K, a_fmt=E4M3FN, b_fmt=E4M3FN,
                scale_a=np.float32(2.0 ** -3), scale_b=np.float32(2.0 ** -3),
                scale_result=np.float32(1.0 / 16))


def set_e5m2_f16_8192x28672x8200(M=8192, N=28672, K=8200):
    a = gauss_codes(rng(6, 0), (M, K), 32.0, E5M2, 0.01)
    b = gauss_codes(rng(6, 1), (N, K), 32.0, E5M2, 0.01)
    return dict(a=a, b=b, K=K, a_fmt=E5M2, b_fmt=E5M2,
                scale_a=np.float32(2.0 ** -10), scale_b=np.float32(2.0 ** -10))


def set_bmm_l8_2048x2048x4096(L=8, M=2048, N=2048, K=4096):
    """Batched per-tensor set (TileOPs BmmFP8FwdOp): Gaussian codes as the block-scaled set, one scale per operand."""
    a = gauss_codes(rng(7, 0), (L, M, K), 64.0)
    b = gauss_codes(rng(7, 1), (L, N, K), 64.0)
    return dict(a=a, b=b, K=K, a_fmt=E4M3FN, b_fmt=E4M3FN,
                scale_a=np.float32(0.5), scale_b=np.float32(0.25))


def bias_bf16_bits(N: int, config: int = 3):
    """A bf16 bias [N] (bit patterns), N(0, 16) values truncated to bf16."""
    x = rng(config, 3).normal(0.0, 16.0, size=N).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def e8m0_atom_codes(g, MN, K, L, sf=32, lo=-8, hi=4):
    """E8M0 scale-factor codes 127 + U{lo..hi} (factors 2^lo .. 2^hi) for every byte of the cuDNN
    GEMM + Amax page's scale tensor, in its storage shape (L, ceil(MN/128), ceil(K/(4 sf)), 32, 4, 4)."""
    shape = (L, -(-MN // 128), -(-K // (4 * sf)), 32, 4, 4)
    return (127 + g.integers(lo, hi + 1, size=shape)).astype(np.uint8)


def set_mx_atom_l8_2048x2048x8192(L=8, M=2048, N=2048, K=8192):
    """The MX set (L=8, 2048 x 2048 x 8192) with the page's own scale format: the same codes, E8M0 factors in
    the atom layout."""
    a = gauss_codes(rng(4, 0), (L, M, K), 64.0)
    b = gauss_codes(rng(4, 1), (L, N, K), 64.0)
    return dict(a=a, b=b, ab_fmt=E4M3FN, sfa=e8m0_atom_codes(rng(4, 5), M, K, L),
                sfb=e8m0_atom_codes(rng(4, 6), N, K, L), sf_vec=32)


def set_fp4_l8_2048x2048x8192(L=8, M=2048, N=2048, K=8192, sf=32, config=8):
    """FP4 set: uniform random bytes (each two E2M1 codes, all 16 codes equally likely) as a
    [L, M, K/2] and b [L, N, K/2]; E8M0 factors 2^U{-8..4} in the page's storage shape."""
    a = rng(config, 0).integers(0, 256, size=(L, M, K // 2), dtype=np.uint8)
    b = rng(config, 1).integers(0, 256, size=(L, N, K // 2), dtype=np.uint8)
    return dict(a=a, b=b, ab_fmt=5, sfa=e8m0_atom_codes(rng(config, 2), M, K, L, sf),
                sfb=e8m0_atom_codes(rng(config, 3), N, K, L, sf), sf_vec=sf, K=K)


def group_sizes(g, G, batch_sum, empty=0):
    """Ragged group sizes adding up to batch_sum: multinomial counts with Dirichlet(1) proportions, the first
    `empty` groups (after a seeded shuffle) forced to 0 rows."""
    p = g.dirichlet(np.ones(G))
    dead = g.permutation(G)[:empty]
    p[dead] = 0.0
    p = p / p.sum()
    return g.multinomial(batch_sum, p).astype(np.int32)


def set_grouped_8x8192x4096x4096(G=8, batch_sum=8192, N=4096, K=4096, empty=0, config=9):
    """Grouped set (TileOPs GroupedGemmFwdOp, NT): a [batch_sum, K] and b [G, N, K] Gaussian codes as
    the block-scaled set, ragged group sizes, one scale per operand."""
    sizes = group_sizes(rng(config, 3), G, batch_sum, empty)
    offsets = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int32)
    a = gauss_codes(rng(config, 0), (batch_sum, K), 64.0)
    b = gauss_codes(rng(config, 1), (G, N, K), 64.0)
    return dict(a=a, b=b, sizes=sizes, offsets=offsets, K=K, scale_a=np.float32(0.5), scale_b=np.float32(0.25))


def e4m3_atom_codes(g, MN, K, L, sf=16):
    """E4M3 scale-factor codes for every byte of the page's scale tensor (storage shape as e8m0_atom_codes):
    positive normal values (1 + m/8) 2^(e-7), e ~ U{3..11}, m ~ U{0..7}, i.e. factors in [2^-4, 30]."""
    shape = (L, -(-MN // 128), -(-K // (4 * sf)), 32, 4, 4)
    e = g.integers(3, 12, size=shape)
    m = g.integers(0, 8, size=shape)
    return ((e << 3) | m).astype(np.uint8)


def set_nvfp4_l8_2048x2048x8192(L=8, M=2048, N=2048, K=8192, config=11):
    """FP4 operands (uniform random bytes) with E4M3 factors per 16 values in the page's layout."""
    a = rng(config, 0).integers(0, 256, size=(L, M, K // 2), dtype=np.uint8)
    b = rng(config, 1).integers(0, 256, size=(L, N, K // 2), dtype=np.uint8)
    return dict(a=a, b=b, ab_fmt=5, sfa=e4m3_atom_codes(rng(config, 2), M, K, L),
                sfb=e4m3_atom_codes(rng(config, 3), N, K, L), sf_vec=16, K=K)


def set_grouped_layout(G, batch_sum, N, K, empty, transpose_a, transpose_b, config):
    """Grouped set in one of GroupedGemmFwdOp's layouts: Gaussian codes as set_grouped_8x8192x4096x4096,
    ragged group sizes, one scale per operand. a [batch_sum, K] (or [batch_sum, N] with transpose_a); b
    [G, N, K] (NT), [G, K, N] (NN), [batch_sum, K] (TN) or [K, batch_sum] (TT)."""
    sizes = group_sizes(rng(config, 3), G, batch_sum, empty)
    offsets = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int32)
    a = gauss_codes(rng(config, 0), (batch_sum, N if transpose_a else K), 64.0)
    if transpose_a:
        bshape = (K, batch_sum) if transpose_b else (batch_sum, K)
    else:
        bshape = (G, N, K) if transpose_b else (G, K, N)
    b = gauss_codes(rng(config, 1), bshape, 64.0)
    return dict(a=a, b=b, sizes=sizes, offsets=offsets, scale_a=np.float32(0.5), scale_b=np.float32(0.25))
