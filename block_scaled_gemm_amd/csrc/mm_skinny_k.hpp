// mm_skinny_k.hpp -- skinny-M FP8 GEMM with every K step of a workgroup in
// flight at once (internal to libmmfp8).
//
// For M <= 16 MT with per-tensor scales (the GemmFP8FwdOp of "TileOPs: Linear
// Algebra Operators" at decode-like row counts) the run is bound by streaming
// b (N x K bytes) from HBM once. A workgroup owns a 16 MT x 16 NBF output tile
// over all of K, which is at most NW * SPW steps of 128 (the launcher's
// condition). Its NW waves take the steps round-robin, SPW each, and issue
// all their loads at once: b
// straight into registers in the MFMA operand layout (lane (r, g) holds
// k = 32 g .. 32 g + 31 of row r), a in contiguous 1 KB pieces that go through
// the wave's own LDS slot (XOR-swizzled as in gemm_tile) to reach the same
// layout. Each step is multiplied as soon as its own loads have landed. Fast
// accumulation chains a wave's steps; slow gives every 128-element chunk a
// fresh fp32 partial that is then added to the wave's accumulator. The waves'
// tiles are added in wave order through LDS, and wave w stores fragments
// w, w + NW, ... of the tile.
//
// Compared with gemm_skinny (one step per wave in flight at MT = 4) this keeps
// twice the waves and steps in flight with fewer registers per wave.
#pragma once

#include "mm_kernels.hpp"

namespace mmfp8 {

template <int MT, int NBF, int MODE, int FA, int FB, int NW, int SPW>
__global__ void __launch_bounds__(NW * 64) gemm_skinny_k(GemmArgs p) {
    static_assert(MODE == MODE_FAST || MODE == MODE_SLOW, "per-tensor scales");
    static_assert(SPW >= 1 && SPW <= 4, "steps in flight per wave");
    constexpr int AROWS = 16 * MT, NB = 16 * NBF;
    constexpr int A_INS = AROWS / 8;   // 1 KB loads of a per step
    constexpr int SLOT = AROWS * kBK;  // one step of a
    constexpr int NFRAG = MT * NBF;
    constexpr int RED = NW * NFRAG * 1024;
    constexpr int LDSB = NW * SLOT > RED ? NW * SLOT : RED;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDSB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * NB;
    const int K = p.K, KT = (K + kBK - 1) / kBK;
    const int fr = lane & 15, fg = lane >> 4;
    const rsrc_t ra = make_rsrc(p.a, operand_extent(p.M, p.lda, K));
    const rsrc_t rb = make_rsrc(p.b + (int64_t)n0 * p.ldb, operand_extent(min(NB, p.N - n0), p.ldb, K));
    // epilogue scales, read now so that their latency hides behind the main loop
    const float alpha = p.sa[0] * p.sb[0];
    const bool fp8_out = p.d_type == T_E4M3 || p.d_type == T_E5M2;
    const float sr = (fp8_out && p.scale_result) ? p.scale_result[0] : 1.0f;

    // a: instruction q reads rows 8q .. 8q+7 of the step; lane l takes row
    // 8q + l/8, chunk c = l%8, and stores it at chunk c ^ swz(row),
    // swz(r) = (r & 7) ^ ((r >> 3) & 1): the fragment reads are then free of
    // LDS bank conflicts.
    const int ld_row = lane >> 3, ld_chunk = lane & 7;
    uint32_t aoff[A_INS];
    int awr[A_INS];
#pragma unroll
    for (int q = 0; q < A_INS; ++q) {
        const int row = q * 8 + ld_row;
        aoff[q] = (uint32_t)(row * p.lda + ld_chunk * 16);
        awr[q] = row * kBK + ((ld_chunk ^ ld_row ^ (q & 1)) << 4);
    }
    uint32_t boff[NBF];
#pragma unroll
    for (int j = 0; j < NBF; ++j) boff[j] = (uint32_t)((j * 16 + fr) * p.ldb + 32 * fg);
    const int fsw = (fr & 7) ^ (fr >> 3);
    const int foff0 = fr * kBK + (((2 * fg) ^ fsw) << 4);
    const int foff1 = fr * kBK + (((2 * fg + 1) ^ fsw) << 4);
    uint8_t* const slot = lds + wave * SLOT;

    struct Step {
        i32x4 a[A_INS];
        i32x8 b[NBF];
    };
    // Loads of step kt; chunks starting at or past K read zero (the range check
    // returns 0 for an out-of-range offset); a chunk straddling K is masked below.
    auto load = [&](int kt, Step& st) {
        const uint32_t kb = (uint32_t)(kt * kBK);
        const bool tail = kt * kBK + kBK > K;
#pragma unroll
        for (int q = 0; q < A_INS; ++q) {
            uint32_t off = aoff[q] + kb;
            if (tail && (int)kb + ld_chunk * 16 >= K) off = kOOB;
            st.a[q] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
        }
        const int k0 = kt * kBK + 32 * fg;
#pragma unroll
        for (int j = 0; j < NBF; ++j) {
            uint32_t o0 = boff[j] + kb, o1 = boff[j] + kb + 16;
            if (tail && k0 >= K) o0 = kOOB;
            if (tail && k0 + 16 >= K) o1 = kOOB;
            const i32x4 b0 = __builtin_amdgcn_raw_buffer_load_b128(rb, o0, 0, 0);
            const i32x4 b1 = __builtin_amdgcn_raw_buffer_load_b128(rb, o1, 0, 0);
            st.b[j] = cat(b0, b1);
        }
    };
    auto keep = [&](int ks, int d) -> uint32_t {  // byte mask of dword d of a chunk at ks
        const int nb = K - ks - 4 * d;
        return nb >= 4 ? 0xFFFFFFFFu : (nb <= 0 ? 0u : ((1u << (8 * nb)) - 1u));
    };
    auto mask = [&](int kt, Step& st) {
        const int ks = kt * kBK + ld_chunk * 16;
        if (ks < K && K < ks + 16) {
#pragma unroll
            for (int q = 0; q < A_INS; ++q)
#pragma unroll
                for (int d = 0; d < 4; ++d) st.a[q][d] = (int)((uint32_t)st.a[q][d] & keep(ks, d));
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kh = kt * kBK + 32 * fg + 16 * h;
            if (kh < K && K < kh + 16) {
#pragma unroll
                for (int j = 0; j < NBF; ++j)
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        st.b[j][4 * h + d] = (int)((uint32_t)st.b[j][4 * h + d] & keep(kh, d));
            }
        }
    };

    f32x4 acc[MT][NBF];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NBF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    {
        Step buf[SPW];
#pragma unroll
        for (int u = 0; u < SPW; ++u) {
            const int kt = wave + NW * u;
            if (kt < KT) load(kt, buf[u]);
        }
#pragma unroll
        for (int u = 0; u < SPW; ++u) {
            const int kt = wave + NW * u;
            if (kt >= KT) break;
            Step& cur = buf[u];
            if (kt * kBK + kBK > K && (K & 15)) mask(kt, cur);
            // a through the wave's slot (the previous step's fragment reads of it
            // have completed: their results fed that step's MFMAs)
#pragma unroll
            for (int q = 0; q < A_INS; ++q) *(i32x4*)(slot + awr[q]) = cur.a[q];
            bf16x8 bb[NBF][4];
#pragma unroll
            for (int j = 0; j < NBF; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) bb[j][q] = to_bf16x8<FB>(cur.b[j], q, 1.0f);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const i32x8 af = cat(*(const i32x4*)(slot + i * 16 * kBK + foff0),
                                     *(const i32x4*)(slot + i * 16 * kBK + foff1));
                bf16x8 ab[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) ab[q] = to_bf16x8<FA>(af, q, 1.0f);
#pragma unroll
                for (int j = 0; j < NBF; ++j) {
                    f32x4 part = MODE == MODE_FAST ? acc[i][j] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int q = 0; q < 4; ++q) part = mfma_bf16(bb[j][q], ab[q], part);
                    if (MODE == MODE_FAST) acc[i][j] = part;
                    else acc[i][j] += part;
                }
            }
        }
    }

    // the waves' tiles, added in wave order: wave w then holds fragments
    // f = w, w + NW, ... of the workgroup's tile
    __syncthreads();
    f32x4* red = (f32x4*)lds;  // [NW][NFRAG][64]
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NBF; ++j) red[(wave * NFRAG + i * NBF + j) * 64 + lane] = acc[i][j];
    __syncthreads();
    constexpr int FPW = (NFRAG + NW - 1) / NW;  // fragments per wave (some waves may have one fewer)
    f32x4 v[FPW];
#pragma unroll
    for (int c = 0; c < FPW; ++c) {
        const int f = wave + NW * c;
        if (f < NFRAG) {
            f32x4 s = red[f * 64 + lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) s += red[(w * NFRAG + f) * 64 + lane];
            v[c] = s;
        }
    }

    auto epilogue = [&](auto ot, auto bi) {
        constexpr int OT = decltype(ot)::value;
        constexpr bool BI = decltype(bi)::value != 0;
#pragma unroll
        for (int c = 0; c < FPW; ++c) {
            const int f = wave + NW * c;
            if (f >= NFRAG) continue;
            const int i = f / NBF, j = f % NBF;
            const int m = i * 16 + fr;
            const int n = n0 + j * 16 + 4 * fg;
            const int valid = (m < p.M) ? max(0, min(4, p.N - n)) : 0;
            uint32_t out[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // +0.0f turns a -0 sum into +0: a sum of products starts from +0
                float x = (v[c][r] + 0.0f) * alpha;
                if constexpr (BI) x += n + r < p.N ? load_bias<OT>(p.bias, n + r) : 0.0f;
                if constexpr (OT == T_E4M3 || OT == T_E5M2) x *= sr;
                out[r] = convert_t<OT>(x);
            }
            if (valid > 0) store4<OT>(p.d, (int64_t)m * p.ldd + n, out, valid, p.vec_store != 0);
        }
    };
    with_out_type(p.d_type, [&](auto ot) {
        constexpr int OT = decltype(ot)::value;
        if constexpr (OT == T_F32 || OT == T_BF16 || OT == T_F16) {
            if (p.bias) epilogue(ot, IC<1>{});
            else epilogue(ot, IC<0>{});
        } else {
            epilogue(ot, IC<0>{});
        }
    });
}

}  // namespace mmfp8
