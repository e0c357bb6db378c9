// Operand packing for the layouts whose contraction axis is not innermost in
// memory ("TileOPs: Linear Algebra Operators": BmmFP8FwdOp with b as [B, K, N],
// and GroupedGemmFwdOp's NN, TN and TT layouts). The GEMM kernels read both
// operands with the contraction innermost, so such an operand is first copied
// into a buffer in that order, one extra read and write of it, as the page
// describes for BmmFP8FwdOp.
//
// Both kernels move 64 x 64 byte tiles through LDS. transpose_kernel is the
// plain transpose. group_pack_kernel serves groups that split the
// contraction: it gives every group its own 16-byte aligned run of columns in
// the packed buffer, so that each group's slice is a GEMM operand of its own,
// transposing the source or not.
//
// The copies are bound by HBM traffic, not arithmetic: whole aligned tiles
// move in 16-byte pieces, the rest byte by byte.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mm_launch.hpp"

namespace mmfp8 {

namespace {

constexpr int kPT = 64;  // tile edge in bytes

// Start columns of the groups in the packed buffer: group g begins at the sum
// of its predecessors' sizes, each rounded up to 16 (negative sizes count as
// 0). One wave.
__global__ __launch_bounds__(64) void group_starts_kernel(const int* sizes, int G, int64_t* start) {
    const int lane = threadIdx.x;
    int64_t before = 0;
    for (int g0 = 0; g0 < G; g0 += 64) {
        const int g = g0 + lane;
        const int64_t own = g < G ? ((max(sizes[g], 0) + (int64_t)15) & ~(int64_t)15) : 0;
        int64_t incl = own;
        for (int d = 1; d < 64; d <<= 1) {
            const int64_t v = __shfl_up(incl, d);
            if (lane >= d) incl += v;
        }
        if (g < G) start[g] = before + incl - own;
        before += __shfl(incl, 63);
    }
}

// [row][byte] tiles of 64 x 64 bytes in LDS, rows of 68 bytes: a column read
// (lanes 16 rows apart) spreads over the banks.
constexpr int kPitchW = kPT / 4 + 1;
constexpr int kPitch = 4 * kPitchW;

// dst row c0 + c, bytes 16 q .. 16 q + 15 of the tile: column c of tile rows
// 16 q .. 16 q + 15, gathered into one 16-byte piece.
__device__ __forceinline__ uint4 tile_column16(const uint8_t* tile, int c, int q) {
    uint32_t v[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint8_t* col = tile + (16 * q + 4 * d) * kPitch + c;
        v[d] = (uint32_t)col[0] | ((uint32_t)col[kPitch] << 8) | ((uint32_t)col[2 * kPitch] << 16) |
               ((uint32_t)col[3 * kPitch] << 24);
    }
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Plain transpose, dst[l][c][r] = src[l][r][c]. Whole tiles of 16-byte
// aligned rows move in 16-byte pieces (one per lane each way); edge tiles and
// unaligned operands byte by byte, lanes along the contiguous axis.
__global__ __launch_bounds__(256) void transpose_kernel(const uint8_t* __restrict__ src, int64_t R, int64_t C,
                                                        int64_t ld_src, int64_t src_batch, uint8_t* __restrict__ dst,
                                                        int64_t ld_dst, int64_t dst_batch) {
    __shared__ uint32_t tile_w[kPT * kPitchW];  // [r][c]
    uint8_t* tile = reinterpret_cast<uint8_t*>(tile_w);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t r0 = (int64_t)blockIdx.x * kPT, c0 = (int64_t)blockIdx.y * kPT;
    src += (int64_t)blockIdx.z * src_batch;
    dst += (int64_t)blockIdx.z * dst_batch;
    const bool full = r0 + kPT <= R && c0 + kPT <= C;  // uniform per workgroup
    const bool vload = full && ((ld_src | src_batch) & 15) == 0 && ((uintptr_t)src & 15) == 0;
    const bool vstore = full && ((ld_dst | dst_batch) & 15) == 0 && ((uintptr_t)dst & 15) == 0;
    if (vload) {  // row i, bytes 16 j .. 16 j + 15
        const int i = t >> 2, j = t & 3;
        const uint4 v = *reinterpret_cast<const uint4*>(src + (r0 + i) * ld_src + c0 + 16 * j);
        uint32_t* row = tile_w + i * kPitchW + 4 * j;
        row[0] = v.x;
        row[1] = v.y;
        row[2] = v.z;
        row[3] = v.w;
    } else {
        for (int i = w; i < kPT; i += 4) {
            const int64_t r = r0 + i, c = c0 + lane;
            tile[i * kPitch + lane] = (r < R && c < C) ? src[r * ld_src + c] : (uint8_t)0;
        }
    }
    __syncthreads();
    if (vstore) {
        const int c = t >> 2, q = t & 3;
        *reinterpret_cast<uint4*>(dst + (c0 + c) * ld_dst + r0 + 16 * q) = tile_column16(tile, c, q);
    } else {
        for (int i = w; i < kPT; i += 4) {
            const int64_t c = c0 + i, r = r0 + lane;
            if (r < R && c < C) dst[c * ld_dst + r] = tile[lane * kPitch + i];
        }
    }
}

// Packing for groups that split the contraction, driven by the destination:
// dst is [C][dst_cols] and column x belongs to the group g whose start
// start[g] is the last <= x; it holds packed row offsets[g] + x - start[g]
// when that lies within the group's sizes[g] rows (and within R), else 0.
// TRANS: the source is [R][ld_src] (row r's C bytes contiguous); otherwise
// [C][ld_src] (row c holds the packed rows). Every byte of dst's C rows up to
// dst_cols is written, in 16-byte pieces when the tile is whole.
template <bool TRANS>
__global__ __launch_bounds__(256) void group_pack_kernel(const uint8_t* __restrict__ src, int64_t R, int64_t C,
                                                         int64_t ld_src, uint8_t* __restrict__ dst,
                                                         int64_t dst_cols, const int* sizes, const int* offsets,
                                                         const int64_t* start, int G) {
    __shared__ uint32_t tile_w[kPT * kPitchW];  // [destination column][c]
    __shared__ int64_t rowmap[kPT];
    uint8_t* tile = reinterpret_cast<uint8_t*>(tile_w);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t x0 = (int64_t)blockIdx.x * kPT, c0 = (int64_t)blockIdx.y * kPT;
    if (w == 0) {
        const int64_t x = x0 + lane;
        int lo = 0, hi = G;  // first g with start[g] > x lies in [lo, hi]
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (start[mid] <= x) lo = mid + 1;
            else hi = mid;
        }
        const int g = lo - 1;
        int64_t r = -1;
        if (g >= 0 && x < dst_cols) {
            const int64_t k = x - start[g];
            const int64_t row = (int64_t)offsets[g] + k;
            if (k < (int64_t)sizes[g] && row >= 0 && row < R) r = row;
        }
        rowmap[lane] = r;
    }
    __syncthreads();
    if constexpr (TRANS) {  // tile row i = source row rowmap[i], bytes 16 j .. 16 j + 15 of its C
        const int i = t >> 2, j = t & 3;
        const int64_t r = rowmap[i];
        const int64_t c = c0 + 16 * j;
        uint32_t* row = tile_w + i * kPitchW + 4 * j;
        if (r >= 0 && c + 16 <= C && ((ld_src & 15) | ((uintptr_t)src & 15)) == 0) {
            const uint4 v = *reinterpret_cast<const uint4*>(src + r * ld_src + c);
            row[0] = v.x;
            row[1] = v.y;
            row[2] = v.z;
            row[3] = v.w;
        } else {
            uint8_t* b = tile + i * kPitch + 16 * j;
            for (int e = 0; e < 16; ++e) b[e] = (r >= 0 && c + e < C) ? src[r * ld_src + c + e] : (uint8_t)0;
        }
    } else {  // source row c0 + i, lanes along the destination columns
        const int64_t r = rowmap[lane];
        for (int i = w; i < kPT; i += 4) {
            const int64_t c = c0 + i;
            tile[lane * kPitch + i] = (r >= 0 && c < C) ? src[c * ld_src + r] : (uint8_t)0;
        }
    }
    __syncthreads();
    if (x0 + kPT <= dst_cols && c0 + kPT <= C) {  // uniform; dst_cols and the rows are 16-byte aligned
        const int c = t >> 2, q = t & 3;
        *reinterpret_cast<uint4*>(dst + (c0 + c) * dst_cols + x0 + 16 * q) = tile_column16(tile, c, q);
    } else {
        for (int i = w; i < kPT; i += 4) {
            const int64_t c = c0 + i, x = x0 + lane;
            if (x < dst_cols && c < C) dst[c * dst_cols + x] = tile[lane * kPitch + i];
        }
    }
}

}  // namespace

hipError_t launch_group_starts(const int* sizes, int G, int64_t* start, hipStream_t s) {
    hipLaunchKernelGGL(group_starts_kernel, dim3(1), dim3(64), 0, s, sizes, G, start);
    return hipGetLastError();
}

hipError_t launch_transpose(const uint8_t* src, int64_t L, int64_t R, int64_t C, int64_t ld_src, int64_t src_batch,
                            uint8_t* dst, int64_t ld_dst, int64_t dst_batch, hipStream_t s) {
    const dim3 grid((unsigned)((R + kPT - 1) / kPT), (unsigned)((C + kPT - 1) / kPT), (unsigned)L);
    hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, s, src, R, C, ld_src, src_batch, dst, ld_dst, dst_batch);
    return hipGetLastError();
}

hipError_t launch_group_pack(bool trans, const uint8_t* src, int64_t R, int64_t C, int64_t ld_src, uint8_t* dst,
                             int64_t dst_cols, const int* sizes, const int* offsets, const int64_t* start, int G,
                             hipStream_t s) {
    const dim3 grid((unsigned)((dst_cols + kPT - 1) / kPT), (unsigned)((C + kPT - 1) / kPT), 1);
    if (trans)
        hipLaunchKernelGGL(group_pack_kernel<true>, grid, dim3(256), 0, s, src, R, C, ld_src, dst, dst_cols, sizes,
                           offsets, start, G);
    else
        hipLaunchKernelGGL(group_pack_kernel<false>, grid, dim3(256), 0, s, src, R, C, ld_src, dst, dst_cols, sizes,
                           offsets, start, G);
    return hipGetLastError();
}

}  // namespace mmfp8
