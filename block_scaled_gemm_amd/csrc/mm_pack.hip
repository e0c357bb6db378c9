// Operand packing for the layouts whose contraction axis is not innermost in
// memory ("TileOPs: Linear Algebra Operators": BmmFP8FwdOp with b as [B, K, N],
// and GroupedGemmFwdOp's NN, TN and TT layouts). The GEMM kernels read both
// operands with the contraction innermost, so such an operand is first copied
// into a buffer in that order, one extra read and write of it, as the page
// describes for BmmFP8FwdOp.
//
// One kernel serves every case. A 64 x 64 byte tile of "rows" r (the axis that
// becomes innermost) and "columns" c goes through LDS; the output is
// dst[c][r + shift(r)]. TRANS: the source holds the tile as src[r][c] (a
// transpose); otherwise as src[c][r] (a copy that moves each row's bytes by
// shift). shift is 0 for the plain transposes; for groups that split the
// contraction it moves each group to its own 16-byte aligned start column,
// so that every group's slice is a GEMM operand of its own.
//
// The copies are bound by HBM traffic, not arithmetic: byte accesses along
// the contiguous axis, 64 consecutive bytes per wave instruction.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mm_launch.hpp"

namespace mmfp8 {

namespace {

constexpr int kPT = 64;  // tile edge in bytes

// Start columns of the groups in the packed buffer: group g begins at the sum
// of its predecessors' sizes, each rounded up to 16 (negative sizes count as
// 0). shift[g] = start[g] - offsets[g]: the move of group g's rows. One wave.
__global__ __launch_bounds__(64) void group_starts_kernel(const int* sizes, const int* offsets, int G,
                                                          int64_t* start, int64_t* shift) {
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
        if (g < G) {
            const int64_t s = before + incl - own;
            start[g] = s;
            shift[g] = s - offsets[g];
        }
        before += __shfl(incl, 63);
    }
}

// The group of packed row r: the last g with offsets[g] <= r (valid
// metadata puts r in that group; an empty group shares its start with the
// next and so is never the last). -1 when r precedes every group.
__device__ int group_of_row(const int* offsets, int G, int64_t r) {
    int lo = 0, hi = G;  // first g with offsets[g] > r lies in [lo, hi]
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)offsets[mid] <= r) lo = mid + 1;
        else hi = mid;
    }
    return lo - 1;
}

template <bool TRANS>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ src, int64_t R, int64_t C,
                                                   int64_t ld_src, int64_t src_batch, uint8_t* __restrict__ dst,
                                                   int64_t ld_dst, int64_t dst_batch, int64_t dst_cols,
                                                   const int* offsets, const int64_t* shift, int G) {
    __shared__ uint8_t tile[kPT][kPT + 1];  // [r][c]; the odd pitch spreads a column over the banks
    __shared__ int64_t sh[kPT];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t r0 = (int64_t)blockIdx.x * kPT, c0 = (int64_t)blockIdx.y * kPT;
    src += (int64_t)blockIdx.z * src_batch;
    dst += (int64_t)blockIdx.z * dst_batch;
    if (w == 0) {
        int64_t s = 0;
        const int64_t r = r0 + lane;
        if (G > 0 && r < R) {
            const int g = group_of_row(offsets, G, r);
            s = g >= 0 ? shift[g] : -(dst_cols + R);  // a row before every group is dropped
        }
        sh[lane] = s;
    }
    for (int i = w; i < kPT; i += 4) {
        if constexpr (TRANS) {  // source row r0 + i, lanes along c
            const int64_t r = r0 + i, c = c0 + lane;
            tile[i][lane] = (r < R && c < C) ? src[r * ld_src + c] : (uint8_t)0;
        } else {                // source row c0 + i, lanes along r
            const int64_t c = c0 + i, r = r0 + lane;
            tile[lane][i] = (r < R && c < C) ? src[c * ld_src + r] : (uint8_t)0;
        }
    }
    __syncthreads();
    for (int i = w; i < kPT; i += 4) {  // destination row c0 + i, lanes along r
        const int64_t c = c0 + i, r = r0 + lane;
        if (r < R && c < C) {
            const int64_t col = r + sh[lane];
            if (col >= 0 && col < dst_cols) dst[c * ld_dst + col] = tile[lane][i];
        }
    }
}

}  // namespace

hipError_t launch_group_starts(const int* sizes, const int* offsets, int G, int64_t* start, int64_t* shift,
                               hipStream_t s) {
    hipLaunchKernelGGL(group_starts_kernel, dim3(1), dim3(64), 0, s, sizes, offsets, G, start, shift);
    return hipGetLastError();
}

hipError_t launch_pack(bool trans, const uint8_t* src, int64_t L, int64_t R, int64_t C, int64_t ld_src,
                       int64_t src_batch, uint8_t* dst, int64_t ld_dst, int64_t dst_batch, int64_t dst_cols,
                       const int* offsets, const int64_t* shift, int G, hipStream_t s) {
    const dim3 grid((unsigned)((R + kPT - 1) / kPT), (unsigned)((C + kPT - 1) / kPT), (unsigned)L);
    if (trans)
        hipLaunchKernelGGL(pack_kernel<true>, grid, dim3(256), 0, s, src, R, C, ld_src, src_batch, dst, ld_dst,
                           dst_batch, dst_cols, offsets, shift, G);
    else
        hipLaunchKernelGGL(pack_kernel<false>, grid, dim3(256), 0, s, src, R, C, ld_src, src_batch, dst, ld_dst,
                           dst_batch, dst_cols, offsets, shift, G);
    return hipGetLastError();
}

}  // namespace mmfp8
