// Shared pieces of the two projection kernels: the fused epilogues and the
// mapping of a workgroup's weight-tile rows onto weight rows.
#pragma once

#include "sfm_internal.h"

namespace sfm {

typedef float v4f __attribute__((ext_vector_type(4)));

// Weight row of B-tile row j.  For SwiGLU each wave's TN tile rows are TN/2
// gate rows followed by the TN/2 up rows of the same output columns, so a lane
// holds the gate and up values of one output column in its accumulators
// [i][j] and [i][j + FN/2].
template <int EPI, int BN, int TN>
__device__ __forceinline__ int64_t weight_row(int j, int tn, int N) {
    if constexpr (EPI == SFM_EPI_SWIGLU) {
        constexpr int half = TN / 2;
        const int wb = j / TN, jj = j % TN;
        const int64_t base = (int64_t)tn * (BN / 2) + wb * half;
        return jj < half ? base + jj : (int64_t)(N / 2) + base + (jj - half);
    } else {
        return (int64_t)tn * BN + j;
    }
}

// Epilogue over a wave's FM x FN grid of 16x16 accumulators.  Accumulator
// acc[i][j][r] of lane l is output row m0w + 16 i + 4 (l >> 4) + r and B-tile
// row n0w + 16 j + (l & 15).  row_scale(row) and col_scale(weight row) give the
// dequantisation factors (1 for bf16 operands).
template <int EPI, int BN, int TN, int FM, int FN, typename RowScale, typename ColScale>
__device__ __forceinline__ void gemm_epilogue(const v4f (&acc)[FM][FN], int m0w, int wn, int tn, int lane, int M,
                                              int N, int L, uint16_t* out, const uint16_t* resid, const float* gate,
                                              int64_t gate_stride, RowScale row_scale, ColScale col_scale) {
    const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m0w + i * 16 + 4 * lg + r;
            if (row >= M) continue;
            const float s_a = row_scale(row);
            if constexpr (EPI == SFM_EPI_SWIGLU) {
                const int F = N / 2;
#pragma unroll
                for (int j = 0; j < FN / 2; ++j) {
                    const int64_t col = (int64_t)tn * (BN / 2) + wn * (TN / 2) + j * 16 + lr;
                    const float g = acc[i][j][r] * s_a * col_scale(col);
                    const float u = acc[i][j + FN / 2][r] * s_a * col_scale(F + col);
                    const float sg = g / (1.0f + expf(-g));
                    out[(int64_t)row * F + col] = f32_to_bf16(sg * u);
                }
            } else {
                const int b = row / L;
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int64_t col = (int64_t)tn * BN + wn * TN + j * 16 + lr;
                    const float y = acc[i][j][r] * s_a * col_scale(col);
                    if constexpr (EPI == SFM_EPI_STORE) {
                        out[(int64_t)row * N + col] = f32_to_bf16(y);
                    } else {
                        const float xr = bf16_to_f32(resid[(int64_t)row * N + col]);
                        out[(int64_t)row * N + col] = f32_to_bf16(xr + gate[(int64_t)b * gate_stride + col] * y);
                    }
                }
            }
        }
    }
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on
// XCD b % 8); renumber so that each XCD gets one contiguous range of ids and
// the tiles it works on at the same time share its L2.
__device__ __forceinline__ int xcd_tile_id() {
    const int b = blockIdx.x, n = gridDim.x;
    const int q = n >> 3, r = n & 7, x = b & 7;
    return x * q + min(x, r) + (b >> 3);
}

// Tile (tm, tn) of linear id t in a grouped raster: ids walk GM tile-rows down
// before moving one tile-column right, so a run of 32 ids touches GM A
// row-blocks and 32 / GM weight column-blocks.
__device__ __forceinline__ void grouped_tile(int t, int ntm, int ntn, int GM, int& tm, int& tn) {
    const int group = t / (GM * ntn);
    const int first = group * GM;
    const int gm = min(ntm - first, GM);
    const int r = t - group * GM * ntn;
    tm = first + r % gm;
    tn = r / gm;
}

}  // namespace sfm
