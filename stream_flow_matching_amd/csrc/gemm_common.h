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

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (v_cvt_pk_bf16_f32, round to nearest even): low half a.
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// silu(g) * u with the hardware exp2 and reciprocal (each within 1 ulp in
// fp32; the product is rounded to bf16 afterwards).
__device__ __forceinline__ float swiglu_fast(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g)) * u;
}

// Epilogue over a wave's FM x FN grid of 32x32 accumulators: element r of
// acc[i][j] in lane l is output row m0w + 32 i + 8 (r >> 2) + 4 (l >> 5) + (r & 3)
// and B-tile row n0w + 32 j + (l & 31).  Every value is computed (rows past M
// hold copies of row M - 1); only the stores are predicated, and a wave whose
// rows are all in range stores without checks.
template <int EPI, int BN, int TN, int FM, int FN, typename RowScale, typename ColScale>
__device__ __forceinline__ void gemm_epilogue32(const v16f (&acc)[FM][FN], int m0w, int wn, int tn, int lane, int M,
                                                int N, int L, uint16_t* out, const uint16_t* resid, const float* gate,
                                                int64_t gate_stride, RowScale row_scale, ColScale col_scale) {
    const int lc = lane & 31, lg = lane >> 5;
    const bool full = m0w + 32 * FM <= M;
    if constexpr (EPI == SFM_EPI_SWIGLU) {
        const int F = N / 2;
        float cg[FN / 2], cu[FN / 2];
        int64_t col[FN / 2];
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
            col[j] = (int64_t)tn * (BN / 2) + wn * (TN / 2) + j * 32 + lc;
            cg[j] = col_scale(col[j]);
            cu[j] = col_scale(F + col[j]);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0w + i * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
                const float s_a = row_scale(min(row, M - 1));
#pragma unroll
                for (int j = 0; j < FN / 2; ++j) {
                    const float g = acc[i][j][r] * s_a * cg[j];
                    const float u = acc[i][j + FN / 2][r] * s_a * cu[j];
                    const uint16_t v = (uint16_t)cvt_bf16x2(swiglu_fast(g, u), 0.f);
                    if (full || row < M) out[(int64_t)row * F + col[j]] = v;
                }
            }
        }
    } else {
        float cs[FN];
        int64_t col[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            col[j] = (int64_t)tn * BN + wn * TN + j * 32 + lc;
            cs[j] = col_scale(col[j]);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0w + i * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
                const int rc = min(row, M - 1);
                const float s_a = row_scale(rc);
                const float* gb = gate + (int64_t)(rc / L) * gate_stride;
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const float y = acc[i][j][r] * s_a * cs[j];
                    const int64_t o = (int64_t)row * N + col[j];
                    if constexpr (EPI == SFM_EPI_STORE) {
                        if (full || row < M) out[o] = (uint16_t)cvt_bf16x2(y, 0.f);
                    } else {
                        if (full || row < M) {
                            const float xr = bf16_to_f32(resid[o]);
                            out[o] = (uint16_t)cvt_bf16x2(xr + gb[col[j]] * y, 0.f);
                        }
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
