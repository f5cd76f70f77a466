// Shared pieces of the two projection kernels: the fused epilogues and the
// mapping of a workgroup's weight-tile rows onto weight rows.
#pragma once

#include <atomic>
#include <cstdint>
#include <type_traits>

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

// Epilogue of a wave's TM x TN tile of 32x32 accumulators (TM = 32 FM,
// TN = 32 FN) computed with the weight fragment as the MFMA's first operand,
// so that acc[i][j] holds the transposed block: element r of acc[i][j] in lane
// l is tile row 32 i + (l & 31) and B-tile column 32 j + 8 (r >> 2) + 4 (l >> 5)
// + (r & 3).  A lane thus owns one row per i and four consecutive columns per
// (j, r >> 2): one row scale per i, the column scales four at a time, and one
// 8-byte (bf16) or 16-byte (fp32) LDS write per four values.  The tile is
// staged through the wave's own LDS region and read back in 16-byte row chunks
// for the global stores.
//   STORE / SWIGLU: bf16 rows of OC = TN (TN / 2) columns, 16-byte chunk c of
//     row r at physical chunk c ^ s(r) (s spreads the 32 rows of a write over
//     the banks).
//   RESID_GATE: gate * y staged in fp32, TM / 2 rows per pass, rows padded by one
//     chunk when TN / 4 chunks are not a multiple of 16 (else XOR-swizzled);
//     the pass's residual chunks are loaded before its staging writes, so their
//     latency overlaps them, then added on the way out (one bf16 rounding).
// Scales come from LDS, where the kernel put them before its main loop: rsl
// = row scales of the wave's rows, csl = scales of the wave's B-tile columns,
// gl = gate rows times column scales, gate[b][n] * sw[n], of batches bt0,
// bt0 + 1, bt0 + 2 (stride BN floats, offset to the wave's columns; RESID
// only), so that gate * y = (acc * sa) * gl.  The gate row of token row m is batch m / L
// and a wave's rows touch at most two batches (L >= TM).  lds: the wave's
// staging region (at least TM * TN * 2 bytes; the RESID padding needs
// TM / 2 * (TN * 4 + 16)).
template <int EPI, int BN, int TN, int FM, int FN>
__device__ __forceinline__ void gemm_epilogue_lds(const v16f (&acc)[FM][FN], uint8_t* lds, int m0w, int wn, int tn,
                                                    int lane, int M, int N, int L, uint16_t* out,
                                                    const uint16_t* resid, const float* rsl, const float* csl,
                                                    const float* gl, int bt0) {
    constexpr int TM = 32 * FM;
    const int lc = lane & 31, lg = lane >> 5;
    float rs[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) rs[i] = rsl[32 * i + lc];
    auto colscale = [&](int c) { return *reinterpret_cast<const v4f*>(csl + c); };

    if constexpr (EPI == SFM_EPI_STORE || EPI == SFM_EPI_SWIGLU) {
        constexpr bool SW = EPI == SFM_EPI_SWIGLU;
        constexpr int OC = SW ? TN / 2 : TN;  // output columns of the wave tile
        constexpr int NCH = OC / 8;           // 16-byte chunks per LDS row
        static_assert(NCH == 4 || NCH == 8 || NCH == 16, "row swizzle");
        // rows 16 / NCH apart share a bank line; XOR-ing their chunks by the row's line index
        // puts 16 consecutive rows on 16 distinct 16-byte bank slots
        auto swz = [](int ch, int row) { return ch ^ ((row / (16 / NCH)) & (NCH - 1)); };
        const int64_t ld_out = SW ? N / 2 : N;
        const int64_t col0 = SW ? (int64_t)tn * (BN / 2) + wn * (TN / 2) : (int64_t)tn * BN + wn * TN;
        constexpr int NJ = SW ? FN / 2 : FN;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            // the column scales of the four groups first (one wait instead of one per group)
            v4f cgs[4], cus[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                cgs[q] = colscale(32 * j + 8 * q + 4 * lg);
                if constexpr (SW) cus[q] = colscale(32 * j + 8 * q + 4 * lg + TN / 2);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = 32 * j + 8 * q + 4 * lg;
                const v4f cg = cgs[q];
                const v4f cu = SW ? cus[q] : cg;
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    float y[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (SW)
                            y[e] = swiglu_fast(acc[i][j][4 * q + e] * rs[i] * cg[e],
                                               acc[i][j + FN / 2][4 * q + e] * rs[i] * cu[e]);
                        else
                            y[e] = acc[i][j][4 * q + e] * rs[i] * cg[e];
                    }
                    const int row = 32 * i + lc;
                    *reinterpret_cast<uint2*>(lds + row * (OC * 2) + (swz(c >> 3, row) << 4) + lg * 8) =
                        make_uint2(cvt_bf16x2(y[0], y[1]), cvt_bf16x2(y[2], y[3]));
                }
            }
        }
        // read back: chunk q of the tile is row q / NCH, chunk q % NCH; 32-bit offsets from the
        // wave's first output element
        uint16_t* const obase = out + (int64_t)m0w * ld_out + col0;
#pragma unroll
        for (int s = 0; s < TM * NCH / 64; ++s) {
            const int q = 64 * s + lane, row = q / NCH, ch = q % NCH;
            const uint4 v = *reinterpret_cast<const uint4*>(lds + row * (OC * 2) + (swz(ch, row) << 4));
            if (m0w + row < M) *reinterpret_cast<uint4*>(obase + row * (int)ld_out + ch * 8) = v;
        }
    } else {
        constexpr int NCH = TN / 4;                   // 16-byte chunks (four fp32) per row
        constexpr bool PAD = NCH % 16 != 0;
        constexpr int PITCH = TN * 4 + (PAD ? 16 : 0);
        auto swz = [](int ch, int row) { return PAD ? ch : ch ^ (row & 15); };
        constexpr int PR = TM / 2;                    // rows per pass
        constexpr int NS = PR * NCH / 64;             // chunks per lane per pass
        static_assert(PR * NCH % 64 == 0, "whole chunks per lane");
        const int64_t col0 = (int64_t)tn * BN + wn * TN;
        const int r_first = min(m0w, M - 1), r_last = min(m0w + TM - 1, M - 1);
        const int b_first = r_first / L, b_last = r_last / L;
        const int row_split = (b_first + 1) * L;
        // 32-bit offsets from the wave's first row (residual rows past M are read as row M - 1)
        const uint16_t* const rbase = resid + (int64_t)m0w * N + col0;
        uint16_t* const obase = out + (int64_t)m0w * N + col0;
        const bool full = m0w + TM <= M;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            // residual chunks of this pass first: their latency overlaps the staging writes
            uint2 rv[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int q = 64 * s + lane, row = q / NCH, ch = q % NCH;
                const int grow = min(m0w + PR * p + row, M - 1);
                rv[s] = *reinterpret_cast<const uint2*>(rbase + (grow - m0w) * N + ch * 4);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                // gate * column scale of the first and the last batch of the wave's rows
                v4f g0[4], g1[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = 32 * j + 8 * q + 4 * lg;
                    g0[q] = *reinterpret_cast<const v4f*>(gl + (b_first - bt0) * BN + c);
                    g1[q] = *reinterpret_cast<const v4f*>(gl + (b_last - bt0) * BN + c);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = 32 * j + 8 * q + 4 * lg;
#pragma unroll
                    for (int ii = 0; ii < FM / 2; ++ii) {
                        const int i = p * (FM / 2) + ii;
                        const int row = 32 * ii + lc;  // row inside the pass
                        const v4f g = m0w + 32 * i + lc < row_split ? g0[q] : g1[q];
                        v4f v;
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = (acc[i][j][4 * q + e] * rs[i]) * g[e];
                        *reinterpret_cast<v4f*>(lds + row * PITCH + (swz(c >> 2, row) << 4)) = v;
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's own staging writes
            auto read_back = [&](auto guarded) {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const int q = 64 * s + lane, row = PR * p + q / NCH, ch = q % NCH;
                    const v4f v = *reinterpret_cast<const v4f*>(lds + (q / NCH) * PITCH + (swz(ch, q / NCH) << 4));
                    uint2 pk;
                    pk.x = cvt_bf16x2(bf16_to_f32((uint16_t)rv[s].x) + v[0],
                                      bf16_to_f32((uint16_t)(rv[s].x >> 16)) + v[1]);
                    pk.y = cvt_bf16x2(bf16_to_f32((uint16_t)rv[s].y) + v[2],
                                      bf16_to_f32((uint16_t)(rv[s].y >> 16)) + v[3]);
                    if (!decltype(guarded)::value || m0w + row < M)
                        *reinterpret_cast<uint2*>(obase + row * N + ch * 4) = pk;
                }
            };
            if (full)
                read_back(std::false_type{});
            else
                read_back(std::true_type{});
        }
    }
}

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once per
// device: the attribute is held per device, and `done` keeps one bit per device
// ordinal (0..63) for the kernel it belongs to.
inline void raise_lds_limit_once(const void* kern, size_t bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    const uint64_t bit = 1ull << (dev & 63);
    if (done.load(std::memory_order_acquire) & bit) return;
    (void)hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    done.fetch_or(bit, std::memory_order_release);
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
