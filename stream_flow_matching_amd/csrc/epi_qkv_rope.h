// The QKV projection's epilogue with QK-RMSNorm and the 3D rotary embedding
// folded in, shared by the FP8 and the NF4 GEMMs (launch_gemm_fp8_qkv_rope,
// launch_gemm_nf4_qkv_rope).  Research note "Ideogram 4.0", "Model
// architecture": RMSNorm of each head's q and k with a learned gamma, then
// MRoPE over the first 128 dims in sections of 24 / 20 / 20 frequency pairs
// (time / height / width axis); v passes unchanged.
#pragma once

#include "gemm_common.h"

namespace sfm {

namespace {

// QKV epilogue with QK-RMSNorm and the rotary embedding folded in
constexpr int kEpiQkvRope = 4;

// The epilogue of a wave's 128 x 128 accumulator block (acc[i][j][r] = row 32 i + (l & 31),
// column 32 j + 8 (r >> 2) + 4 (l >> 5) + (r & 3), as in gemm_epilogue_lds) of a 256 x 256 tile
// of the QKV output: with 256-column tiles, tile column tn is head tn % H of q, k or v
// (part tn / H), and the wave holds columns wn 128 .. wn 128 + 127 of that head.  Every value
// is first rounded to bf16 (the projection's output precision); for q and k these values
// overwrite the accumulators, which the normalising pass then reads.  gml: the tile's gamma (q_norm
// for q tiles, k_norm for k tiles) as 128 packed bf16 pairs in LDS, loaded by the kernel at its
// start (load_qk_gamma).
//   q, k: the row's sum of squares over the head (the lane, its partner lane l ^ 32, then the
//     other column wave through `xch` in LDS), u / sqrt(mean(u^2) + eps) * gamma, and for the
//     dims j < 64 / j + 64 of wave 0 the rotation of pair j (the partner of fragment column j
//     is fragment column j + 2 of the same lane) by the row's position on pair j's axis; bf16
//     rows staged through the wave's LDS region and stored as 16-byte chunks at
//     q / k[b][h][l][d].
//   v: fp16 (saturated at +-65504), transposed through LDS into [d][token] in the stored key
//     order of vt_slot and stored as 16-byte chunks of V^T[b][h][d][l] when the wave's rows are
//     128 valid rows of one sample starting at a multiple of 32 of its sequence; otherwise each
//     value is stored on its own.
// The kernel prologue's part of the epilogue: thread tid < 128 loads dword tid of the gamma of
// tile column tn's part (q_norm for q heads, k_norm for k heads; none for v) for gml.
__device__ __forceinline__ uint32_t load_qk_gamma(const RopeArgs& ra, int tn, int tid) {
    const int part = tn / ra.H;
    if (part >= 2 || tid >= 128) return 0u;
    return reinterpret_cast<const uint32_t*>(part == 0 ? ra.qn : ra.kn)[tid];
}

template <int FM, int FN>
__device__ __forceinline__ void epilogue_qkv_rope(v16f (&acc)[FM][FN], uint8_t* lds, float* xch, int m0w,
                                                  int wm, int wn, int tn, int lane, int M, int L, const float* rsl,
                                                  const float* csl, const uint32_t* gml, const RopeArgs& ra) {
    constexpr int TM = 32 * FM, TN = 32 * FN;
    static_assert(TM == 128 && TN == 128, "a 256 x 256 tile: one head per tile column");
    const int lc = lane & 31, lg = lane >> 5;
    const int part = tn / ra.H, h = tn - part * ra.H;
    float rs[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) rs[i] = rsl[32 * i + lc];
    // the column scales of a group of four columns; the projection's output values (bf16, the
    // STORE epilogue's rounding) of accumulator elements (i, j, 4 q .. 4 q + 3) under them
    auto colscale = [&](int j, int q) { return *reinterpret_cast<const v4f*>(csl + 32 * j + 8 * q + 4 * lg); };
    auto y4 = [&](int i, int j, int q, v4f cs) {
        const uint32_t lo = cvt_bf16x2(acc[i][j][4 * q] * rs[i] * cs[0], acc[i][j][4 * q + 1] * rs[i] * cs[1]);
        const uint32_t hi = cvt_bf16x2(acc[i][j][4 * q + 2] * rs[i] * cs[2], acc[i][j][4 * q + 3] * rs[i] * cs[3]);
        return v4f{__uint_as_float(lo << 16), __uint_as_float(lo & 0xFFFF0000u), __uint_as_float(hi << 16),
                   __uint_as_float(hi & 0xFFFF0000u)};
    };
    // the wave's rows span at most two samples (L >= 256 > TM)
    const int b_first = min(m0w, M - 1) / L, split = (b_first + 1) * L;
    if (part < 2) {
        // the rows' positions on the three axes and the first column group's cos / sin (wave 0
        // rotates), ahead of the sums of squares so that the loads' latency runs under them
        int pax[FM][3];
        if (wn == 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int m = min(m0w + 32 * i + lc, M - 1);
                const int b = m < split ? b_first : b_first + 1, l = m - b * L;
                const int Tb = ra.varlen ? ra.lens.len[b] : ra.T;
#pragma unroll
                for (int a = 0; a < 3; ++a) pax[i][a] = axis_pos(l, ra.T, Tb, ra.gw, a);
            }
        }
        // wave 0: cos / sin of the four rows for column group g = 4 j + q (pairs p0 .. p0 + 3, which
        // share an axis: the section boundaries 24 and 44 are multiples of 4), one group ahead
        v4f c2[2][FM], s2[2][FM];
        auto load_cs = [&](int slot, int g) {
            const int p0 = 32 * (g >> 2) + 8 * (g & 3) + 4 * lg;
            const int ax = p0 < 24 ? 0 : (p0 < 44 ? 1 : 2);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                c2[slot][i] = *reinterpret_cast<const v4f*>(ra.cos_t + pax[i][ax] * 64 + p0);
                s2[slot][i] = *reinterpret_cast<const v4f*>(ra.sin_t + pax[i][ax] * 64 + p0);
            }
        };
        if (wn == 0) load_cs(0, 0);
        // the output values replace the accumulators, which the normalisation below reads back
        float rn[FM] = {};
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v4f cs = colscale(j, q);
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const v4f u = y4(i, j, q, cs);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        rn[i] += u[e] * u[e];
                        acc[i][j][4 * q + e] = u[e];
                    }
                }
            }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            rn[i] += __shfl_xor(rn[i], 32, 64);
            if (lg == 0) xch[(2 * wm + wn) * TM + 32 * i + lc] = rn[i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < FM; ++i)
            rn[i] = 1.0f / sqrtf((rn[i] + xch[(2 * wm + (wn ^ 1)) * TM + 32 * i + lc]) / 256.0f + ra.eps);
        // gamma (q_norm or k_norm of the tile's part) from LDS, where the kernel put it at its start
        auto gamma4 = [&](int j, int q) {
            const uint2 g2 = *reinterpret_cast<const uint2*>(gml + (wn * TN + 32 * j + 8 * q + 4 * lg) / 2);
            return v4f{__uint_as_float(g2.x << 16), __uint_as_float(g2.x & 0xFFFF0000u), __uint_as_float(g2.y << 16),
                       __uint_as_float(g2.y & 0xFFFF0000u)};
        };
        // bf16 rows of 128 columns: 16-byte chunk c of row r at physical chunk c ^ (r & 15)
        auto stage = [&](int row, int ch, v4f o) {
            *reinterpret_cast<uint2*>(lds + row * 256 + ((ch ^ (row & 15)) << 4) + lg * 8) =
                make_uint2(cvt_bf16x2(o[0], o[1]), cvt_bf16x2(o[2], o[3]));
        };
#pragma unroll
        for (int j = 0; j < FN / 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // columns c (fragment column j) and c + 64 (fragment column j + 2)
                const int g = 4 * j + q;
                if (wn == 0 && g + 1 < 2 * FN) load_cs((g + 1) & 1, g + 1);
                const v4f ga = gamma4(j, q), gb = gamma4(j + FN / 2, q);
                const v4f* c = c2[g & 1];
                const v4f* sn = s2[g & 1];
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    v4f a, bb;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a[e] = acc[i][j][4 * q + e];
                        bb[e] = acc[i][j + FN / 2][4 * q + e];
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a[e] = a[e] * rn[i] * ga[e];
                        bb[e] = bb[e] * rn[i] * gb[e];
                    }
                    if (wn == 0) {
                        v4f ra4, rb4;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            ra4[e] = a[e] * c[i][e] - bb[e] * sn[i][e];
                            rb4[e] = bb[e] * c[i][e] + a[e] * sn[i][e];
                        }
                        a = ra4;
                        bb = rb4;
                    }
                    stage(32 * i + lc, 4 * j + q, a);
                    stage(32 * i + lc, 4 * (j + FN / 2) + q, bb);
                }
            }
        uint16_t* const dst = part == 0 ? ra.q : ra.k;
#pragma unroll
        for (int s = 0; s < TM * 16 / 64; ++s) {
            const int qq = 64 * s + lane, row = qq >> 4, ch = qq & 15;
            const uint4 v = *reinterpret_cast<const uint4*>(lds + row * 256 + ((ch ^ (row & 15)) << 4));
            const int m = m0w + row;
            if (m < M) {
                const int b = m < split ? b_first : b_first + 1, l = m - b * L;
                *reinterpret_cast<uint4*>(dst + (((int64_t)b * ra.H + h) * ra.Lp + l) * 256 + wn * TN + ch * 8) = v;
            }
        }
    } else {
        auto f16 = [](float v) { return (_Float16)fminf(fmaxf(v, -65504.0f), 65504.0f); };
        const int l0 = m0w - b_first * L;
        if (m0w + TM <= split && m0w + TM <= M && (l0 & 31) == 0) {
            // [d][stored token] fp16 rows of 256 bytes: 16-byte chunk c of row d at physical chunk
            // c ^ ((d >> 2) & 15); the lane's token 32 i + lc sits at 32 i + vt_slot(lc)
            const int sl = vt_slot(lc);
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const v4f cs = colscale(j, q);
#pragma unroll
                    for (int i = 0; i < FM; ++i) {
                        const v4f u = y4(i, j, q, cs);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int d = 32 * j + 8 * q + 4 * lg + e, t = 32 * i + sl;
                            *reinterpret_cast<_Float16*>(lds + d * 256 + (((t >> 3) ^ ((d >> 2) & 15)) << 4) +
                                                         (t & 7) * 2) = f16(u[e]);
                        }
                    }
                }
            uint16_t* const vt = ra.vt + ((int64_t)b_first * ra.H + h) * 256 * ra.Lp;
#pragma unroll
            for (int s = 0; s < TN * 16 / 64; ++s) {
                const int qq = 64 * s + lane, d = qq >> 4, ch = qq & 15;
                const uint4 v = *reinterpret_cast<const uint4*>(lds + d * 256 + ((ch ^ ((d >> 2) & 15)) << 4));
                *reinterpret_cast<uint4*>(vt + (int64_t)(wn * TN + d) * ra.Lp + l0 + ch * 8) = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int m = m0w + 32 * i + lc;
                if (m >= M) continue;
                const int b = m < split ? b_first : b_first + 1, l = m - b * L;
                _Float16* const base = reinterpret_cast<_Float16*>(ra.vt) +
                                       (((int64_t)b * ra.H + h) * 256 + wn * TN) * ra.Lp + (l & ~31) + vt_slot(l & 31);
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const v4f u = y4(i, j, q, colscale(j, q));
#pragma unroll
                        for (int e = 0; e < 4; ++e) base[(int64_t)(32 * j + 8 * q + 4 * lg + e) * ra.Lp] = f16(u[e]);
                    }
            }
        }
    }
}

}  // namespace

}  // namespace sfm
