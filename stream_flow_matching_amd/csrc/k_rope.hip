// QK-RMSNorm + 3-D MRoPE and the head-major relayout for attention.
//
// Research note, "Model architecture", block internals: QK-RMSNorm (ViT-22B
// style) and multimodal RoPE with mrope_section (24, 20, 20), rope_theta 5e6;
// text tokens use a 1-D position on all three axes, image tokens (t, h, w).
// Per token and head: u <- u / sqrt(mean(u^2) + eps) * gamma, then the pairs
// (j, j + 64), j < 64, rotate by the angle pos[axis(j)] * theta^(-j/64) with
// axis t for j < 24, h for 24 <= j < 44, w for 44 <= j < 64; dims 128..255
// pass through.  cos / sin come from the context's table (computed on the host
// in double precision, rounded to fp32), indexed by (integer position, j).
//
// One workgroup handles 64 tokens of one head.  q and k rows (256 dims) are
// processed two per wave at a time, 16 bytes per lane (lane & 31 owns dims
// 8c .. 8c+7, c = lane & 31), four row pairs in flight per wave: the row's sum
// of squares is reduced with DPP row rotations and a cross-row swap, and the
// rotation partner of dims 8c.. (c < 16) is the chunk c ^ 8, one DPP row
// rotation by 8 away.  Aligned groups of four pair indices never straddle a
// section boundary (24 and 44 are multiples of 4), so a lane's cos / sin come
// as two float4 loads per table.  The v slice is transposed through LDS into
// vt[b][h][d][token] as fp16 (every bf16 value with |v| <= 65504 is exact in
// fp16; larger ones saturate), the operand format of the attention kernel's P V
// product.  Inside every group of 32 tokens the stored order is
// [4g..4g+3, 16+4g..16+4g+3] for g = 0..3: the eight keys one lane of the
// attention kernel needs are then contiguous.
#include "sfm_internal.h"

namespace sfm {

namespace {

constexpr int kTok = 64;

__device__ __forceinline__ uint16_t bf16_to_f16_bits(uint16_t b) {
    const float f = fminf(fmaxf(bf16_to_f32(b), -65504.0f), 65504.0f);
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// x of lane (l & ~15) | ((l + 8) & 15): the chunk eight 16-byte chunks away in a 16-lane row
__device__ __forceinline__ float ror8(float x) { return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false)); }
__device__ __forceinline__ float ror_n(float x, int n) {
    switch (n) {
        case 4: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, false));
        case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xF, 0xF, false));
        default: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xF, 0xF, false));
    }
}
// sum over the 32 lanes of each half-wave
__device__ __forceinline__ float half_sum(float x) {
    x += ror8(x);
    x += ror_n(x, 4);
    x += ror_n(x, 2);
    x += ror_n(x, 1);
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ void unpack8(uint4 w, float (&u)[8]) {
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        u[2 * e] = __uint_as_float(a[e] << 16);
        u[2 * e + 1] = __uint_as_float(a[e] & 0xFFFF0000u);
    }
}

__global__ __launch_bounds__(256) void qk_norm_rope_kernel(const uint16_t* __restrict__ qkv,
                                                           const uint16_t* __restrict__ qn,
                                                           const uint16_t* __restrict__ kn,
                                                           const float* __restrict__ cos_t,
                                                           const float* __restrict__ sin_t, uint16_t* __restrict__ q,
                                                           uint16_t* __restrict__ k, uint16_t* __restrict__ vt, int T,
                                                           int gw, int L, int Lp, int H, float eps, TextLens lens,
                                                           int varlen) {
    __shared__ uint16_t vs[256][kTok + 2];  // [d][token] fp16 bits, padded row
    const int l0 = blockIdx.x * kTok;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int Tb = varlen ? lens.len[b] : T;
    const int D = H * 256;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row_stride = 3 * (int64_t)D;
    const uint16_t* base = qkv + (int64_t)b * L * row_stride;

    const int c = lane & 31, hw = lane >> 5;   // 16-byte chunk of the row, which row of the pair
    const bool rot = c < 16, first = c < 8;
    const int j0 = 8 * (c & 7);                // pair index of this lane's first dim (rotated chunks)
    const int axA = j0 < 24 ? 0 : (j0 < 44 ? 1 : 2), axB = j0 + 4 < 24 ? 0 : (j0 + 4 < 44 ? 1 : 2);
    float gq[8], gk[8];
    unpack8(*reinterpret_cast<const uint4*>(qn + 8 * c), gq);
    unpack8(*reinterpret_cast<const uint4*>(kn + 8 * c), gk);

    // 128 rows (64 q then 64 k), 8 per round of the four waves, 4 rounds per batch
    constexpr int kU = 4;
    for (int r0 = 0; r0 < 2 * kTok; r0 += 8 * kU) {
        float u[kU][8];
        int lrow[kU];
#pragma unroll
        for (int v = 0; v < kU; ++v) {
            const int r = r0 + 8 * v + 2 * wave + hw;
            const int part = r / kTok, l = l0 + r % kTok;
            lrow[v] = l;
            uint4 w = make_uint4(0, 0, 0, 0);
            if (l < L) w = *reinterpret_cast<const uint4*>(base + (int64_t)l * row_stride + part * D + h * 256 + 8 * c);
            unpack8(w, u[v]);
        }
#pragma unroll
        for (int v = 0; v < kU; ++v) {
            const int r = r0 + 8 * v + 2 * wave + hw;
            const int part = r / kTok, l = lrow[v];
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += u[v][e] * u[v][e];
            const float rn = 1.0f / sqrtf(half_sum(ss) / 256.0f + eps);
#pragma unroll
            for (int e = 0; e < 8; ++e) u[v][e] = u[v][e] * rn * (part == 0 ? gq[e] : gk[e]);
            const int lc = min(l, L - 1);
            const int pa = axis_pos(lc, T, Tb, gw, axA), pb = axis_pos(lc, T, Tb, gw, axB);
            const float4 ca = *reinterpret_cast<const float4*>(cos_t + pa * 64 + j0);
            const float4 cb = *reinterpret_cast<const float4*>(cos_t + pb * 64 + j0 + 4);
            const float4 sa = *reinterpret_cast<const float4*>(sin_t + pa * 64 + j0);
            const float4 sb = *reinterpret_cast<const float4*>(sin_t + pb * 64 + j0 + 4);
            const float cs[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
            const float sn[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = ror8(u[v][e]);
                // dims j (first half): a cos - b sin; dims j + 64: b cos + a sin
                const float rv = first ? u[v][e] * cs[e] - p * sn[e] : u[v][e] * cs[e] + p * sn[e];
                o[e] = rot ? rv : u[v][e];
            }
            uint16_t* dst = (part == 0 ? q : k) + (((int64_t)b * H + h) * Lp + l) * 256 + 8 * c;
            uint4 pk = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                                  pack_bf16x2(o[6], o[7]));
            if (l >= L) pk = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(dst) = pk;
        }
    }

    // v: load [64 tokens][256 d] (16 bytes per thread-step), store transposed into LDS
    for (int i = threadIdx.x; i < kTok * 32; i += 256) {
        const int t = i & 63, c = i >> 6;  // token t, 8-dim chunk c
        const int l = l0 + t;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (l < L) u = *reinterpret_cast<const uint4*>(base + (int64_t)l * row_stride + 2 * D + h * 256 + c * 8);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vs[c * 8 + 2 * e][t] = bf16_to_f16_bits((uint16_t)(w[e] & 0xFFFF));
            vs[c * 8 + 2 * e + 1][t] = bf16_to_f16_bits((uint16_t)(w[e] >> 16));
        }
    }
    __syncthreads();
    // write vt[b][h][d][l0 .. l0+63]: thread writes stored slots 8c .. 8c+7 (16 bytes) of one d row;
    // inside each group of 32 tokens, slot 8g + e holds token 4g + e (e < 4) or 16 + 4g + (e - 4)
    for (int i = threadIdx.x; i < 256 * (kTok / 8); i += 256) {
        const int d = i >> 3, c = i & 7;
        const int t0 = 32 * (c >> 2) + 4 * (c & 3);
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = t0 + (e >= 2 ? 16 : 0) + 2 * (e & 1);
            w[e] = (uint32_t)vs[d][t] | ((uint32_t)vs[d][t + 1] << 16);
        }
        uint16_t* dst = vt + (((int64_t)b * H + h) * 256 + d) * Lp + l0 + c * 8;
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// one workgroup per (head, sample): rows [L, Lp) of q and k, and the V^T columns that hold
// tokens [L, Lp) (inside the last partial group of 32 some of them sit before column L)
__global__ __launch_bounds__(256) void attn_pad_zero_kernel(uint16_t* __restrict__ q, uint16_t* __restrict__ k,
                                                            uint16_t* __restrict__ vt, int L, int Lp, int H) {
    const int h = blockIdx.x, b = blockIdx.y, np = Lp - L;
    const int64_t bh = (int64_t)b * H + h;
    uint16_t* qr = q + (bh * Lp + L) * 256;
    uint16_t* kr = k + (bh * Lp + L) * 256;
    for (int i = threadIdx.x; i < np * 256; i += 256) qr[i] = kr[i] = 0;
    for (int i = threadIdx.x; i < 256 * np; i += 256) {
        const int d = i / np, t = L + i % np;
        vt[(bh * 256 + d) * Lp + (t & ~31) + vt_slot(t & 31)] = 0;
    }
}

}  // namespace

hipError_t launch_attn_pad_zero(uint16_t* q, uint16_t* k, uint16_t* vt, int B, int L, int H, hipStream_t st) {
    const int Lp = padded_len(L);
    if (Lp == L || B == 0) return hipSuccess;
    hipLaunchKernelGGL(attn_pad_zero_kernel, dim3(H, B), dim3(256), 0, st, q, k, vt, L, Lp, H);
    return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const uint16_t* qkv, const uint16_t* qn, const uint16_t* kn, const float* cos_t,
                               const float* sin_t, uint16_t* q, uint16_t* k, uint16_t* vt, int B, int T, int gh,
                               int gw, int H, float eps, const TextLens* lens, hipStream_t st) {
    const int L = T + gh * gw;
    const int Lp = padded_len(L);
    TextLens tl{};
    if (lens) tl = *lens;
    hipLaunchKernelGGL(qk_norm_rope_kernel, dim3(Lp / kTok, H, B), dim3(256), 0, st, qkv, qn, kn, cos_t, sin_t, q,
                       k, vt, T, gw, L, Lp, H, eps, tl, lens ? 1 : 0);
    return hipGetLastError();
}

}  // namespace sfm
