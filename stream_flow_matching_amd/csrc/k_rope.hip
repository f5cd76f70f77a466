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
// One workgroup handles 64 tokens of one head: q and k rows are normalised and
// rotated one wave-row at a time (lane t owns dims 2t, 2t+1 and 128+2t,
// 128+2t+1; the rotation partner of dims 2t, 2t+1 lives in lane t ^ 32), and
// the v slice is transposed through LDS into vt[b][h][d][token] as fp16 (every
// bf16 value with |v| <= 65504 is exact in fp16; larger ones saturate), the
// operand format of the attention kernel's P V product.  Inside every group of
// 32 tokens the stored order is [4g..4g+3, 16+4g..16+4g+3] for g = 0..3: the
// eight keys one lane of the attention kernel needs are then contiguous.
#include "sfm_internal.h"

namespace sfm {

namespace {

constexpr int kTok = 64;

__device__ __forceinline__ uint16_t bf16_to_f16_bits(uint16_t b) {
    const float f = fminf(fmaxf(bf16_to_f32(b), -65504.0f), 65504.0f);
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ int axis_pos(int l, int T, int gw, int axis) {
    if (l < T) return l;
    const int i = l - T;
    if (axis == 0) return T;
    if (axis == 1) return T + i / gw;
    return T + i % gw;
}

__global__ __launch_bounds__(256) void qk_norm_rope_kernel(const uint16_t* __restrict__ qkv,
                                                           const uint16_t* __restrict__ qn,
                                                           const uint16_t* __restrict__ kn,
                                                           const float* __restrict__ cos_t,
                                                           const float* __restrict__ sin_t, uint16_t* __restrict__ q,
                                                           uint16_t* __restrict__ k, uint16_t* __restrict__ vt, int T,
                                                           int gw, int L, int Lp, int H, float eps) {
    __shared__ uint16_t vs[256][kTok + 2];  // [d][token] fp16 bits, padded row
    const int l0 = blockIdx.x * kTok;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int D = H * 256;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row_stride = 3 * (int64_t)D;
    const uint16_t* base = qkv + (int64_t)b * L * row_stride;

    // rotary index of this lane's first pair of dims
    const int j = (2 * lane) & 63;  // dims 2*lane, 2*lane+1 -> pair index j, j+1
    const bool first_half = lane < 32;
    const int axis = j < 24 ? 0 : (j < 44 ? 1 : 2);  // pairs never straddle a section boundary

    // q (part 0) and k (part 1): 2 * 64 rows of 256 per workgroup, one row per wave at a time
    for (int it = wave; it < 2 * kTok; it += 4) {
        const int part = it / kTok;
        const int l = l0 + (it % kTok);
        uint16_t* dst = (part == 0 ? q : k) + (((int64_t)b * H + h) * Lp + l) * 256;
        if (l >= L) {
            reinterpret_cast<uint32_t*>(dst)[lane] = 0u;
            reinterpret_cast<uint32_t*>(dst + 128)[lane] = 0u;
            continue;
        }
        const uint16_t* src = base + (int64_t)l * row_stride + part * D + h * 256;
        const uint32_t w0 = reinterpret_cast<const uint32_t*>(src)[lane];
        const uint32_t w1 = reinterpret_cast<const uint32_t*>(src + 128)[lane];
        float u0 = __uint_as_float(w0 << 16), u1 = __uint_as_float(w0 & 0xFFFF0000u);
        float u2 = __uint_as_float(w1 << 16), u3 = __uint_as_float(w1 & 0xFFFF0000u);
        const float ss = wave_sum(u0 * u0 + u1 * u1 + u2 * u2 + u3 * u3);
        const float r = 1.0f / sqrtf(ss / 256.0f + eps);
        const uint16_t* g = part == 0 ? qn : kn;
        u0 = u0 * r * bf16_to_f32(g[2 * lane]);
        u1 = u1 * r * bf16_to_f32(g[2 * lane + 1]);
        u2 = u2 * r * bf16_to_f32(g[128 + 2 * lane]);
        u3 = u3 * r * bf16_to_f32(g[128 + 2 * lane + 1]);
        const float p0 = __shfl_xor(u0, 32, 64);
        const float p1 = __shfl_xor(u1, 32, 64);
        const int pos = axis_pos(l, T, gw, axis);
        const float c0 = cos_t[pos * 64 + j], c1 = cos_t[pos * 64 + j + 1];
        const float s0 = sin_t[pos * 64 + j], s1 = sin_t[pos * 64 + j + 1];
        float o0, o1;
        if (first_half) {  // dims j, j+1: a*cos - b*sin
            o0 = u0 * c0 - p0 * s0;
            o1 = u1 * c1 - p1 * s1;
        } else {           // dims j+64, j+65: b*cos + a*sin
            o0 = u0 * c0 + p0 * s0;
            o1 = u1 * c1 + p1 * s1;
        }
        reinterpret_cast<uint32_t*>(dst)[lane] = pack_bf16x2(o0, o1);
        reinterpret_cast<uint32_t*>(dst + 128)[lane] = pack_bf16x2(u2, u3);
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

}  // namespace

hipError_t launch_qk_norm_rope(const uint16_t* qkv, const uint16_t* qn, const uint16_t* kn, const float* cos_t,
                               const float* sin_t, uint16_t* q, uint16_t* k, uint16_t* vt, int B, int T, int gh,
                               int gw, int H, float eps, hipStream_t st) {
    const int L = T + gh * gw;
    const int Lp = padded_len(L);
    hipLaunchKernelGGL(qk_norm_rope_kernel, dim3(Lp / kTok, H, B), dim3(256), 0, st, qkv, qn, kn, cos_t, sin_t, q,
                       k, vt, T, gw, L, Lp, H, eps);
    return hipGetLastError();
}

}  // namespace sfm
