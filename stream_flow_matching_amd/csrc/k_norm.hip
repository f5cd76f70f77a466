// Row-wise HBM-bound kernels: the fused AdaLN RMSNorm (+ per-token E4M3
// quantisation of its output), per-token quantisation of other GEMM inputs,
// the bf16-weight GEMV used for the AdaLN modulation and timestep MLP, and the
// sinusoidal timestep embedding.
//
// AdaLN (Ideogram 4.0 research note, "Model architecture": the timestep
// embedding produces per-block scale and gate for the attention and MLP
// residual paths): h = bf16(x / sqrt(mean(x^2) + eps) * (1 + scale)).
#include "sfm_internal.h"

namespace sfm {

namespace {

constexpr int kRowThreads = 256;
constexpr int kRowWaves = kRowThreads / 64;

// Each thread owns up to MAXC chunks of 8 bf16 (16 bytes) of the row.
template <int MAXC>
__device__ __forceinline__ void load_row(const uint16_t* row, int nchunk, float (&v)[MAXC][8]) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = threadIdx.x + c * kRowThreads;
        if (ch < nchunk) {
            const uint4 u = *reinterpret_cast<const uint4*>(row + (int64_t)ch * 8);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[c][2 * i] = __uint_as_float(w[i] << 16);
                v[c][2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[c][i] = 0.f;
        }
    }
}

// Quantise a row held in registers (already bf16 values) to E4M3 with the
// per-row scale alpha/448, and write codes + scale.
template <int MAXC>
__device__ __forceinline__ void quant_store_row(float (&v)[MAXC][8], int nchunk, float amax, uint8_t* qrow,
                                                float* srow) {
    const float inv = amax > 0.f ? 448.0f / amax : 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = threadIdx.x + c * kRowThreads;
        if (ch < nchunk) {
            uint32_t lo = 0, hi = 0;
            lo = cvt_fp8x2<false>(clamp448(v[c][0] * inv), clamp448(v[c][1] * inv), lo);
            lo = cvt_fp8x2<true>(clamp448(v[c][2] * inv), clamp448(v[c][3] * inv), lo);
            hi = cvt_fp8x2<false>(clamp448(v[c][4] * inv), clamp448(v[c][5] * inv), hi);
            hi = cvt_fp8x2<true>(clamp448(v[c][6] * inv), clamp448(v[c][7] * inv), hi);
            *reinterpret_cast<uint2*>(qrow + (int64_t)ch * 8) = make_uint2(lo, hi);
        }
    }
    if (threadIdx.x == 0) *srow = amax / 448.0f;
}

template <int MAXC, bool FP8>
__global__ __launch_bounds__(kRowThreads) void adaln_kernel(const uint16_t* __restrict__ x, int64_t rpb_in,
                                                            int64_t row_off, int rpb, const float* __restrict__ scale,
                                                            int64_t scale_stride, uint8_t* __restrict__ hq,
                                                            float* __restrict__ hs, uint16_t* __restrict__ h, int D,
                                                            float eps) {
    __shared__ float red[kRowWaves];
    const int64_t m = blockIdx.x;  // output row
    const int64_t b = m / rpb;
    const int64_t r = m % rpb;
    const uint16_t* xrow = x + (b * rpb_in + row_off + r) * D;
    const float* sc = scale + b * scale_stride;
    const int nchunk = D / 8;
    float v[MAXC][8];
    load_row<MAXC>(xrow, nchunk, v);
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += v[c][i] * v[c][i];
    ss = block_sum<kRowWaves>(ss, red);
    const float rinv = 1.0f / sqrtf(ss / (float)D + eps);
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = threadIdx.x + c * kRowThreads;
        if (ch < nchunk) {
            const float4 s0 = *reinterpret_cast<const float4*>(sc + ch * 8);
            const float4 s1 = *reinterpret_cast<const float4*>(sc + ch * 8 + 4);
            const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v[c][i] = round_bf16((v[c][i] * rinv) * (1.0f + s[i]));
                amax = fmaxf(amax, fabsf(v[c][i]));
            }
        }
    }
    if constexpr (FP8) {
        amax = block_max<kRowWaves>(amax, red);
        quant_store_row<MAXC>(v, nchunk, amax, hq + m * D, hs + m);
    } else {
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int ch = threadIdx.x + c * kRowThreads;
            if (ch < nchunk) {
                uint4 o;
                o.x = pack_bf16x2(v[c][0], v[c][1]);
                o.y = pack_bf16x2(v[c][2], v[c][3]);
                o.z = pack_bf16x2(v[c][4], v[c][5]);
                o.w = pack_bf16x2(v[c][6], v[c][7]);
                *reinterpret_cast<uint4*>(h + m * D + (int64_t)ch * 8) = o;
            }
        }
    }
}

// RMSNorm with a weight over a long fp32 row, rounded to bf16, then per-row
// E4M3 quantisation: the input side of the text-conditioning projection
// (SimpleTuner Ideogram 4 quick start, "Text embed cache": 13 x 4096 fp32
// features per token go through the frozen llm_cond_norm before
// llm_cond_proj).  One workgroup of 1024 threads per row; thread t holds the
// 4-element groups 4 (t + 1024 c), c < MAXC, in registers, so the row is read
// once: sum of squares, h = bf16(x * rinv * w) with its absolute maximum, then
// the codes.  cols % 4 == 0, cols <= 4096 MAXC.
constexpr int kLongThreads = 1024;

template <int MAXC>
__global__ __launch_bounds__(kLongThreads) void rmsnorm_f32_quant_kernel(const float* __restrict__ x, int cols,
                                                                         const uint16_t* __restrict__ w,
                                                                         uint8_t* __restrict__ q,
                                                                         float* __restrict__ s, float eps) {
    __shared__ float red[kLongThreads / 64];
    const int64_t m = blockIdx.x;
    const float* row = x + m * cols;
    float v[MAXC][4];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int i = 4 * (threadIdx.x + kLongThreads * c);
        float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < cols) u = *reinterpret_cast<const float4*>(row + i);
        v[c][0] = u.x;
        v[c][1] = u.y;
        v[c][2] = u.z;
        v[c][3] = u.w;
        ss += u.x * u.x + u.y * u.y + u.z * u.z + u.w * u.w;
    }
    ss = block_sum<kLongThreads / 64>(ss, red);
    const float rinv = 1.0f / sqrtf(ss / (float)cols + eps);
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int i = 4 * (threadIdx.x + kLongThreads * c);
        if (i < cols) {
            const uint2 g = *reinterpret_cast<const uint2*>(w + i);
            const float gw[4] = {__uint_as_float(g.x << 16), __uint_as_float(g.x & 0xFFFF0000u),
                                 __uint_as_float(g.y << 16), __uint_as_float(g.y & 0xFFFF0000u)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[c][e] = round_bf16((v[c][e] * rinv) * gw[e]);
                amax = fmaxf(amax, fabsf(v[c][e]));
            }
        }
    }
    amax = block_max<kLongThreads / 64>(amax, red);
    const float inv = amax > 0.f ? 448.0f / amax : 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int i = 4 * (threadIdx.x + kLongThreads * c);
        if (i < cols) {
            uint32_t code = 0;
            code = cvt_fp8x2<false>(clamp448(v[c][0] * inv), clamp448(v[c][1] * inv), code);
            code = cvt_fp8x2<true>(clamp448(v[c][2] * inv), clamp448(v[c][3] * inv), code);
            *reinterpret_cast<uint32_t*>(q + m * cols + i) = code;
        }
    }
    if (threadIdx.x == 0) s[m] = amax / 448.0f;
}

template <int MAXC>
__global__ __launch_bounds__(kRowThreads) void quant_rows_kernel(const uint16_t* __restrict__ a, int cols,
                                                                 uint8_t* __restrict__ q, float* __restrict__ s) {
    __shared__ float red[kRowWaves];
    const int64_t m = blockIdx.x;
    const int nchunk = cols / 8;
    float v[MAXC][8];
    load_row<MAXC>(a + m * cols, nchunk, v);
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
    amax = block_max<kRowWaves>(amax, red);
    quant_store_row<MAXC>(v, nchunk, amax, q + m * cols, s + m);
}

// out_l[b][n] = sum_k w_l[n][k] * act(in[b][k]) + bias_l[n] for the layers l
// of the grid's y dimension (weights and biases by pointer per layer, outputs
// out + l * out_stride); each wave computes kGemvR consecutive output rows
// (their weight rows in flight together), act = SiLU or identity; k % 8 == 0,
// B <= kGemvB.
constexpr int kGemvB = 8;
constexpr int kGemvR = 4;
__global__ __launch_bounds__(256) void gemv_kernel(const float* __restrict__ in, int act_silu, GemvLayers p,
                                                   float* __restrict__ out, int64_t out_stride, int B, int n_out,
                                                   int k) {
    extern __shared__ float xin[];  // [B][k]
    const uint16_t* __restrict__ w = p.w[blockIdx.y];
    const float* __restrict__ bias = p.bias[blockIdx.y];
    out += (int64_t)blockIdx.y * out_stride;
    for (int i = threadIdx.x; i < B * k; i += 256) {
        const float t = in[i];
        xin[i] = act_silu ? t / (1.0f + expf(-t)) : t;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int64_t n0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kGemvR;
    if (n0 >= n_out) return;
    float acc[kGemvR][kGemvB];
#pragma unroll
    for (int j = 0; j < kGemvR; ++j)
#pragma unroll
        for (int b = 0; b < kGemvB; ++b) acc[j][b] = 0.f;
    for (int k0 = lane * 8; k0 < k; k0 += 512) {
        uint4 u[kGemvR];
#pragma unroll
        for (int j = 0; j < kGemvR; ++j)
            u[j] = n0 + j < n_out ? *reinterpret_cast<const uint4*>(w + (n0 + j) * k + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < kGemvR; ++j) {
            const uint32_t ww[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
            float wf[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                wf[2 * i] = __uint_as_float(ww[i] << 16);
                wf[2 * i + 1] = __uint_as_float(ww[i] & 0xFFFF0000u);
            }
#pragma unroll
            for (int b = 0; b < kGemvB; ++b) {
                if (b < B) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[j][b] += wf[i] * xin[b * k + k0 + i];
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kGemvR; ++j)
#pragma unroll
        for (int b = 0; b < kGemvB; ++b) {
            if (b < B) {
                const float t = wave_sum_dpp(acc[j][b]);
                if (lane == 0 && n0 + j < n_out) out[(int64_t)b * n_out + n0 + j] = t + (bias ? bias[n0 + j] : 0.f);
            }
        }
}

// e[b][i] = cos(1000 t f_i), e[b][half + i] = sin(1000 t f_i), f_i = 10000^(-i/half);
// the angle and the trig functions in double precision, rounded to fp32.
__global__ void timestep_embed_kernel(float t, float* e, int B, int dim) {
    const int half = dim / 2;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= half) return;
    const double f = pow(10000.0, -(double)i / (double)half);
    const double a = 1000.0 * (double)t * f;
    const float c = (float)cos(a), s = (float)sin(a);
    for (int b = 0; b < B; ++b) {
        e[b * dim + i] = c;
        e[b * dim + half + i] = s;
    }
}

}  // namespace

hipError_t launch_gemv(const float* in, int act_silu, const uint16_t* w, const float* bias, float* out, int B,
                       int n_out, int k, hipStream_t st) {
    GemvLayers p{};
    p.w[0] = w;
    p.bias[0] = bias;
    return launch_gemv_layers(in, act_silu, p, 1, out, 0, B, n_out, k, st);
}

hipError_t launch_gemv_layers(const float* in, int act_silu, const GemvLayers& p, int layers, float* out,
                              int64_t out_stride, int B, int n_out, int k, hipStream_t st) {
    if (B > kGemvB || layers < 1 || layers > kGemvMaxLayers) return hipErrorInvalidValue;
    const size_t shm = (size_t)B * k * sizeof(float);
    hipLaunchKernelGGL(gemv_kernel, dim3((n_out + 4 * kGemvR - 1) / (4 * kGemvR), layers), dim3(256), shm, st, in,
                       act_silu, p, out, out_stride, B, n_out, k);
    return hipGetLastError();
}

template <bool FP8>
static hipError_t launch_adaln_any(const uint16_t* x, int64_t rpb_in, int64_t row_off, int rpb, const float* scale,
                                   int64_t scale_stride, uint8_t* hq, float* hs, uint16_t* h, int B, int D, float eps,
                                   hipStream_t st) {
    const int nchunk = D / 8;
    const dim3 grid((unsigned)((int64_t)B * rpb));
    if (nchunk <= kRowThreads)
        hipLaunchKernelGGL((adaln_kernel<1, FP8>), grid, dim3(kRowThreads), 0, st, x, rpb_in, row_off, rpb, scale,
                           scale_stride, hq, hs, h, D, eps);
    else if (nchunk <= 3 * kRowThreads)
        hipLaunchKernelGGL((adaln_kernel<3, FP8>), grid, dim3(kRowThreads), 0, st, x, rpb_in, row_off, rpb, scale,
                           scale_stride, hq, hs, h, D, eps);
    else if (nchunk <= 4 * kRowThreads)
        hipLaunchKernelGGL((adaln_kernel<4, FP8>), grid, dim3(kRowThreads), 0, st, x, rpb_in, row_off, rpb, scale,
                           scale_stride, hq, hs, h, D, eps);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_adaln_fp8(const uint16_t* x, int64_t rpb_in, int64_t row_off, int rpb, const float* scale,
                            int64_t scale_stride, uint8_t* hq, float* hs, int B, int D, float eps, hipStream_t st) {
    return launch_adaln_any<true>(x, rpb_in, row_off, rpb, scale, scale_stride, hq, hs, nullptr, B, D, eps, st);
}

hipError_t launch_adaln_bf16(const uint16_t* x, int64_t rpb_in, int64_t row_off, int rpb, const float* scale,
                             int64_t scale_stride, uint16_t* h, int B, int D, float eps, hipStream_t st) {
    return launch_adaln_any<false>(x, rpb_in, row_off, rpb, scale, scale_stride, nullptr, nullptr, h, B, D, eps, st);
}

hipError_t launch_quant_rows(const uint16_t* a, int rows, int cols, uint8_t* q, float* s, hipStream_t st) {
    const int nchunk = cols / 8;
    if (rows == 0) return hipSuccess;
    if (nchunk <= kRowThreads)
        hipLaunchKernelGGL(quant_rows_kernel<1>, dim3(rows), dim3(kRowThreads), 0, st, a, cols, q, s);
    else if (nchunk <= 3 * kRowThreads)
        hipLaunchKernelGGL(quant_rows_kernel<3>, dim3(rows), dim3(kRowThreads), 0, st, a, cols, q, s);
    else if (nchunk <= 6 * kRowThreads)
        hipLaunchKernelGGL(quant_rows_kernel<6>, dim3(rows), dim3(kRowThreads), 0, st, a, cols, q, s);
    else if (nchunk <= 8 * kRowThreads)
        hipLaunchKernelGGL(quant_rows_kernel<8>, dim3(rows), dim3(kRowThreads), 0, st, a, cols, q, s);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_rmsnorm_f32_quant(const float* x, int rows, int cols, const uint16_t* w, uint8_t* q, float* s,
                                    float eps, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    if (cols % 4) return hipErrorInvalidValue;
    const int chunks = (cols / 4 + kLongThreads - 1) / kLongThreads;
    if (chunks <= 4)
        hipLaunchKernelGGL(rmsnorm_f32_quant_kernel<4>, dim3(rows), dim3(kLongThreads), 0, st, x, cols, w, q, s, eps);
    else if (chunks <= 16)
        hipLaunchKernelGGL(rmsnorm_f32_quant_kernel<16>, dim3(rows), dim3(kLongThreads), 0, st, x, cols, w, q, s, eps);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_timestep_embed(float t, float* e, int B, int dim, hipStream_t st) {
    hipLaunchKernelGGL(timestep_embed_kernel, dim3((dim / 2 + 127) / 128), dim3(128), 0, st, t, e, B, dim);
    return hipGetLastError();
}

}  // namespace sfm
