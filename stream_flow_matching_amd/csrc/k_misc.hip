// Small kernels: the asymmetric-CFG Euler update, standalone weight
// dequantisation, the fp32-accumulating linear used by the latent embedding and
// the final projection, and a strided row copy for assembling [text | image].
#include "sfm_internal.h"

namespace sfm {

namespace {

// Research note, "Training method": Euler step z_{t-dt} = z_t + v dt on the
// guided velocity; asymmetric CFG v = v_u + w (v_c - v_u) (scale 4.0 in the
// deployment post, section 1.3).  Four elements per thread.
__global__ void euler_cfg_kernel(const float* __restrict__ z, const float* __restrict__ vc,
                                 const float* __restrict__ vu, float* zo, float* vo, int64_t n, float g, float dt) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i + 4 <= n) {
        const float4 a = *reinterpret_cast<const float4*>(z + i);
        const float4 c = *reinterpret_cast<const float4*>(vc + i);
        const float4 u = *reinterpret_cast<const float4*>(vu + i);
        float4 v, r;
        v.x = u.x + g * (c.x - u.x);
        v.y = u.y + g * (c.y - u.y);
        v.z = u.z + g * (c.z - u.z);
        v.w = u.w + g * (c.w - u.w);
        r.x = a.x + dt * v.x;
        r.y = a.y + dt * v.y;
        r.z = a.z + dt * v.z;
        r.w = a.w + dt * v.w;
        *reinterpret_cast<float4*>(zo + i) = r;
        if (vo) *reinterpret_cast<float4*>(vo + i) = v;
    } else {
        for (int64_t j = i; j < n; ++j) {
            const float v = vu[j] + g * (vc[j] - vu[j]);
            zo[j] = z[j] + dt * v;
            if (vo) vo[j] = v;
        }
    }
}

// OCP E4M3FN code -> fp32 (exact): E == 0 is m * 2^-9, otherwise
// (1 + m/8) * 2^(E-7), rebuilt as fp32 bits; 0x7F / 0xFF are NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float v = e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    if (e == 15u && m == 7u) v = __uint_as_float(0x7FC00000u);
    return (c & 0x80u) ? -v : v;
}

// FP8: w = fp32(decode(q) * s[n]); 8 weights per thread.
__global__ void dequant_fp8_kernel(const uint8_t* __restrict__ q, const float* __restrict__ s, void* out,
                                   int out_bf16, int n, int k) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i >= (int64_t)n * k) return;
    const int64_t row = i / k;
    const float sc = s[row];
    const uint2 u = *reinterpret_cast<const uint2*>(q + i);
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = e4m3_to_f32((u.x >> (8 * e)) & 0xFFu) * sc;
        v[4 + e] = e4m3_to_f32((u.y >> (8 * e)) & 0xFFu) * sc;
    }
    if (out_bf16) {
        uint4 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        o.z = pack_bf16x2(v[4], v[5]);
        o.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + i) = o;
    } else {
        float* f = reinterpret_cast<float*>(out) + i;
        *reinterpret_cast<float4*>(f) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(f + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// MXFP4: w = e2m1(q) * 2^(e - 127) for the E8M0 exponent e of the 32-element block; 8 weights
// (4 bytes, element 2i in the low nibble) per thread.  E2M1: sign, 2 exponent bits (bias 1,
// 0 = subnormal halves), 1 mantissa bit.  The product is exact (ldexp of a 2-bit significand).
__global__ void dequant_mx_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ ex, void* out,
                                  int out_bf16, int n, int k) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i >= (int64_t)n * k) return;
    const int sh = (int)ex[i / 32] - 127;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(q + i / 2);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t c = (w >> (4 * e)) & 15u;
        const uint32_t ee = (c >> 1) & 3u, m = c & 1u;
        const float mag = ee == 0 ? 0.5f * (float)m : __builtin_ldexpf(1.0f + 0.5f * (float)m, (int)ee - 1);
        v[e] = __builtin_ldexpf((c & 8u) ? -mag : mag, sh);
    }
    if (out_bf16) {
        uint4 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        o.z = pack_bf16x2(v[4], v[5]);
        o.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + i) = o;
    } else {
        float* f = reinterpret_cast<float*>(out) + i;
        *reinterpret_cast<float4*>(f) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(f + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// NF4: w = fp32(code[q] * absmax[block of 64]); 8 weights (4 bytes) per thread.
__global__ void dequant_nf4_kernel(const uint8_t* __restrict__ q, const float* __restrict__ absmax, Nf4Code code,
                                   void* out, int out_bf16, int n, int k) {
    __shared__ float lut[16];
    if (threadIdx.x < 16) lut[threadIdx.x] = code.v[threadIdx.x];
    __syncthreads();
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i >= (int64_t)n * k) return;
    const float am = absmax[i / 64];
    const uint32_t w = *reinterpret_cast<const uint32_t*>(q + i / 2);
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t byte = (w >> (8 * e)) & 0xFFu;
        v[2 * e] = lut[byte >> 4] * am;
        v[2 * e + 1] = lut[byte & 15] * am;
    }
    if (out_bf16) {
        uint4 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        o.z = pack_bf16x2(v[4], v[5]);
        o.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + i) = o;
    } else {
        float* f = reinterpret_cast<float*>(out) + i;
        *reinterpret_cast<float4*>(f) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(f + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// out[m][n] = sum_k a[m][k] w[n][k] + bias[n] with fp32 FMA accumulation:
// 64 x 64 output tile per workgroup, 4 x 4 outputs per thread, k-steps of 32
// staged in LDS as fp32.
constexpr int kSL = 64, kSK = 32;
template <bool A_BF16, bool O_BF16>
__global__ __launch_bounds__(256) void small_linear_kernel(const void* __restrict__ a_, int64_t a_rpb,
                                                           int64_t a_bs, int64_t a_off, const uint16_t* __restrict__ w,
                                                           const float* __restrict__ bias, void* out_, int64_t o_rpb,
                                                           int64_t o_bs, int64_t o_off, int M, int N, int K) {
    __shared__ float as[kSK][kSL + 4];
    __shared__ float ws[kSK][kSL + 4];
    const int m0 = blockIdx.x * kSL, n0 = blockIdx.y * kSL;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += kSK) {
        // 64 rows x 32 k = 2048 values each for a and w: 8 per thread
        for (int e = threadIdx.x; e < kSL * kSK; e += 256) {
            const int r = e / kSK, kk = e % kSK;
            const int m = min(m0 + r, M - 1);
            const int64_t arow = (m / a_rpb) * a_bs + a_off + m % a_rpb;
            float av;
            if constexpr (A_BF16)
                av = bf16_to_f32(reinterpret_cast<const uint16_t*>(a_)[arow * K + k0 + kk]);
            else
                av = reinterpret_cast<const float*>(a_)[arow * K + k0 + kk];
            as[kk][r] = av;
            const int nn = min(n0 + r, N - 1);
            ws[kk][r] = bf16_to_f32(w[(int64_t)nn * K + k0 + kk]);
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < kSK; ++kk) {
            float av[4], wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = as[kk][ty * 4 + i];
                wv[i] = ws[kk][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], wv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= M) continue;
        const int64_t orow = (m / o_rpb) * o_bs + o_off + m % o_rpb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= N) continue;
            const float y = acc[i][j] + (bias ? bias[n] : 0.f);
            if constexpr (O_BF16)
                reinterpret_cast<uint16_t*>(out_)[orow * N + n] = f32_to_bf16(y);
            else
                reinterpret_cast<float*>(out_)[orow * N + n] = y;
        }
    }
}

// out fp32 = A W^T + bias for a bf16 A (row mapping as above) and bf16 W [N][K]
// on bf16 matrix cores: a workgroup computes 32 rows x 128 columns, wave w the
// columns 32w .. 32w+31 as 2 x 2 tiles of v_mfma_f32_16x16x32_bf16 (fp32
// accumulation).  A and W fragments come straight from global memory (16
// contiguous bytes of K per lane) in batches of four k-steps, one batch ahead.
// K % 32 == 0.  Rows are clamped for loading, columns past N are not stored.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void bf16_linear_f32_kernel(const uint16_t* __restrict__ a, int64_t a_rpb,
                                                              int64_t a_bs, int64_t a_off,
                                                              const uint16_t* __restrict__ w,
                                                              const float* __restrict__ bias, float* __restrict__ out,
                                                              int64_t o_rpb, int64_t o_bs, int64_t o_off, int M, int N,
                                                              int K) {
    constexpr int kB = 4;  // k-steps of 32 per batch
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int m0 = blockIdx.x * 32, n0 = blockIdx.y * 128 + wave * 32;
    const uint16_t* ap[2];
    const uint16_t* wp[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = min(m0 + 16 * i + lr, M - 1);
        ap[i] = a + ((m / a_rpb) * a_bs + a_off + m % a_rpb) * K + 8 * lg;
        const int n = min(n0 + 16 * i + lr, N - 1);
        wp[i] = w + (int64_t)n * K + 8 * lg;
    }
    f32x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t fa[2][kB][2], fb[2][kB][2];
    auto load = [&](int slot, int k0) {
#pragma unroll
        for (int s = 0; s < kB; ++s)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int k = min(k0 + 32 * s, K - 32);
                fa[slot][s][i] = *reinterpret_cast<const bf16x8_t*>(ap[i] + k);
                fb[slot][s][i] = *reinterpret_cast<const bf16x8_t*>(wp[i] + k);
            }
    };
    const int nb = (K / 32 + kB - 1) / kB;
    load(0, 0);
    for (int bt = 0; bt < nb; bt += 2) {
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int b = bt + par;
            if (b >= nb) break;
            if (b + 1 < nb) load(par ^ 1, (b + 1) * kB * 32);
#pragma unroll
            for (int s = 0; s < kB; ++s) {
                if ((b * kB + s) * 32 >= K) break;
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[par][s][i], fb[par][s][j], acc[i][j],
                                                                            0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + 16 * j + lr;
            if (n >= N) continue;
            const float bn = bias ? bias[n] : 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * i + 4 * lg + r;
                if (m >= M) continue;
                out[((m / o_rpb) * o_bs + o_off + m % o_rpb) * N + n] = acc[i][j][r] + bn;
            }
        }
}

// dst rows b*dst_rpb + r <- src rows b*src_rpb + r, r < rows; cols % 8 == 0.
__global__ void copy_rows_kernel(const uint16_t* __restrict__ src, int64_t src_rpb, uint16_t* __restrict__ dst,
                                 int64_t dst_rpb, int rows, int cols) {
    const int64_t row = blockIdx.x;
    const int b = blockIdx.y;
    const uint16_t* s = src + ((int64_t)b * src_rpb + row) * cols;
    uint16_t* d = dst + ((int64_t)b * dst_rpb + row) * cols;
    for (int c = threadIdx.x * 8; c < cols; c += blockDim.x * 8)
        *reinterpret_cast<uint4*>(d + c) = *reinterpret_cast<const uint4*>(s + c);
}

}  // namespace

hipError_t launch_euler_cfg(const float* z, const float* vc, const float* vu, float* zo, float* vo, int64_t n,
                            float g, float dt, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int64_t threads = (n + 3) / 4;
    hipLaunchKernelGGL(euler_cfg_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, z, vc, vu, zo,
                       vo, n, g, dt);
    return hipGetLastError();
}

hipError_t launch_dequant_fp8(const uint8_t* q, const float* s, void* out, int out_bf16, int n, int k,
                              hipStream_t st) {
    const int64_t threads = ((int64_t)n * k) / 8;
    if (threads == 0) return hipSuccess;
    hipLaunchKernelGGL(dequant_fp8_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, q, s, out,
                       out_bf16, n, k);
    return hipGetLastError();
}

hipError_t launch_dequant_mx(const uint8_t* q, const uint8_t* ex, void* out, int out_bf16, int n, int k,
                             hipStream_t st) {
    const int64_t threads = (int64_t)n * k / 8;
    if (threads == 0) return hipSuccess;
    hipLaunchKernelGGL(dequant_mx_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, q, ex, out,
                       out_bf16, n, k);
    return hipGetLastError();
}

hipError_t launch_dequant_nf4(const uint8_t* q, const float* absmax, const Nf4Code& code, void* out, int out_bf16,
                              int n, int k, hipStream_t st) {
    const int64_t threads = ((int64_t)n * k) / 8;
    if (threads == 0) return hipSuccess;
    hipLaunchKernelGGL(dequant_nf4_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, q, absmax,
                       code, out, out_bf16, n, k);
    return hipGetLastError();
}

hipError_t launch_small_linear(const void* a, int a_bf16, int64_t a_rpb, int64_t a_bstride, int64_t a_off,
                               const uint16_t* w, const float* bias, void* out, int out_bf16, int64_t o_rpb,
                               int64_t o_bstride, int64_t o_off, int M, int N, int K, hipStream_t st) {
    if (M == 0) return hipSuccess;
    if (a_bf16 && !out_bf16 && K % 32 == 0) {
        hipLaunchKernelGGL(bf16_linear_f32_kernel, dim3((M + 31) / 32, (N + 127) / 128), dim3(256), 0, st,
                           (const uint16_t*)a, a_rpb, a_bstride, a_off, w, bias, (float*)out, o_rpb, o_bstride,
                           o_off, M, N, K);
        return hipGetLastError();
    }
    const dim3 grid((M + kSL - 1) / kSL, (N + kSL - 1) / kSL);
    if (a_bf16 && out_bf16)
        hipLaunchKernelGGL((small_linear_kernel<true, true>), grid, dim3(256), 0, st, a, a_rpb, a_bstride, a_off, w,
                           bias, out, o_rpb, o_bstride, o_off, M, N, K);
    else if (a_bf16)
        hipLaunchKernelGGL((small_linear_kernel<true, false>), grid, dim3(256), 0, st, a, a_rpb, a_bstride, a_off, w,
                           bias, out, o_rpb, o_bstride, o_off, M, N, K);
    else if (out_bf16)
        hipLaunchKernelGGL((small_linear_kernel<false, true>), grid, dim3(256), 0, st, a, a_rpb, a_bstride, a_off, w,
                           bias, out, o_rpb, o_bstride, o_off, M, N, K);
    else
        hipLaunchKernelGGL((small_linear_kernel<false, false>), grid, dim3(256), 0, st, a, a_rpb, a_bstride, a_off,
                           w, bias, out, o_rpb, o_bstride, o_off, M, N, K);
    return hipGetLastError();
}

hipError_t launch_copy_rows(const uint16_t* src, int64_t src_rpb, uint16_t* dst, int64_t dst_rpb, int B, int rows,
                            int cols, hipStream_t st) {
    if (rows == 0 || B == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_rows_kernel, dim3(rows, B), dim3(256), 0, st, src, src_rpb, dst, dst_rpb, rows, cols);
    return hipGetLastError();
}

}  // namespace sfm
