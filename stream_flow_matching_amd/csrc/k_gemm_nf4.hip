// NF4-weight projection: the block-64 NF4 decode is fused into the weight
// operand load, the product runs on bf16 matrix cores (fp32 accumulation).
//
// Deployment post, section 2.1: NF4 (QLoRA NormalFloat-4), blocks of 64
// weights with one scale each.  Weight element w[n][k] =
// bf16(fp32(code[q[n][k]] * absmax[(n*K + k) / 64])); nibble 2i of a row is the
// high nibble of byte i.  The activation is bf16 (no input quantisation).
//
// Structure: BM x BN tile per workgroup, K walked in steps of 64 (one NF4
// block per weight row per step).  A (bf16) is staged global -> registers ->
// LDS; each thread decodes 32 weights (16 packed bytes + their block's absmax)
// into bf16 and writes them to LDS, with the 16-byte chunks XOR-swizzled by
// (row & 7).  v_mfma_f32_16x16x32_bf16: lane l holds rows (l & 15) and the
// 8-element k-slice (l >> 4) of both operands.
#include "gemm_common.h"

namespace sfm {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;          // k per step (elements)
constexpr int kRow = kBK * 2;    // bytes per LDS row (bf16)

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRow + ((chunk ^ (row & 7)) << 4); }

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void gemm_nf4_kernel(
    const uint16_t* __restrict__ A, const uint8_t* __restrict__ Wq, const float* __restrict__ absmax, Nf4Code code,
    uint16_t* out, const uint16_t* resid, const float* __restrict__ gate, int64_t gate_stride, int M, int N, int K,
    int L, int ntn) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int ACH = BM * 8 / NT;        // 16-byte A chunks per thread per step
    constexpr int BPT = BN * 2 / NT;        // 32-weight groups per thread per step
    static_assert(ACH * NT == BM * 8 && BPT * NT == BN * 2, "tile / thread mismatch");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ float lut[16];
    // buffer b: A tile at smem + b*(BM+BN)*kRow, B tile right after it
    auto lds_a = [&](int buf) { return smem + buf * (BM + BN) * kRow; };
    auto lds_b = [&](int buf) { return smem + buf * (BM + BN) * kRow + BM * kRow; };
    if (threadIdx.x < 16) lut[threadIdx.x] = code.v[threadIdx.x];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int bid = xcd_tile_id();
    const int tm = bid / ntn, tn = bid % ntn;
    const int m0 = tm * BM;
    const int kblocks = K / 64;

    const uint16_t* a_src[ACH];
    int a_dst[ACH];
#pragma unroll
    for (int c = 0; c < ACH; ++c) {
        const int i = tid + c * NT;
        const int row = i >> 3, ch = i & 7;
        a_src[c] = A + (int64_t)min(m0 + row, M - 1) * K + ch * 8;
        a_dst[c] = swz(row, ch);
    }
    const uint8_t* b_src[BPT];
    const float* b_am[BPT];
    int b_row[BPT], b_half[BPT];
#pragma unroll
    for (int c = 0; c < BPT; ++c) {
        const int i = tid + c * NT;
        const int row = i >> 1, half = i & 1;
        const int64_t wr = weight_row<EPI, BN, TN>(row, tn, N);
        b_src[c] = Wq + wr * (K / 2) + half * 16;
        b_am[c] = absmax + wr * kblocks;
        b_row[c] = row;
        b_half[c] = half;
    }

    u32x4 ra[ACH], rb[BPT];
    float rs[BPT];
    auto gload = [&](int kt) {
#pragma unroll
        for (int c = 0; c < ACH; ++c) ra[c] = *reinterpret_cast<const u32x4*>(a_src[c] + kt * kBK);
#pragma unroll
        for (int c = 0; c < BPT; ++c) {
            rb[c] = *reinterpret_cast<const u32x4*>(b_src[c] + kt * (kBK / 2));
            rs[c] = b_am[c][kt];
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int c = 0; c < ACH; ++c) *reinterpret_cast<u32x4*>(lds_a(buf) + a_dst[c]) = ra[c];
#pragma unroll
        for (int c = 0; c < BPT; ++c) {
            const uint32_t w[4] = {rb[c].x, rb[c].y, rb[c].z, rb[c].w};
            // 16 bytes = 32 nibbles = weights k0 + 32*half + [0, 32), 4 chunks of 8 bf16
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t byte = (w[q4] >> (8 * e)) & 0xFFu;
                    const float hi = lut[byte >> 4] * rs[c];   // element 2i: high nibble
                    const float lo = lut[byte & 15] * rs[c];   // element 2i+1: low nibble
                    o[e] = pack_bf16x2(hi, lo);
                }
                *reinterpret_cast<u32x4*>(lds_b(buf) + swz(b_row[c], b_half[c] * 4 + q4)) = u32x4{o[0], o[1], o[2], o[3]};
            }
        }
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int lr = lane & 15, lg = lane >> 4;
    const int nk = K / kBK;
    gload(0);
    __syncthreads();  // lut visible
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const uint8_t* la = lds_a(buf);
        const uint8_t* lb = lds_b(buf);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 bfr[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(lb + swz(wn * TN + j * 16 + lr, ks * 4 + lg)));
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const bf16x8 afr = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(la + swz(wm * TM + i * 16 + lr, ks * 4 + lg)));
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[j], acc[i][j], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    gemm_epilogue<EPI, BN, TN, FM, FN>(
        acc, m0 + wm * TM, wn, tn, lane, M, N, L, out, resid, gate, gate_stride, [](int) { return 1.0f; },
        [](int64_t) { return 1.0f; });
}

template <int BM, int BN, int WM, int WN, int EPI>
hipError_t launch_cfg(const uint16_t* a, const uint8_t* w, const float* am, const Nf4Code& code, uint16_t* out,
                      const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N, int K, int L,
                      hipStream_t st) {
    const int ntm = (M + BM - 1) / BM;
    const int ntn = N / BN;
    const size_t shm = 2 * (BM + BN) * kRow;
    auto kern = gemm_nf4_kernel<BM, BN, WM, WN, EPI>;
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(ntm * ntn), dim3(WM * WN * 64), shm, st, a, w, am, code, out, resid, gate,
                       gate_stride, M, N, K, L, ntn);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_nf4(int epi, const uint16_t* a, const uint8_t* w, const float* absmax, const Nf4Code& code,
                           uint16_t* out, const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N,
                           int K, int L, hipStream_t st) {
    if (M == 0) return hipSuccess;
    switch (epi) {
        case SFM_EPI_STORE:
            return launch_cfg<128, 128, 2, 2, SFM_EPI_STORE>(a, w, absmax, code, out, resid, gate, gate_stride, M, N,
                                                             K, L, st);
        case SFM_EPI_RESID_GATE:
            return launch_cfg<128, 128, 2, 2, SFM_EPI_RESID_GATE>(a, w, absmax, code, out, resid, gate, gate_stride,
                                                                  M, N, K, L, st);
        case SFM_EPI_SWIGLU:
            return launch_cfg<128, 128, 2, 2, SFM_EPI_SWIGLU>(a, w, absmax, code, out, resid, gate, gate_stride, M, N,
                                                              K, L, st);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace sfm
