// FP8-E4M3 x FP8-E4M3 projection on gfx950 matrix cores with fused epilogues.
//
// y[m][n] = (sum_k dec(A[m][k]) * dec(W[n][k])) * sa[m] * sw[n]
//   A: per-token E4M3 codes of a bf16 activation (sa = amax/448 per row),
//   W: E4M3 weight codes with a per-output-channel fp32 scale (the released
//      checkpoint is FP8 E4M3: deployment post, section 2).
// Epilogues (research note, block internals): plain bf16 store (QKV), gated
// residual x + gate * y (attention output and MLP down projections), SwiGLU
// silu(gate) * up with the gate and up rows of one output column computed by
// the same lane.
//
// Structure: one workgroup computes a BM x BN tile with WM x WN waves; K is
// walked in steps of 128 bytes.  Operand tiles are staged global -> registers
// -> LDS (double buffered, one barrier per step), stored K-contiguous with the
// 16-byte chunks XOR-swizzled by (row & 7) so that the MFMA operand reads of 16
// consecutive rows hit distinct bank groups.  Each wave issues
// v_mfma_f32_16x16x128_f8f6f4 on 16x16 sub-tiles: A operand = 16 token rows x
// 128 k, B operand = 16 weight rows x 128 k; lane l holds rows (l & 15) and the
// 32-byte k-slice (l >> 4) of both, so the product is independent of how the
// instruction orders k inside a lane.  Output lane l holds rows 4*(l>>4)+r,
// column l & 15.
#include "gemm_common.h"

namespace sfm {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 4); }

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void gemm_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, uint16_t* out, const uint16_t* resid, const float* __restrict__ gate,
    int64_t gate_stride, int M, int N, int K, int L, int ntn) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int ACH = BM * (kBK / 16) / NT;  // 16-byte chunks per thread per step
    constexpr int BCH = BN * (kBK / 16) / NT;
    static_assert(ACH * NT == BM * 8 && BCH * NT == BN * 8, "tile / thread mismatch");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    // buffer b: A tile at smem + b*(BM+BN)*kBK, B tile right after it
    auto lds_a = [&](int buf) { return smem + buf * (BM + BN) * kBK; };
    auto lds_b = [&](int buf) { return smem + buf * (BM + BN) * kBK + BM * kBK; };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    const int bid = xcd_tile_id();
    const int tm = bid / ntn, tn = bid % ntn;
    const int m0 = tm * BM;

    // global source pointers of this thread's chunks
    const uint8_t* a_src[ACH];
    int a_dst[ACH];
#pragma unroll
    for (int c = 0; c < ACH; ++c) {
        const int i = tid + c * NT;
        const int row = i >> 3, ch = i & 7;
        const int gm = min(m0 + row, M - 1);
        a_src[c] = A + (int64_t)gm * K + ch * 16;
        a_dst[c] = swz(row, ch);
    }
    const uint8_t* b_src[BCH];
    int b_dst[BCH];
#pragma unroll
    for (int c = 0; c < BCH; ++c) {
        const int i = tid + c * NT;
        const int row = i >> 3, ch = i & 7;
        b_src[c] = W + weight_row<EPI, BN, TN>(row, tn, N) * K + ch * 16;
        b_dst[c] = swz(row, ch);
    }

    u32x4 ra[ACH], rb[BCH];
    auto gload = [&](int k0) {
#pragma unroll
        for (int c = 0; c < ACH; ++c) ra[c] = *reinterpret_cast<const u32x4*>(a_src[c] + k0);
#pragma unroll
        for (int c = 0; c < BCH; ++c) rb[c] = *reinterpret_cast<const u32x4*>(b_src[c] + k0);
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int c = 0; c < ACH; ++c) *reinterpret_cast<u32x4*>(lds_a(buf) + a_dst[c]) = ra[c];
#pragma unroll
        for (int c = 0; c < BCH; ++c) *reinterpret_cast<u32x4*>(lds_b(buf) + b_dst[c]) = rb[c];
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int lr = lane & 15, lg = lane >> 4;
    const int nk = K / kBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * kBK);
        const uint8_t* la = lds_a(buf);
        const uint8_t* lb = lds_b(buf);
        v8i bf[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = wn * TN + j * 16 + lr;
            const u32x4 x0 = *reinterpret_cast<const u32x4*>(lb + swz(row, 2 * lg));
            const u32x4 x1 = *reinterpret_cast<const u32x4*>(lb + swz(row, 2 * lg + 1));
            bf[j] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * TM + i * 16 + lr;
            const u32x4 x0 = *reinterpret_cast<const u32x4*>(la + swz(row, 2 * lg));
            const u32x4 x1 = *reinterpret_cast<const u32x4*>(la + swz(row, 2 * lg + 1));
            const v8i af = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 0, 0, 0, 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    gemm_epilogue<EPI, BN, TN, FM, FN>(
        acc, m0 + wm * TM, wn, tn, lane, M, N, L, out, resid, gate, gate_stride,
        [&](int row) { return sa[row]; }, [&](int64_t col) { return sw[col]; });
}

template <int BM, int BN, int WM, int WN, int EPI>
hipError_t launch_cfg(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* out,
                      const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N, int K, int L,
                      hipStream_t st) {
    const int ntm = (M + BM - 1) / BM;
    const int ntn = N / BN;
    const size_t shm = 2 * (BM + BN) * kBK;
    auto kern = gemm_fp8_kernel<BM, BN, WM, WN, EPI>;
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(ntm * ntn), dim3(WM * WN * 64), shm, st, a, sa, w, sw, out, resid, gate,
                       gate_stride, M, N, K, L, ntn);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8(int epi, const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                           uint16_t* out, const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N,
                           int K, int L, hipStream_t st) {
    if (M == 0) return hipSuccess;
    switch (epi) {
        case SFM_EPI_STORE:
            return launch_cfg<128, 128, 2, 2, SFM_EPI_STORE>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K, L,
                                                             st);
        case SFM_EPI_RESID_GATE:
            return launch_cfg<128, 128, 2, 2, SFM_EPI_RESID_GATE>(a, sa, w, sw, out, resid, gate, gate_stride, M, N,
                                                                  K, L, st);
        case SFM_EPI_SWIGLU:
            return launch_cfg<128, 128, 2, 2, SFM_EPI_SWIGLU>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K,
                                                              L, st);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace sfm
