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
// Structure: one workgroup of four waves (2 x 2) computes a BM x BN tile; K is
// walked in steps of 128 bytes.  Both operand tiles go global -> LDS with
// buffer_load ... lds (no staging registers), two stages, one barrier per
// step; every 1 KiB wave-load covers 8 rows of 128 bytes and applies the XOR
// swizzle (16-byte chunk ^ ((row >> 1) & 7)) through its source offsets: the
// LDS serves 256 bytes (64 banks) per clock, two 128-byte rows per bank line,
// and the swizzle puts the 16 rows that one MFMA operand read touches into 16
// distinct 16-byte bank slots.  Rows past
// M are clamped to row M - 1 for loading (their results are never stored).
// Each wave issues v_mfma_f32_16x16x128_f8f6f4 on 16x16 sub-tiles: A operand
// = 16 token rows x 128 k, B operand = 16 weight rows x 128 k; lane l holds
// rows (l & 15) and the 32-byte k-slice (l >> 4) of both, so the product is
// independent of how the instruction orders k inside a lane.  Output lane l
// holds rows 4*(l>>4)+r, column l & 15.  Tiles are numbered XCD by XCD and, in
// each XCD's range, in 8-row groups (L2 reuse of both operands).
#include "gemm_common.h"

namespace sfm {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define SFM_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kBK = 128;
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kGroupM = 8;

// Direct global -> LDS loads of one pipeline stage: AI wave-loads of the A
// tile and BI of the weight tile, 1 KiB each (lane l writes bytes 16 l .. 16 l + 15).
template <int AI, int BI>
struct StageLoader {
    __amdgpu_buffer_rsrc_t ra, rb;
    const uint32_t* aoff;
    const uint32_t* boff;
    uint32_t lds0;   // this wave's first 1 KiB block
    uint32_t bbase;  // byte offset of the weight tile inside a stage

    __device__ __forceinline__ void issue(uint8_t* stage, int k0) const {
#pragma unroll
        for (int i = 0; i < AI; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, SFM_LDS(stage + lds0 + i * 4096), 16, aoff[i], k0, 0, 0);
#pragma unroll
        for (int i = 0; i < BI; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, SFM_LDS(stage + bbase + lds0 + i * 4096), 16, boff[i], k0, 0,
                                                     0);
    }
};

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, uint16_t* out, const uint16_t* resid, const float* __restrict__ gate,
    int64_t gate_stride, int M, int N, int K, int L, int ntm, int ntn) {
    constexpr int TM = BM / 2, TN = BN / 2;    // wave tile
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int AI = BM / 32, BI = BN / 32;  // 1 KiB wave-loads per stage per wave
    constexpr int STAGE = (BM + BN) * kBK;
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    grouped_tile(xcd_tile_id(), ntm, ntn, kGroupM, tm, tn);
    const int m0 = tm * BM;

    // per-lane source offsets: wave-load i of this wave covers tile rows 8 (wave + 4 i) + (lane >> 3),
    // physical chunk lane & 7 holding logical chunk (lane & 7) ^ ((row >> 1) & 7), where
    // (row >> 1) & 7 = (4 (wave & 1) + (lane >> 4)) & 7 for every i
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, 0x7FFFFFFF, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)W, 0, 0x7FFFFFFF, kRsrcWord3);
    const int lrow = lane >> 3, lch = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
    uint32_t aoff[AI], boff[BI];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
        const int row = min(m0 + 8 * (wave + 4 * i) + lrow, M - 1);
        aoff[i] = (uint32_t)row * (uint32_t)K + lch * 16;
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
        const int64_t wr = weight_row<EPI, BN, TN>(8 * (wave + 4 * i) + lrow, tn, N);
        boff[i] = (uint32_t)wr * (uint32_t)K + lch * 16;
    }
    const StageLoader<AI, BI> ld{ra, rb, aoff, boff, (uint32_t)wave * 1024u, (uint32_t)(BM * kBK)};
    auto issue = [&](uint8_t* stage, int k0) { ld.issue(stage, k0); };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int lr = lane & 15, lg = lane >> 4;
    // fragment rows have (row >> 1) & 7 == (lr >> 1) & 7: chunk offsets are per-lane constants
    const int sx = (lr >> 1) & 7;
    const int c0 = ((2 * lg) ^ sx) << 4, c1 = ((2 * lg + 1) ^ sx) << 4;
    const int arow = (wm * TM + lr) * kBK, brow = BM * kBK + (wn * TN + lr) * kBK;

    auto compute = [&](const uint8_t* stg) {
        v8i bf[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const uint8_t* p = stg + brow + j * 16 * kBK;
            const u32x4 x0 = *reinterpret_cast<const u32x4*>(p + c0);
            const u32x4 x1 = *reinterpret_cast<const u32x4*>(p + c1);
            bf[j] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
        // A fragments one row-tile ahead; the scheduling barriers keep the
        // compiler from hoisting all of them (register pressure)
        v8i af[2];
        auto load_af = [&](int slot, int i) {
            const uint8_t* p = stg + arow + i * 16 * kBK;
            const u32x4 x0 = *reinterpret_cast<const u32x4*>(p + c0);
            const u32x4 x1 = *reinterpret_cast<const u32x4*>(p + c1);
            af[slot] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        };
        load_af(0, 0);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            if (i + 1 < FM) load_af((i + 1) & 1, i + 1);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] =
                    __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i & 1], bf[j], acc[i][j], 0, 0, 0, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    uint8_t* st0 = smem;
    uint8_t* st1 = smem + STAGE;
    // K % 256 == 0 (checked by the caller): an even number of 128-byte steps,
    // so the two-stage loop has a single exit
    const int nk = K / kBK;
    issue(st0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        issue(st1, (kt + 1) * kBK);
        compute(st0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 2 < nk) issue(st0, (kt + 2) * kBK);
        compute(st1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    gemm_epilogue<EPI, BN, TN, FM, FN>(
        acc, m0 + wm * TM, wn, tn, lane, M, N, L, out, resid, gate, gate_stride,
        [&](int row) { return sa[row]; }, [&](int64_t col) { return sw[col]; });
}

template <int BM, int BN, int EPI>
hipError_t launch_cfg(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* out,
                      const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N, int K, int L,
                      hipStream_t st) {
    const int ntm = (M + BM - 1) / BM;
    const int ntn = N / BN;
    const size_t shm = 2 * (BM + BN) * kBK;
    auto kern = gemm_fp8_kernel<BM, BN, EPI>;
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(ntm * ntn), dim3(256), shm, st, a, sa, w, sw, out, resid, gate, gate_stride, M, N, K,
                       L, ntm, ntn);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* out,
                      const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N, int K, int L,
                      hipStream_t st) {
    // 256 x 256 tiles when they give at least ~3 rounds of workgroups over the
    // 256 compute units, else 256 x 128, else 128 x 128
    const int64_t t256 = (int64_t)((M + 255) / 256) * (N / 256);
    const int64_t t128 = (int64_t)((M + 255) / 256) * (N / 128);
    if (N % 256 == 0 && t256 >= 700)
        return launch_cfg<256, 256, EPI>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K, L, st);
    if (t128 >= 400)
        return launch_cfg<256, 128, EPI>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K, L, st);
    return launch_cfg<128, 128, EPI>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K, L, st);
}

}  // namespace

hipError_t launch_gemm_fp8(int epi, const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                           uint16_t* out, const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N,
                           int K, int L, hipStream_t st) {
    if (M == 0) return hipSuccess;
    switch (epi) {
        case SFM_EPI_STORE:
            return launch_epi<SFM_EPI_STORE>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K, L, st);
        case SFM_EPI_RESID_GATE:
            return launch_epi<SFM_EPI_RESID_GATE>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K, L, st);
        case SFM_EPI_SWIGLU:
            return launch_epi<SFM_EPI_SWIGLU>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K, L, st);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace sfm
