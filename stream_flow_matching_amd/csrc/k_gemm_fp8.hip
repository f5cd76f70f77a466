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
// Structure: one workgroup of four waves (2 x 2) computes a BM x BN tile.  K
// is walked in stages of 128 bytes held in a two-stage LDS ring; operand tiles
// go global -> LDS with buffer_load ... lds (no staging registers).  Each stage
// is two halves of 64 k, one v_mfma_f32_32x32x64_f8f6f4 deep, and the
// fragments of a half are read from LDS while the matrix cores work on the
// previous half (two register sets), so the MFMA stream does not wait on LDS.
// Two barriers per stage: one after the waves have read the stage's last half,
// which frees the stage for the loads two stages ahead, and one before the
// next stage is read.  The 1 KiB wave-loads are interleaved one by one with the
// MFMAs of the three quarter-stages after the first barrier, which keeps the
// four waves' loads below the rate the CU's load path accepts.  Every
// wave-load covers 8 rows of 128 bytes; its source offsets apply the XOR
// swizzle 16-byte chunk ^ ((row >> 1) & 7), which puts the 16 rows that one
// quarter of a ds_read_b128 touches into 16 distinct 16-byte slots of the 64
// LDS banks.  Rows past M are clamped to row M - 1 for loading (their results
// are never stored).  MFMA operands: lane l holds row (l & 31) and the same
// 32-byte k-slice (l >> 5) of A and W, so the product does not depend on how
// the instruction orders k inside a lane.  The weight fragment is the first
// operand, so each accumulator block is transposed: a lane owns four
// consecutive output columns of one row, which the epilogue scales and stages
// through LDS in 8- or 16-byte pieces.  The row and column scales (and the gate
// rows of the gated residual) are loaded into LDS behind the ring at the start,
// under the first stages' loads.  Tiles are numbered XCD by XCD and, in each
// XCD's range, in 8-row groups (L2 reuse of both operands).
#include <algorithm>

#include "epi_qkv_rope.h"

namespace sfm {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define SFM_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kBK = 128;  // k bytes per stage
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kGroupM = 8;
// epilogue of a split-K part: the raw fp32 sums of its k range (no scales), reduced by
// splitk_reduce_kernel
constexpr int kEpiPartial = 3;

// s_waitcnt with vmcnt <= VM and lgkmcnt == 0 (expcnt not waited on)
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}

// Workgroup barrier for LDS that has already been waited for (wait_vm_lgkm0):
// the empty asm statements keep the compiler from moving LDS accesses across
// it, and no fence is used because a fence would also drain the loads still
// in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One 1 KiB wave-load: lane l copies 16 bytes from byte voff + soff of the
// buffer to LDS bytes lds + 16 l .. lds + 16 l + 15.  (A free function: the
// address-space cast inside a lambda of a kernel template loses the kernel's
// host-side stub.)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, SFM_LDS(lds), 16, voff, soff, 0, 0);
}

// LDS of one configuration: the two-stage ring (also the epilogue's staging, a quarter per
// wave), then the epilogue's scales.  WF 0: FP8 weights (128 bytes per row and stage); WF 1:
// MXFP4 weights (64 bytes per row and stage).
template <int BM, int BN, int EPI, int WF>
struct GemmLds {
    static constexpr int TM = BM / 2, TN = BN / 2;
    static constexpr int WROW = WF ? kBK / 2 : kBK;
    static constexpr int STAGE = BM * kBK + BN * WROW;
    static constexpr int EPI_BYTES = EPI == SFM_EPI_RESID_GATE ? TM / 2 * (TN * 4 + ((TN / 4) % 16 ? 16 : 0))
                                     : EPI == kEpiPartial      ? 0
                                                               : TM * (EPI == SFM_EPI_SWIGLU ? TN / 2 : TN) * 2;
    static constexpr int RING = 2 * STAGE > 4 * EPI_BYTES ? 2 * STAGE : 4 * EPI_BYTES;
    static constexpr size_t BYTES = (size_t)RING + (size_t)(BM + 4 * BN) * 4;
};

template <int BM, int BN, int EPI, int WF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, const uint8_t* __restrict__ wexp, uint16_t* out, const uint16_t* resid,
    const float* __restrict__ gate, int64_t gate_stride, int M, int N, int K, int L, int ntm, int ntn, int kps,
    float* __restrict__ part, RopeArgs rope) {
    constexpr bool MX = WF == 1;
    using Lds = GemmLds<BM, BN, EPI, WF>;
    constexpr int TM = BM / 2, TN = BN / 2;    // wave tile
    constexpr int FM = TM / 32, FN = TN / 32;  // 32 x 32 MFMA tiles per wave
    // 1 KiB wave-loads per stage per wave: A 8 rows x 128 bytes each; W the same for FP8, 16
    // rows x 64 bytes for MXFP4
    constexpr int AI = BM / 32, BI = MX ? BN / 64 : BN / 32;
    constexpr int NV = AI + BI;                // vector-memory ops per stage per wave
    constexpr int NF = FM + FN;                // fragments per half-stage
    constexpr int NQ = (FM / 2) * FN;          // MFMAs per quarter-stage
    constexpr int STAGE = Lds::STAGE, WROW = Lds::WROW;
    static_assert(FM % 2 == 0, "quarter-stages split the row tiles in two");
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    // split-K (kps > 0): workgroup id = split * tiles + tile; split s walks k blocks of 256
    // [s kps, (s + 1) kps), else the whole K
    int tile = xcd_tile_id(), kbeg = 0, klen = K;
    const int split = kps > 0 ? tile / (ntm * ntn) : 0;
    if (kps > 0) {
        tile -= split * ntm * ntn;
        kbeg = split * kps * 256;
        klen = min(K - kbeg, kps * 256);
    }
    grouped_tile(tile, ntm, ntn, kGroupM, tm, tn);
    // the divisions above run on the vector ALU; naming the results wave-uniform keeps the
    // buffer descriptors and the loop bounds in scalar registers (a descriptor left in vector
    // registers turns every direct load of the loop into a per-lane waterfall)
    tm = __builtin_amdgcn_readfirstlane(tm);
    tn = __builtin_amdgcn_readfirstlane(tn);
    kbeg = __builtin_amdgcn_readfirstlane(kbeg);
    klen = __builtin_amdgcn_readfirstlane(klen);
    const int m0 = tm * BM;

    // wave-load v of this wave covers tile rows 8 (wave + 4 v) + (lane >> 3); the lane writes
    // physical chunk lane & 7, which holds logical chunk (lane & 7) ^ ((row >> 1) & 7), and
    // (row >> 1) & 7 == (4 (wave & 1) + (lane >> 4)) & 7 for every v
    // The activation view starts at the tile's first row (64-bit base), so the 32-bit offsets
    // stay below BM * K bytes whatever M * K is; the weight view (N * K < 2^31 bytes, checked
    // by the host) starts at W.
    const uint8_t* const A0 = A + (int64_t)m0 * K;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)A0, 0, 0x7FFFFFFF, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)W, 0, 0x7FFFFFFF, kRsrcWord3);
    // zero-length views: loads through them touch no memory (the tail stages)
    const __amdgpu_buffer_rsrc_t ra0 = __builtin_amdgcn_make_buffer_rsrc((void*)A0, 0, 0, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb0 = __builtin_amdgcn_make_buffer_rsrc((void*)W, 0, 0, kRsrcWord3);
    const int lrow = lane >> 3, lch = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
    uint32_t voff[NV];
#pragma unroll
    for (int v = 0; v < AI; ++v) {
        const int row = min(m0 + 8 * (wave + 4 * v) + lrow, M - 1);
        voff[v] = (uint32_t)(row - m0) * (uint32_t)K + lch * 16;
    }
#pragma unroll
    for (int v = 0; v < BI; ++v) {
        if constexpr (MX) {
            // 16 rows of 64 bytes: lane l row 16 (wave + 4 v) + (l >> 2), physical chunk l & 3 =
            // logical chunk ^ ((row >> 2) & 3) = logical ^ ((l >> 4) & 3)
            const int64_t wr = weight_row<EPI, BN, TN>(16 * (wave + 4 * v) + (lane >> 2), tn, N);
            voff[AI + v] = (uint32_t)wr * (uint32_t)(K / 2) + (((lane & 3) ^ ((lane >> 4) & 3)) * 16);
        } else {
            const int64_t wr = weight_row<EPI, BN, TN>(8 * (wave + 4 * v) + lrow, tn, N);
            voff[AI + v] = (uint32_t)wr * (uint32_t)K + lch * 16;
        }
    }
    // LDS destination of wave-load v inside a stage (uniform per wave)
    auto vmem = [&](int v, uint8_t* stg, __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB, int k0) {
        if (v < AI)
            dma16(rA, stg + wave * 1024 + v * 4096, voff[v], k0);
        else
            dma16(rB, stg + BM * kBK + wave * 1024 + (v - AI) * 4096, voff[v], MX ? k0 / 2 : k0);
    };

    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

    // fragment rows have (row >> 1) & 7 == (lr >> 1) & 7: chunk offsets are per-lane constants;
    // half h of a 128-byte row holds logical chunks 4h .. 4h + 3
    const int lr = lane & 31, lg = lane >> 5, sx = (lr >> 1) & 7;
    // MXFP4: the FP4 operand's lane (row, half g) holds 16 values at k 16 g + t and 16 at
    // 32 + 16 g + t (t < 16), and its E8M0 scale covers all 32.  Numbering the k of each 64-k half
    // so that a W lane holds the 32 consecutive k of one MX block, lane g of W reads logical
    // chunk 2 h + g of its 64-byte row and the FP8 activation lane g reads chunks g and 2 + g of
    // the half (instead of 2 g and 2 g + 1)
    const int cc[2][2] = {{((MX ? lg : 2 * lg) ^ sx) << 4, ((MX ? 2 + lg : 2 * lg + 1) ^ sx) << 4},
                          {((MX ? 4 + lg : 4 + 2 * lg) ^ sx) << 4, ((MX ? 6 + lg : 4 + 2 * lg + 1) ^ sx) << 4}};
    const int cw[2] = {((0 + lg) ^ ((lr >> 2) & 3)) << 4, ((2 + lg) ^ ((lr >> 2) & 3)) << 4};
    const int arow = (wm * TM + lr) * kBK, brow = BM * kBK + (wn * TN + lr) * WROW;

    // fragment f of a half: f < FN is weight column tile f, else row tile f - FN
    v8i fr[2][NF];
    auto ds = [&](int set, int f, const uint8_t* stg, int h) {
        if (MX && f < FN) {
            const u32x4 x0 = *reinterpret_cast<const u32x4*>(stg + brow + f * 32 * WROW + cw[h]);
            fr[set][f] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, 0, 0, 0, 0};
            return;
        }
        const uint8_t* p = stg + (f < FN ? brow + f * 32 * kBK : arow + (f - FN) * 32 * kBK);
        const u32x4 x0 = *reinterpret_cast<const u32x4*>(p + cc[h][0]);
        const u32x4 x1 = *reinterpret_cast<const u32x4*>(p + cc[h][1]);
        fr[set][f] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    };
    // MXFP4 block exponents of the stage: one 32-bit word (the stage's four blocks) per W fragment
    // row; lane g of half h uses byte 2 h + g.  Loaded one stage ahead.
    uint32_t eoff[FN], su[FN], sn[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        eoff[j] = MX ? (uint32_t)weight_row<EPI, BN, TN>(wn * TN + 32 * j + lr, tn, N) * (uint32_t)(K / 32) +
                           (uint32_t)(kbeg / 32)
                     : 0u;
        su[j] = sn[j] = 0u;
    }
    auto load_exp = [&](uint32_t (&dst)[FN], int t) {
#pragma unroll
        for (int j = 0; j < FN; ++j) dst[j] = *reinterpret_cast<const uint32_t*>(wexp + eoff[j] + 4 * t);
    };
    auto mfma = [&](int set, int q, int i0) {
        const int i = i0 + q / FN, j = q % FN;
        if constexpr (MX)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr[set][j], fr[set][FN + i], acc[i][j], 4, 0, 0,
                                                                        (int)(su[j] >> (16 * set + 8 * lg)), 0, 127);
        else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr[set][j], fr[set][FN + i], acc[i][j], 0, 0, 0,
                                                                        0, 0, 0);
    };
    // quarter-stage: NQ MFMAs on fragment set `set`, row tiles i0 .. i0 + FM/2, with the
    // fragment reads for set `rset` from half rh of rstg (if RD) and wave-loads v0 .. v1 into
    // lstg spread over them
    auto quarter = [&](int set, int i0, bool RD, int rset, const uint8_t* rstg, int rh, int v0, int v1,
                       uint8_t* lstg, __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB, int k0) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            mfma(set, q, i0);
#pragma unroll
            for (int v = v0 + q * (v1 - v0) / NQ; v < v0 + (q + 1) * (v1 - v0) / NQ; ++v) vmem(v, lstg, rA, rB, k0);
            if (RD)
#pragma unroll
                for (int f = q * NF / NQ; f < (q + 1) * NF / NQ; ++f) ds(rset, f, rstg, rh);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // the epilogue's scales go to LDS behind the ring: row scales [BM], column scales [BN] and,
    // for the gated residual, gate * column scale for the (at most three) batches the tile's rows
    // touch [3][BN]; their loads are issued before the first stages' and land under them
    constexpr int NSC = BM + (EPI == SFM_EPI_RESID_GATE ? 4 : 1) * BN;
    constexpr int NSL = (NSC + 255) / 256;
    float* scl = reinterpret_cast<float*>(smem + Lds::RING);
    const int bt0 = EPI == SFM_EPI_RESID_GATE ? min(m0, M - 1) / L : 0;
    float scv[NSL];
#pragma unroll
    for (int k = 0; k < NSL; ++k) {
        const int e = tid + 256 * k;
        float v = 1.0f;
        if (e < BM) {
            if (sa) v = sa[min(m0 + e, M - 1)];
        } else if (e < BM + BN) {
            if (sw) v = sw[weight_row<EPI, BN, TN>(e - BM, tn, N)];
        } else if (e < NSC) {
            const int g = (e - BM - BN) / BN, c = (e - BM - BN) % BN;
            v = gate[(int64_t)min(bt0 + g, (M - 1) / L) * gate_stride + (int64_t)tn * BN + c];
            if (sw) v *= sw[weight_row<EPI, BN, TN>(c, tn, N)];
        }
        scv[k] = v;
    }

    uint32_t qk_gamma = 0u;
    if constexpr (EPI == kEpiQkvRope) qk_gamma = load_qk_gamma(rope, tn, tid);

    // K % 256 == 0 (checked by the caller) and klen a multiple of 256: nks >= 2 and even
    const int nks = klen / kBK;
    if constexpr (MX) load_exp(su, 0);
#pragma unroll
    for (int v = 0; v < NV; ++v) vmem(v, smem, ra, rb, kbeg);
#pragma unroll
    for (int v = 0; v < NV; ++v) vmem(v, smem + STAGE, ra, rb, kbeg + kBK);
    // the partial-sum pointer is only read by the epilogue: take it here, under the wait below,
    // so that no scalar load is in flight when the loop starts (with one pending, the loop head
    // would have to wait for every LDS read, as scalar loads return out of order)
    if constexpr (EPI == kEpiPartial) asm volatile("" ::"s"(part));
    wait_vm_lgkm0<NV>();
#pragma unroll
    for (int k = 0; k < NSL; ++k)
        if (tid + 256 * k < NSC) scl[tid + 256 * k] = scv[k];
    // the QK-norm gamma of the tile's part behind the row-sum exchange area of the epilogue
    if constexpr (EPI == kEpiQkvRope)
        if (tid < 128) reinterpret_cast<uint32_t*>(scl + BM + BN + 4 * TM)[tid] = qk_gamma;
    lds_barrier();
    // in program order, as the loop reads them: the loop head then waits only for the first
    // fragments (issued in another order, the first MFMA would need the last read and the
    // compiler would wait for all of them at the head of every stage)
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        ds(0, f, smem, 0);
        __builtin_amdgcn_sched_barrier(0);
    }

    // stage t: set 0 holds half 0 of stage t on entry and half 0 of stage t + 1 on exit.
    // Barrier A (after the reads of half 1) frees stage t's buffer for the loads of stage
    // t + 2, which are spread over the last three quarters; barrier B (before the reads of
    // stage t + 1) follows the wait for this wave's loads of stage t + 1 (everything but the
    // V1 loads of stage t + 2 issued since).
    constexpr int V1 = (NV + 2) / 3, V2 = (2 * NV + 2) / 3;
    for (int t = 0; t < nks; ++t) {
        uint8_t* cur = smem + (t & 1) * STAGE;
        const uint8_t* nxt = smem + ((t + 1) & 1) * STAGE;
        const bool more = t + 2 < nks;
        const __amdgpu_buffer_rsrc_t rA = more ? ra : ra0;
        const __amdgpu_buffer_rsrc_t rB = more ? rb : rb0;
        const int k2 = kbeg + (t + 2) * kBK;
        // the next stage's block exponents go out before this stage's loads (the waits below
        // then cover them); the last stage re-reads its own word, which keeps the loop free of a
        // branch (a conditional block at the loop head makes the compiler wait for every LDS read
        // before the first MFMA)
        if constexpr (MX) load_exp(sn, min(t + 1, nks - 1));
        quarter(0, 0, true, 1, cur, 1, 0, 0, cur, rA, rB, k2);
        wait_vm_lgkm0<63>();
        lds_barrier();
        quarter(0, FM / 2, false, 1, cur, 1, 0, V1, cur, rA, rB, k2);
        quarter(1, 0, false, 0, cur, 0, V1, V2, cur, rA, rB, k2);
        wait_vm_lgkm0<V2>();
        lds_barrier();
        quarter(1, FM / 2, true, 0, nxt, 0, V2, NV, cur, rA, rB, k2);
        if constexpr (MX)
#pragma unroll
            for (int j = 0; j < FN; ++j) su[j] = sn[j];
    }
    wait_vm_lgkm0<0>();

    // the ring is free once every wave is past its last read: each wave then stages its
    // epilogue in its own quarter of the LDS
    lds_barrier();
    if constexpr (EPI == kEpiPartial) {
        // lane: row 32 i + (l & 31) of the wave tile, columns 32 j + 8 q + 4 (l >> 5) .. + 3
        const int lc = lane & 31, lg = lane >> 5;
        float* pbase = part + (size_t)split * M * N + (int64_t)tn * BN + wn * TN;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = m0 + wm * TM + 32 * i + lc;
            if (row < M)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<v4f*>(pbase + (int64_t)row * N + 32 * j + 8 * q + 4 * lg) =
                            v4f{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        }
    } else if constexpr (EPI == kEpiQkvRope) {
        // the gate area behind the scales (unused by this epilogue) takes the row sums of squares
        epilogue_qkv_rope<FM, FN>(acc, smem + wave * (Lds::RING / 4), scl + BM + BN, m0 + wm * TM, wm, wn, tn, lane, M,
                                  L, scl + wm * TM, scl + BM + wn * TN,
                                  reinterpret_cast<const uint32_t*>(scl + BM + BN + 4 * TM), rope);
    } else {
        gemm_epilogue_lds<EPI, BN, TN, FM, FN>(acc, smem + wave * (Lds::RING / 4), m0 + wm * TM, wn, tn, lane, M, N, L,
                                               out, resid, scl + wm * TM, scl + BM + wn * TN, scl + BM + BN + wn * TN,
                                               bt0);
    }
}

// out[m][n] = bf16((sum over the S parts of part[s][m][n]) * sa[m] * sw[n]); eight outputs per thread
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int S, int M, int N,
                                                            const float* __restrict__ sa,
                                                            const float* __restrict__ sw, uint16_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int n8 = N / 8;
    if (i >= (int64_t)M * n8) return;
    const int64_t m = i / n8;
    const int n = (int)(i % n8) * 8;
    v4f a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) {
        const float* p = part + ((size_t)s * M + m) * N + n;
        a += *reinterpret_cast<const v4f*>(p);
        b += *reinterpret_cast<const v4f*>(p + 4);
    }
    const float r = sa ? sa[m] : 1.0f;
    const v4f c0 = sw ? *reinterpret_cast<const v4f*>(sw + n) : v4f{1.f, 1.f, 1.f, 1.f};
    const v4f c1 = sw ? *reinterpret_cast<const v4f*>(sw + n + 4) : v4f{1.f, 1.f, 1.f, 1.f};
    uint4 o;
    o.x = cvt_bf16x2(a[0] * r * c0[0], a[1] * r * c0[1]);
    o.y = cvt_bf16x2(a[2] * r * c0[2], a[3] * r * c0[3]);
    o.z = cvt_bf16x2(b[0] * r * c1[0], b[1] * r * c1[1]);
    o.w = cvt_bf16x2(b[2] * r * c1[2], b[3] * r * c1[3]);
    *reinterpret_cast<uint4*>(out + m * N + n) = o;
}

template <int BM, int BN, int EPI, int WF = 0>
hipError_t launch_cfg(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* out,
                      const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N, int K, int L,
                      hipStream_t st, int splits = 1, int kps = 0, float* part = nullptr,
                      const uint8_t* wexp = nullptr, const RopeArgs& rope = RopeArgs{}) {
    const int ntm = (M + BM - 1) / BM;
    const int ntn = N / BN;
    // two ring stages, then the epilogue's scales (row, column and three gate rows)
    const size_t shm = GemmLds<BM, BN, EPI, WF>::BYTES;
    auto kern = gemm_fp8_kernel<BM, BN, EPI, WF>;
    static std::atomic<uint64_t> lds_raised{0};
    raise_lds_limit_once((const void*)kern, shm, lds_raised);
    hipLaunchKernelGGL(kern, dim3(ntm * ntn * splits), dim3(256), shm, st, a, sa, w, sw, wexp, out, resid, gate,
                       gate_stride, M, N, K, L, ntm, ntn, kps, part, rope);
    return hipGetLastError();
}

// Rounds of workgroups over the 256 compute units times the work of one tile,
// divided by the main loop's measured efficiency at that tile shape.  With
// `shared` (another pass's kernels fill the last round) the tiles count one by
// one instead of in whole rounds.
inline double tile_cost(int M, int N, int BM, int BN, double eff, bool shared) {
    const int64_t tiles = (int64_t)((M + BM - 1) / BM) * (N / BN);
    return (double)(shared ? tiles : (tiles + 255) / 256 * 256) * BM * BN / eff;
}

template <int EPI, int WF = 0>
hipError_t launch_epi(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* out,
                      const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N, int K, int L,
                      hipStream_t st, const uint8_t* wexp = nullptr, bool shared = false) {
    // the cheapest of the tile shapes that divide N (256 x 192 for the gated residual only)
    double best = 1e300;
    int cfg = 3;
    const double c256 = N % 256 == 0 ? tile_cost(M, N, 256, 256, 0.93, shared) : 1e300;
    const double c192 =
        EPI == SFM_EPI_RESID_GATE && N % 192 == 0 ? tile_cost(M, N, 256, 192, 0.92, shared) : 1e300;
    const double c128 = tile_cost(M, N, 256, 128, 0.81, shared);
    const double c64 = tile_cost(M, N, 128, 128, 0.70, shared);
    if (c256 < best) best = c256, cfg = 0;
    if (c192 < best) best = c192, cfg = 1;
    if (c128 < best) best = c128, cfg = 2;
    if (c64 < best) best = c64, cfg = 3;
    switch (cfg) {
        case 0: return launch_cfg<256, 256, EPI, WF>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K, L, st, 1, 0,
                                                  nullptr, wexp);
        case 1:
            if constexpr (EPI == SFM_EPI_RESID_GATE)
                return launch_cfg<256, 192, EPI, WF>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K, L, st, 1, 0,
                                                  nullptr, wexp);
            return hipErrorInvalidValue;
        case 2: return launch_cfg<256, 128, EPI, WF>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K, L, st, 1, 0,
                                                  nullptr, wexp);
        default: return launch_cfg<128, 128, EPI, WF>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K, L, st, 1, 0,
                                                  nullptr, wexp);
    }
}

}  // namespace

int splitk_parts(int M, int N, int K) {
    const int tiles = ((M + 255) / 256) * (N % 256 == 0 ? N / 256 : N / 128);
    const int kb = K / 256;
    if (tiles >= 128 || kb < 8) return 1;
    const int want = std::min(8, std::max(1, 256 / tiles));
    const int kps = (kb + want - 1) / want;
    return (kb + kps - 1) / kps;
}

hipError_t launch_gemm_fp8_splitk(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* out,
                                  int M, int N, int K, float* part, hipStream_t st) {
    if (M == 0) return hipSuccess;
    const int S = splitk_parts(M, N, K);
    const int kb = K / 256, kps = (kb + S - 1) / S;
    hipError_t e = N % 256 == 0
                       ? launch_cfg<256, 256, kEpiPartial>(a, sa, w, sw, out, nullptr, nullptr, 0, M, N, K, M, st, S,
                                                           kps, part)
                       : launch_cfg<256, 128, kEpiPartial>(a, sa, w, sw, out, nullptr, nullptr, 0, M, N, K, M, st, S,
                                                           kps, part);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)M * (N / 8);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, S, M, N, sa,
                       sw, out);
    return hipGetLastError();
}

hipError_t launch_gemm_fp8(int epi, const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                           uint16_t* out, const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N,
                           int K, int L, hipStream_t st, bool shared) {
    if (M == 0) return hipSuccess;
    switch (epi) {
        case SFM_EPI_STORE:
            return launch_epi<SFM_EPI_STORE>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K, L, st, nullptr, shared);
        case SFM_EPI_RESID_GATE:
            return launch_epi<SFM_EPI_RESID_GATE>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K, L, st, nullptr, shared);
        case SFM_EPI_SWIGLU:
            return launch_epi<SFM_EPI_SWIGLU>(a, sa, w, sw, out, resid, gate, gate_stride, M, N, K, L, st, nullptr, shared);
        default:
            return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_fp8_qkv_rope(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, int M,
                                   int K, int L, const RopeArgs& ra, hipStream_t st) {
    if (M == 0) return hipSuccess;
    return launch_cfg<256, 256, kEpiQkvRope>(a, sa, w, sw, nullptr, nullptr, nullptr, 0, M, 3 * ra.H * 256, K, L, st, 1,
                                             0, nullptr, nullptr, ra);
}

hipError_t launch_gemm_mx(int epi, const uint8_t* a, const float* sa, const uint8_t* w, const uint8_t* wexp,
                          uint16_t* out, const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N,
                          int K, int L, hipStream_t st, bool shared) {
    if (M == 0) return hipSuccess;
    switch (epi) {
        case SFM_EPI_STORE:
            return launch_epi<SFM_EPI_STORE, 1>(a, sa, w, nullptr, out, resid, gate, gate_stride, M, N, K, L, st,
                                                wexp, shared);
        case SFM_EPI_RESID_GATE:
            return launch_epi<SFM_EPI_RESID_GATE, 1>(a, sa, w, nullptr, out, resid, gate, gate_stride, M, N, K, L, st,
                                                     wexp, shared);
        case SFM_EPI_SWIGLU:
            return launch_epi<SFM_EPI_SWIGLU, 1>(a, sa, w, nullptr, out, resid, gate, gate_stride, M, N, K, L, st,
                                                 wexp, shared);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace sfm
