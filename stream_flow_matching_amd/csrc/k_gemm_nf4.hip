// NF4-weight projection: the block-64 NF4 decode is fused into the weight
// operand load, the product runs on bf16 matrix cores (fp32 accumulation).
//
// Deployment post, section 2.1: NF4 (QLoRA NormalFloat-4), blocks of 64
// weights with one scale each.  Weight element w[n][k] =
// bf16(fp32(code[q[n][k]] * absmax[(n*K + k) / 64])); nibble 2i of a row is the
// high nibble of byte i.  The activation is bf16 (no input quantisation).
//
// Structure: one workgroup of four waves (2 x 2) per BM x BN tile; K walks in
// stages of 64 elements, which is exactly one NF4 block of every weight row.
// Both operand tiles live in a two-stage LDS ring as bf16 rows of 128 bytes
// with 16-byte chunks XOR-swizzled by (row >> 1) & 7.  The activation tile
// goes global -> LDS with buffer_load ... lds; the weight tile is decoded by the
// workgroup itself: each thread owns one weight row (two threads per row for
// BN = 128), loads its 32 (16) packed bytes and the block's absmax a stage
// ahead, looks each packed byte up in a 256-entry table of codebook value
// pairs in LDS (one 8-byte read for two weights), multiplies by the absmax
// and rounds to bf16 into the stage; the lookups and the scaling are issued
// a few matrix-core instructions apart so the reads' latency is hidden.  Each stage is
// four 16-k substeps of v_mfma_f32_32x32x16_bf16 with the next substep's
// fragments read during the current one; the decode of the next stage is
// spread over the substeps so that its VALU work runs beside the matrix cores.
// One barrier per stage, before the last substep: it certifies that every wave
// has read the stage (which frees its buffer for the stage two ahead) and that
// the next stage's activation tile and decoded weights are complete.  The
// weight fragment is the MFMA's first operand (transposed accumulator blocks:
// a lane owns four consecutive output columns of a row), and the epilogue's
// gate rows are loaded into LDS behind the ring at the start.
#include <type_traits>

#include "epi_qkv_rope.h"

namespace sfm {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define SFM_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kBK = 64;     // k elements per stage
constexpr int kRowB = 128;  // LDS bytes per tile row per stage
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kGroupM = 8;

// s_waitcnt with vmcnt <= VM and lgkmcnt == 0 (expcnt not waited on)
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}

// s_waitcnt with vmcnt <= VM only
template <int VM>
__device__ __forceinline__ void wait_vm() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS that has already been waited for; the empty asm
// statements keep the compiler from moving LDS accesses across it, and no
// fence is used because a fence would also drain the loads still in flight.
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

// 8 x byte E of w (the byte offset of its entry in the pair table) in one instruction: a
// shift whose source operand selects the byte (SDWA), in place of a bit-field extract and a shift
template <int E>
__device__ __forceinline__ uint32_t byte_x8(uint32_t w) {
    uint32_t r;
    if constexpr (E == 0)
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(w));
    else if constexpr (E == 1)
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(w));
    else if constexpr (E == 2)
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(w));
    else
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(w));
    return r;
}

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_nf4_kernel(
    const uint16_t* __restrict__ A, const uint8_t* __restrict__ Wq, const float* __restrict__ absmax, Nf4Code code,
    uint16_t* out, const uint16_t* resid, const float* __restrict__ gate, int64_t gate_stride, int M, int N, int K,
    int L, int ntm, int ntn, RopeArgs rope) {
    constexpr int TM = BM / 2, TN = BN / 2;    // wave tile
    constexpr int FM = TM / 32, FN = TN / 32;  // 32 x 32 MFMA tiles per wave
    constexpr int NF = FM + FN;                // fragments per substep
    constexpr int AI = BM / 32;                // 1 KiB activation wave-loads per stage per wave
    constexpr int EPT = BN * kBK / 256;        // weights decoded per thread per stage
    constexpr int TPR = kBK / EPT;             // threads per weight row
    constexpr int EPP = EPT / 4;               // weights per decode part (four parts per stage)
    constexpr int NW = EPT / 8;                // packed dwords per thread per stage
    static_assert(TPR * BN == 256 && EPP % 8 == 0, "decode ownership");
    // LDS bytes of one wave's epilogue staging (gemm_epilogue_lds): within the smallest ring array
    constexpr int EPI_BYTES = EPI == SFM_EPI_RESID_GATE ? TM / 2 * (TN * 4 + ((TN / 4) % 16 ? 16 : 0))
                                                        : TM * (EPI == SFM_EPI_SWIGLU ? TN / 2 : TN) * 2;
    static_assert(BN <= BM && EPI_BYTES <= BN * kRowB, "epilogue staging fits a ring array");
    // LDS: the two-stage ring as four separate arrays (activation and weight half of each stage),
    // the codebook of byte pairs (entry b: the values of packed byte b's two elements side by side)
    // and the epilogue's factors.  Distinct arrays let the compiler see that the codebook reads and
    // the decoded-weight writes do not touch the activation halves that the direct global -> LDS
    // loads fill, so it does not make them wait for those loads.
    __shared__ __attribute__((aligned(1024))) uint8_t ring_a0[BM * kRowB];
    __shared__ __attribute__((aligned(1024))) uint8_t ring_a1[BM * kRowB];
    __shared__ __attribute__((aligned(1024))) uint8_t ring_b0[BN * kRowB];
    __shared__ __attribute__((aligned(1024))) uint8_t ring_b1[BN * kRowB];
    // (the table's alignment, the largest, puts it at LDS address 0: a lookup address is then the
    // byte offset alone, with no base to add)
    __shared__ __attribute__((aligned(2048))) float2 lut2[256];
    __shared__ float scl_lds[BM + 4 * BN];
    auto stage_a = [&](int s) -> uint8_t* { return s ? ring_a1 : ring_a0; };
    auto stage_b = [&](int s) -> uint8_t* { return s ? ring_b1 : ring_b0; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    grouped_tile(xcd_tile_id(), ntm, ntn, kGroupM, tm, tn);
    const int m0 = tm * BM;
    const int nks = K / kBK;
    lut2[tid] = make_float2(code.v[tid >> 4], code.v[tid & 15]);  // high nibble: the earlier element
    // the epilogue's factors: row and column scales (1: bf16 operands) and, for the gated
    // residual, the gate rows of the (at most three) batches the tile's rows touch; written here,
    // read after the main loop's barriers
    float* scl = scl_lds;
    const int bt0 = EPI == SFM_EPI_RESID_GATE ? min(m0, M - 1) / L : 0;
    for (int e = tid; e < BM + (EPI == SFM_EPI_RESID_GATE ? 4 : 1) * BN; e += 256) {
        float v = 1.0f;
        if (e >= BM + BN) {
            const int g = (e - BM - BN) / BN, c = (e - BM - BN) % BN;
            v = gate[(int64_t)min(bt0 + g, (M - 1) / L) * gate_stride + (int64_t)tn * BN + c];
        }
        scl[e] = v;
    }
    // the QK-norm gamma of the tile's part behind the row-sum exchange area of the epilogue
    if constexpr (EPI == kEpiQkvRope)
        if (tid < 128) reinterpret_cast<uint32_t*>(scl + BM + BN + 4 * TM)[tid] = load_qk_gamma(rope, tn, tid);

    // activation tile: wave-load v covers tile rows 8 (wave + 4 v) + (lane >> 3), physical chunk
    // lane & 7 holding logical chunk (lane & 7) ^ ((row >> 1) & 7)
    // the view starts at the tile's first row (64-bit base): 32-bit offsets stay below BM * 2K
    // bytes whatever M * K is
    const uint16_t* const A0 = A + (int64_t)m0 * K;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)A0, 0, 0x7FFFFFFF, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ra0 = __builtin_amdgcn_make_buffer_rsrc((void*)A0, 0, 0, kRsrcWord3);
    const int lrow = lane >> 3, lch = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
    uint32_t voff[AI];
#pragma unroll
    for (int v = 0; v < AI; ++v) {
        const int row = min(m0 + 8 * (wave + 4 * v) + lrow, M - 1);
        voff[v] = (uint32_t)(row - m0) * (uint32_t)(K * 2) + lch * 16;
    }

    // weight decode ownership: tile row br, elements eo .. eo + EPT - 1 of each stage
    const int br = tid / TPR, eo = (tid % TPR) * EPT;
    const int64_t wr = weight_row<EPI, BN, TN>(br, tn, N);
    const uint8_t* wsrc = Wq + wr * (K / 2) + eo / 2;
    const float* asrc = absmax + wr * (K / 64);
    const int bsx = (br >> 1) & 7;
    uint32_t nb[2][NW];
    float am[2];
    auto nib_load = [&](int slot, int s) {
        s = min(s, nks - 1);
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(wsrc + (int64_t)s * (kBK / 2) + 16 * i);
            nb[slot][4 * i] = x.x;
            nb[slot][4 * i + 1] = x.y;
            nb[slot][4 * i + 2] = x.z;
            nb[slot][4 * i + 3] = x.w;
        }
        am[slot] = asrc[s];
    };
    // part p: weights eo + EPP p .. + EPP - 1 -> EPP / 8 swizzled 16-byte chunks of row br of the
    // weight half of stage stg.  The main loop spreads it over the matrix-core instructions in
    // pieces: the codebook lookups of chunk c (one per packed byte), and later the scaling and
    // rounding of half a chunk (piece k: chunk k >> 1, elements 4 (k & 1) .. +3), the chunk's
    // 16-byte store after its second half
    float2 cvp[EPP / 2];
    uint32_t ob[EPP / 8][4];
    auto lookup_c = [&](int slot, int p, int c) {
        const uint32_t w = nb[slot][p * (EPP / 8) + c];
        const uint8_t* const t = reinterpret_cast<const uint8_t*>(lut2);
        cvp[4 * c + 0] = *reinterpret_cast<const float2*>(t + byte_x8<0>(w));
        cvp[4 * c + 1] = *reinterpret_cast<const float2*>(t + byte_x8<1>(w));
        cvp[4 * c + 2] = *reinterpret_cast<const float2*>(t + byte_x8<2>(w));
        cvp[4 * c + 3] = *reinterpret_cast<const float2*>(t + byte_x8<3>(w));
    };
    auto finish_k = [&](int slot, int stg, int p, int k) {
        const int c = k >> 1, h = k & 1;
#pragma unroll
        for (int e = 2 * h; e < 2 * h + 2; ++e)
            ob[c][e] = cvt_bf16x2(cvp[4 * c + e].x * am[slot], cvp[4 * c + e].y * am[slot]);
        if (h) {
            const int lc = (eo + EPP * p) / 8 + c;
            *reinterpret_cast<u32x4*>(stage_b(stg) + br * kRowB + ((lc ^ bsx) << 4)) =
                u32x4{ob[c][0], ob[c][1], ob[c][2], ob[c][3]};
        }
    };
    auto decode = [&](int slot, int stg, int p) {
#pragma unroll
        for (int c = 0; c < EPP / 8; ++c) lookup_c(slot, p, c);
#pragma unroll
        for (int k = 0; k < EPP / 4; ++k) finish_k(slot, stg, p, k);
    };
    auto dma = [&](int v, int stg, __amdgpu_buffer_rsrc_t r, int s) {
        dma16(r, stage_a(stg) + wave * 1024 + v * 4096, voff[v], s * (kBK * 2));
    };

    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

    // fragments: lane l holds row (l & 31) and 16-byte chunk 2 ks + (l >> 5) of substep ks
    const int lr = lane & 31, lg = lane >> 5, sx = (lr >> 1) & 7;
    const int arow = (wm * TM + lr) * kRowB, brow = (wn * TN + lr) * kRowB;
    u32x4 fr[2][NF];  // f < FN: weight column tile f, else row tile f - FN
    auto ds = [&](int set, int f, int stg, int ks) {
        const int off = ((2 * ks + lg) ^ sx) << 4;
        fr[set][f] = *reinterpret_cast<const u32x4*>(f < FN ? stage_b(stg) + brow + f * 32 * kRowB + off
                                                            : stage_a(stg) + arow + (f - FN) * 32 * kRowB + off);
    };
    auto mfma = [&](int set, int q) {
        const int i = q / FN, j = q % FN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fr[set][j]),
                                                            __builtin_bit_cast(bf16x8, fr[set][FN + i]), acc[i][j], 0, 0, 0);
    };
    // substep: FM x FN MFMAs on `set`, with spread over them: the fragment reads of (rstg, rks)
    // into rset (if RD), decode part dp of `dslot` into dstg (if DEC), wave-loads v0 .. v1 (if DM)
    auto substep = [&](int set, bool RD, int rset, int rstg, int rks, bool DEC, int dslot, int dstg, int dp,
                       bool DM, int mstg, __amdgpu_buffer_rsrc_t mr, int ms) {
        constexpr int NQ = FM * FN;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            mfma(set, q);
            if (DM)
#pragma unroll
                for (int v = q * AI / NQ; v < (q + 1) * AI / NQ; ++v) dma(v, mstg, mr, ms);
            if (RD)
#pragma unroll
                for (int f = q * NF / NQ; f < (q + 1) * NF / NQ; ++f) ds(rset, f, rstg, rks);
            if (DEC && q >= 1 && q < 1 + EPP / 8) lookup_c(dslot, dp, q - 1);
            if (DEC && q >= NQ / 2 && q < NQ / 2 + EPP / 4) finish_k(dslot, dstg, dp, q - NQ / 2);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // prologue: codebook, weights of stages 0 and 1, activations of stages 0 and 1; stage 0
    // fully decoded, stage 1 decoded in its first part (the rest follows in stage 0)
    nib_load(0, 0);
    nib_load(1, 1);
#pragma unroll
    for (int v = 0; v < AI; ++v) dma(v, 0, ra, 0);
#pragma unroll
    for (int v = 0; v < AI; ++v) dma(v, 1, ra, 1);
    wait_vm_lgkm0<0>();
    lds_barrier();
#pragma unroll
    for (int p = 0; p < 4; ++p) decode(0, 0, p);
    decode(1, 1, 0);
    wait_vm_lgkm0<0>();
    lds_barrier();
#pragma unroll
    for (int f = 0; f < NF; ++f) ds(0, f, 0, 0);

    // stage t: set 0 holds substep 0 of stage t on entry and substep 0 of stage t + 1 on exit;
    // weights of stage t + 1 are decoded in parts 1..3 here (part 0 in stage t - 1), those
    // of stage t + 2 are loaded here and decoded from part 0 on after the barrier
    constexpr int NL = NW / 4 + 1;  // vector loads of one stage's packed weights and absmax
    // the two register slots of packed weights alternate with the stage's parity (compile-time)
    auto stage = [&](auto P, int t) {
        constexpr int s2 = decltype(P)::value, s1 = s2 ^ 1;  // slots of stages t + 2 and t + 1
        constexpr int cur = s2, nxt = s1;                      // ring stages of t (and t + 2), t + 1
        const __amdgpu_buffer_rsrc_t rA = t + 2 < nks ? ra : ra0;
        substep(0, true, 1, cur, 1, true, s1, nxt, 1, false, cur, rA, 0);
        nib_load(s2, t + 2);
        substep(1, true, 0, cur, 2, true, s1, nxt, 2, false, cur, rA, 0);
        substep(0, true, 1, cur, 3, true, s1, nxt, 3, false, cur, rA, 0);
        wait_vm_lgkm0<NL>();  // stage t + 1's activations have landed; this wave's reads and decode writes are done
        lds_barrier();        // ... and every wave's
        substep(1, true, 0, nxt, 0, false, s2, cur, 0, true, cur, rA, t + 2);
        wait_vm<AI>();        // stage t + 2's packed weights (loaded before the wave-loads just issued)
        decode(s2, cur, 0);
    };
    // K % 256 == 0: nks is a multiple of 4
    for (int t = 0; t < nks; t += 2) {
        stage(std::integral_constant<int, 0>{}, t);
        stage(std::integral_constant<int, 1>{}, t + 1);
    }
    wait_vm_lgkm0<0>();
    lds_barrier();
    // each wave stages its tile through one of the four ring arrays
    uint8_t* const estg = wave == 0 ? ring_a0 : wave == 1 ? ring_b0 : wave == 2 ? ring_a1 : ring_b1;
    if constexpr (EPI == kEpiQkvRope)
        epilogue_qkv_rope<FM, FN>(acc, estg, scl + BM + BN, m0 + wm * TM, wm, wn, tn, lane, M, L, scl + wm * TM,
                                  scl + BM + wn * TN, reinterpret_cast<const uint32_t*>(scl + BM + BN + 4 * TM), rope);
    else
        gemm_epilogue_lds<EPI, BN, TN, FM, FN>(acc, estg, m0 + wm * TM, wn, tn, lane, M, N, L, out, resid,
                                                 scl + wm * TM, scl + BM + wn * TN, scl + BM + BN + wn * TN, bt0);
}

template <int BM, int BN, int EPI>
hipError_t launch_cfg(const uint16_t* a, const uint8_t* w, const float* am, const Nf4Code& code, uint16_t* out,
                      const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N, int K, int L,
                      hipStream_t st, const RopeArgs& rope = RopeArgs{}) {
    const int ntm = (M + BM - 1) / BM;
    const int ntn = N / BN;
    auto kern = gemm_nf4_kernel<BM, BN, EPI>;  // all of its LDS is static
    hipLaunchKernelGGL(kern, dim3(ntm * ntn), dim3(256), 0, st, a, w, am, code, out, resid, gate, gate_stride, M, N,
                       K, L, ntm, ntn, rope);
    return hipGetLastError();
}

// Rounds of workgroups over the 256 compute units times the work of one tile.
inline double nf4_tile_cost(int M, int N, int BM, int BN) {
    const int64_t tiles = (int64_t)((M + BM - 1) / BM) * (N / BN);
    return (double)((tiles + 255) / 256) * BM * BN;
}

template <int EPI>
hipError_t launch_epi(const uint16_t* a, const uint8_t* w, const float* am, const Nf4Code& code, uint16_t* out,
                      const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N, int K, int L,
                      hipStream_t st) {
    const double c256 = N % 256 == 0 ? nf4_tile_cost(M, N, 256, 256) : 1e300;
    const double c128 = nf4_tile_cost(M, N, 256, 128) * 1.15;
    if (c256 <= c128) return launch_cfg<256, 256, EPI>(a, w, am, code, out, resid, gate, gate_stride, M, N, K, L, st);
    return launch_cfg<256, 128, EPI>(a, w, am, code, out, resid, gate, gate_stride, M, N, K, L, st);
}

}  // namespace

hipError_t launch_gemm_nf4(int epi, const uint16_t* a, const uint8_t* w, const float* absmax, const Nf4Code& code,
                           uint16_t* out, const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N,
                           int K, int L, hipStream_t st) {
    if (M == 0) return hipSuccess;
    switch (epi) {
        case SFM_EPI_STORE:
            return launch_epi<SFM_EPI_STORE>(a, w, absmax, code, out, resid, gate, gate_stride, M, N, K, L, st);
        case SFM_EPI_RESID_GATE:
            return launch_epi<SFM_EPI_RESID_GATE>(a, w, absmax, code, out, resid, gate, gate_stride, M, N, K, L, st);
        case SFM_EPI_SWIGLU:
            return launch_epi<SFM_EPI_SWIGLU>(a, w, absmax, code, out, resid, gate, gate_stride, M, N, K, L, st);
        default:
            return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_nf4_qkv_rope(const uint16_t* a, const uint8_t* w, const float* absmax, const Nf4Code& code,
                                    int M, int K, int L, const RopeArgs& ra, hipStream_t st) {
    if (M == 0) return hipSuccess;
    return launch_cfg<256, 256, kEpiQkvRope>(a, w, absmax, code, nullptr, nullptr, nullptr, 0, M, 3 * ra.H * 256, K, L,
                                             st, ra);
}

}  // namespace sfm
