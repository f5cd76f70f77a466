// Flash-style joint attention, head_dim 256, matrix cores, fp32 softmax.
//
// Research note, "Model architecture": one shared bidirectional self-attention
// over the whole [text | image] sequence.  o = softmax(q k^T / 16) v per head.
//
// Layout: a workgroup owns 128 queries of one (batch, head); each of its four
// waves owns 32 queries whose q fragments stay in registers.  Key tiles of 64
// keys stream through LDS (K as [key][d], V^T as [d][key]).
// Per tile a wave computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K
// rows, B = Q rows), so every lane holds the scores of ONE query column
// (lane & 15) for keys 4*(lane>>4)+r: the softmax max is a reduction over the
// lane's values and the 4 lanes sharing the column; the running sum stays a
// per-lane partial until the end.  P^T then feeds O^T += V^T P^T directly from
// registers as the B operand (keys k-sliced identically in the V^T operand),
// and O^T's query column is again lane-local, so rescaling is lane-local too.
// The P V product runs in fp16 (P and V^T in fp16, fp32 accumulation): fp16
// keeps 3 more mantissa bits of P than bf16, and V's bf16 values are exact in
// fp16.  P in bf16 perturbs o by about 1e-3 relative, which the per-token FP8
// quantisation of o downstream turns into percent-level changes of the block.
// The running max is only moved when a tile raises it by more than 2^8
// (scores then stay below 2^8 relative to the kept max), which skips most
// rescales of the 128-register accumulator.
#include "sfm_internal.h"

namespace sfm {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kQB = 128;  // queries per workgroup
constexpr int kKB = 64;   // keys per tile
constexpr int kD = 256;
// LDS rows are padded so that the 8 (K, 16-byte reads) or 16 (V^T, 8-byte
// reads) rows read together start in different banks, and every fragment
// address is a per-lane base plus a compile-time offset.
constexpr int kKRow = kD * 2 + 16;   // K tile row (one key): 528 B
constexpr int kVRow = kKB * 2 + 8;   // V^T tile row (one d): 136 B
constexpr int kKBytes = kKB * kKRow;
constexpr int kVBytes = kD * kVRow;

__device__ __forceinline__ int k_off(int key, int chunk16) { return key * kKRow + chunk16 * 16; }
__device__ __forceinline__ int v_off(int d, int chunk8) { return d * kVRow + chunk8 * 8; }

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ vt,
    uint16_t* __restrict__ o, int L, int Lp, int H, int nqb) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* const ktile = smem;               // [64 keys][256 d]
    uint8_t* const vtile = smem + kKBytes;  // [256 d][64 keys]

    // XCD-aware order: each XCD gets a contiguous run of (head, query-block) pairs
    int bid = blockIdx.x;
    const int nwg = gridDim.x;
    if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
    const int qb = bid % nqb;
    const int bh = bid / nqb;  // b * H + h
    const int h = bh % H, b = bh / H;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const uint16_t* Qh = q + (int64_t)bh * Lp * kD;
    const uint16_t* Kh = k + (int64_t)bh * Lp * kD;
    const uint16_t* Vh = vt + (int64_t)bh * kD * Lp;
    const int q0 = qb * kQB + wave * 32;

    // q fragments (B operand of S^T): rows q0 + qt*16 + lr, dims ks*32 + 8*lg .. +8
    bf16x8 qf[2][8];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qf[qt][ks] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(Qh + (int64_t)(q0 + qt * 16 + lr) * kD + ks * 32 + 8 * lg));

    // tile staging: K tile = 64 rows x 32 chunks of 16 B (8 per thread);
    // V^T tile = 256 rows x 8 chunks of 16 B (8 per thread)
    u32x4 rst[8];
    auto gload_k = [&](int key0) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int i = tid + c * 256;
            rst[c] = *reinterpret_cast<const u32x4*>(Kh + (int64_t)(key0 + (i >> 5)) * kD + (i & 31) * 8);
        }
    };
    auto lstore_k = [&]() {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int i = tid + c * 256;
            *reinterpret_cast<u32x4*>(ktile + k_off(i >> 5, i & 31)) = rst[c];
        }
    };
    auto gload_v = [&](int key0) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int i = tid + c * 256;
            rst[c] = *reinterpret_cast<const u32x4*>(Vh + (int64_t)(i >> 3) * Lp + key0 + (i & 7) * 8);
        }
    };
    auto lstore_v = [&]() {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int i = tid + c * 256;
            const int d = i >> 3, c16 = i & 7;
            *reinterpret_cast<u32x2*>(vtile + v_off(d, 2 * c16)) = u32x2{rst[c].x, rst[c].y};
            *reinterpret_cast<u32x2*>(vtile + v_off(d, 2 * c16 + 1)) = u32x2{rst[c].z, rst[c].w};
        }
    };

    v4f oacc[2][16];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) oacc[qt][dt] = v4f{0.f, 0.f, 0.f, 0.f};
    float mrun[2] = {-1e30f, -1e30f};
    float lsum[2] = {0.f, 0.f};
    const float cs = 0.0625f * 1.4426950408889634f;  // 1/sqrt(256) * log2(e)

    const int nkt = (L + kKB - 1) / kKB;
    // Pipeline, one K buffer and one V^T buffer in LDS:
    //   S phase reads K_i while K_{i+1} is fetched into registers; barrier A;
    //   K_{i+1} -> LDS; PV phase reads V_i while V_{i+1} is fetched; barrier B;
    //   V_{i+1} -> LDS (made visible by the next barrier A).
    gload_k(0);
    lstore_k();
    gload_v(0);
    lstore_v();
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const int key0 = kt * kKB;
        const bool more = kt + 1 < nkt;
        if (more) gload_k(key0 + kKB);
        const uint8_t* kl = ktile;
        const uint8_t* vl = vtile;

        // S^T tile: s[qt][t4][r] = score(key = t4*16 + 4*lg + r, query = qt*16 + lr)
        v4f s[2][4];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) s[qt][t4] = v4f{0.f, 0.f, 0.f, 0.f};
        // K fragments double-buffered in registers, one d-slice (ks) ahead;
        // the scheduling barriers keep the compiler from hoisting all 32 loads.
        bf16x8 kf[2][4];
        auto load_kf = [&](int slot, int ks) {
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4)
                kf[slot][t4] =
                    __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kl + k_off(t4 * 16 + lr, ks * 4 + lg)));
        };
        load_kf(0, 0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            if (ks + 1 < 8) load_kf((ks + 1) & 1, ks + 1);
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
                    s[qt][t4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks & 1][t4], qf[qt][ks], s[qt][t4], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (key0 + kKB > L) {  // ragged last tile: mask keys >= L
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (key0 + t4 * 16 + 4 * lg + r >= L) {
                        s[0][t4][r] = -INFINITY;
                        s[1][t4][r] = -INFINITY;
                    }
        }

        // online softmax (exp2 domain), P^T packed as the B operand of O^T += V^T P^T
        f16x8 pf[2][2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            float mx = -INFINITY;
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[qt][t4][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mnew = fmaxf(mrun[qt], mx * cs);
            if (__builtin_amdgcn_ballot_w64(mnew > mrun[qt] + 8.0f) != 0) {
                const float alpha = exp2f(mrun[qt] - mnew);
                mrun[qt] = mnew;
                lsum[qt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < 16; ++dt) oacc[qt][dt] *= alpha;
            }
            const float mref = mrun[qt];
            float ls = 0.f;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                f16x8 ph;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = exp2f(s[qt][2 * h2 + (e >> 2)][e & 3] * cs - mref);
                    ph[e] = (_Float16)p;
                    ls += (float)ph[e];
                }
                pf[qt][h2] = ph;
            }
            lsum[qt] += ls;
        }

        __syncthreads();  // A: every wave is done with K_i (and V_i is visible)
        if (more) {
            lstore_k();
            gload_v(key0 + kKB);
        }

        // O^T[d][query] += sum_key V^T[d][key] P^T[key][query]
        // V^T fragments: 32 (h2, dt) groups, loaded four groups ahead
        f16x8 vf[2][4];
        auto load_vf = [&](int slot, int g) {  // groups 4g .. 4g+3: h2 = g / 4, dt = 4 (g % 4) + u
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int h2 = g >> 2, d = (4 * (g & 3) + u) * 16 + lr;
                const u32x2 lo = *reinterpret_cast<const u32x2*>(vl + v_off(d, h2 * 8 + lg));
                const u32x2 hi = *reinterpret_cast<const u32x2*>(vl + v_off(d, h2 * 8 + 4 + lg));
                vf[slot][u] = __builtin_bit_cast(f16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
            }
        };
        load_vf(0, 0);
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            if (g + 1 < 8) load_vf((g + 1) & 1, g + 1);
            const int h2 = g >> 2;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int dt = 4 * (g & 3) + u;
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
                    oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[g & 1][u], pf[qt][h2], oacc[qt][dt], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();  // B: every wave is done with V_i (and K_{i+1} is visible)
        if (more) lstore_v();
    }

    // normalise and write o[b*L + query][h*256 + d]
    const int D = H * kD;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        float l = lsum[qt];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        const float inv = 1.0f / l;
        const int qi = q0 + qt * 16 + lr;
        if (qi < L) {
            uint16_t* orow = o + ((int64_t)b * L + qi) * D + h * kD;
#pragma unroll
            for (int dt = 0; dt < 16; ++dt) {
                const v4f v = oacc[qt][dt];
                u32x2 w;
                w.x = pack_bf16x2(v[0] * inv, v[1] * inv);
                w.y = pack_bf16x2(v[2] * inv, v[3] * inv);
                *reinterpret_cast<u32x2*>(orow + dt * 16 + 4 * lg) = w;
            }
        }
    }
}

}  // namespace

hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* vt, uint16_t* o, int B, int L,
                            int H, hipStream_t st) {
    if (L == 0) return hipSuccess;
    const int Lp = padded_len(L);
    const int nqb = Lp / kQB;
    const size_t shm = (size_t)kKBytes + kVBytes;
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute((const void*)attn_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        attr_set = true;
    }
    hipLaunchKernelGGL(attn_kernel, dim3(nqb * H * B), dim3(256), shm, st, q, k, vt, o, L, Lp, H, nqb);
    return hipGetLastError();
}

}  // namespace sfm
