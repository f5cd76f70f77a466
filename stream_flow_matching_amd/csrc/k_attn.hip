// Flash-style joint attention, head_dim 256, matrix cores, fp32 softmax.
//
// Research note, "Model architecture": one shared bidirectional self-attention
// over the whole [text | image] sequence.  o = softmax(q k^T / 16) v per head.
//
// Layout: a workgroup owns 192 queries of one (batch, head); each of its twelve
// waves owns 16 queries whose q fragments stay in registers (three waves per
// SIMD, at most 168 registers each: while one wave is in its softmax, two can
// feed the SIMD's matrix core).  Tiles of 64 keys stream global -> LDS with
// buffer_load ... lds (no staging registers): K as [key][d] and V^T as
// [d][key], two stages of 64 KiB, one barrier per tile.  A wave raises its
// priority while it issues matrix-core work and drops it for the softmax, so
// the SIMD's other waves, when they are in their MFMA sections, go first and
// the softmax arithmetic fills the gaps.
// Per tile a wave computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K
// rows, B = Q rows), so every lane holds the scores of ONE query column
// (lane & 15) for keys 4*(lane>>4)+r: the softmax max is a reduction over the
// lane's values and the 4 lanes sharing the column; the running sum of the
// weights comes from one extra MFMA per 32 keys and query tile (a constant
// operand whose first row is ones).  P^T then feeds O^T += V^T P^T directly from
// registers as the B operand, and O^T's query column is again lane-local, so
// rescaling is lane-local too.  The running max is only moved when a tile
// raises it by more than 2^8 (scores then stay below 2^8 relative to the kept
// max), which skips most rescales of the 64-register accumulator.
//
// The P V product runs in fp16 (P and V^T in fp16, fp32 accumulation): fp16
// keeps 3 more mantissa bits of P than bf16.  V's bf16 values are exact in
// fp16 from 2^-17 up to 65504; smaller magnitudes keep fp16's subnormal
// quantum 2^-24 (an absolute error below 2^-25) and larger ones saturate to
// +-65504 in the rotary kernel.  P in bf16 perturbs o by about 1e-3 relative,
// which the per-token FP8 quantisation of o downstream turns into
// percent-level changes of the block.
//
// Schedule: the work is the list of items (batch, head, block of 192 queries),
// batch-major, each with its walk of key tiles.  The grid is one persistent
// workgroup per compute unit (G).  Workgroup g first takes whole items
// r G + g for the R = items / G full rounds, so the workgroups of one XCD walk
// neighbouring items (the same K and V) in step, as a plain grid would; the
// (item, tile) units of the remaining items (stream-K) are then split evenly:
// workgroup g takes tail units [g Ut / G, (g + 1) Ut / G), and every workgroup
// ends at the same time however the items divide the grid.  An item covered
// whole is normalised and stored; the first or last piece of an item shared
// with a neighbouring range is stored as a partial result (O divided by the
// piece's row sums in fp16, the running max and the row sums in fp32) and attn_merge_kernel
// combines an item's pieces the way the online softmax combines key tiles.
//
// LDS rows are XOR-swizzled in 16-byte chunks, applied through the source
// addresses of the direct loads: K rows (512 bytes) by row & 15, V^T rows (128
// bytes, two per 256-byte bank line) by (row >> 1) & 7, so the 16 rows one
// operand read touches land in 16 distinct 16-byte bank slots.  V^T's key
// order inside every group of 32 keys is [4g..4g+3, 16+4g..16+4g+3] for
// g = 0..3 (written that way by the rotary kernel), so a lane's eight P^T keys
// are one 16-byte chunk.
#include <algorithm>

#include "sfm_internal.h"

namespace sfm {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

#define SFM_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kQB = 192;              // queries per workgroup
constexpr int kWaves = kQB / 16;      // one wave per 16 queries
constexpr int kKB = 64;               // keys per tile
constexpr int kD = 256;
constexpr int kKTile = kKB * kD * 2;  // 32 KiB
constexpr int kRsrcWord3 = 0x00020000;

struct Loader {
    __amdgpu_buffer_rsrc_t rk, rv;
    // a tile is 32 wave-loads of K and 32 of V^T (1 KiB each); wave w issues blocks w + 12 i
    uint32_t kvoff[3];      // per-lane byte offsets inside a K tile, block wave + 12 i
    uint32_t vvoff;         // per-lane byte offset inside a V^T tile
    uint32_t lds0;          // this wave's first 1 KiB destination inside a tile
    int Lp2;                // bytes per V^T row
    int nblk;               // 3 for waves 0..7, 2 for waves 8..11 (32 blocks per tile)

    __device__ __forceinline__ void issue(uint8_t* stage, int key0) const {
#pragma unroll
        for (int i = 0; i < 3; ++i)
            if (i < nblk)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, SFM_LDS(stage + lds0 + i * 12288), 16, kvoff[i],
                                                         (uint32_t)(key0 + 24 * i) * 512u, 0, 0);
#pragma unroll
        for (int i = 0; i < 3; ++i)
            if (i < nblk)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, SFM_LDS(stage + kKTile + lds0 + i * 12288), 16, vvoff,
                                                         (uint32_t)(96 * i * Lp2 + key0 * 2), 0, 0);
    }
};

// max over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the lanes holding one query
// column), with the cross-row lane swaps instead of LDS permutes
__device__ __forceinline__ float col_max(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Key tiles of one batch's walk: tiles wholly inside the text padding [Tb, T) are
// skipped, so tile e of the walk is key tile e before the padding and e + nskip after.
struct KeyWalk {
    int skip0, nskip, nkt;
    __host__ __device__ KeyWalk(int L, int T, int Tb) {
        skip0 = (Tb + kKB - 1) / kKB;
        nskip = T / kKB - skip0 > 0 ? T / kKB - skip0 : 0;
        nkt = (L + kKB - 1) / kKB - nskip;
    }
    __host__ __device__ int key(int e) const { return (e < skip0 ? e : e + nskip) * kKB; }
};

// A partial result: per wave, O^T / l as the lanes hold it ([dt][lane] four fp16; |O / l| is at
// most max |v|, and fp16 keeps 3 more bits than the bf16 output), then (m, l) of its 16
// queries in fp32; two slots per workgroup (the piece that starts inside an item, the piece
// that ends inside one).  Sizes in floats.
constexpr int kPartO = kWaves * 16 * 64 * 2;
constexpr int kPartFloats = kPartO + kWaves * 16 * 2;

// Tail unit u (units counted from the first tile of item I0; items numbered batch-major, Hn per
// batch): the item holding it, as batch b and item index it inside the batch, and the item's
// first tail unit.
struct UnitPos {
    int b, it;
    int64_t first;
};
__host__ __device__ __forceinline__ UnitPos locate_tail(int64_t u, int I0, int Hn, int L, int T,
                                                        const TextLens& lens, int varlen) {
    int b = I0 / Hn, i0 = I0 - b * Hn;
    int64_t pre = 0;
    for (;;) {
        const KeyWalk kw(L, T, varlen ? lens.len[b] : T);
        const int64_t nb = (int64_t)(Hn - i0) * kw.nkt;
        if (u < pre + nb) {
            const int k = (int)((u - pre) / kw.nkt);
            return UnitPos{b, i0 + k, pre + (int64_t)k * kw.nkt};
        }
        pre += nb;
        ++b;
        i0 = 0;
    }
}

__global__ __launch_bounds__(768) __attribute__((amdgpu_waves_per_eu(3, 3))) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ vt,
    uint16_t* __restrict__ o, float* __restrict__ part, int L, int Lp, int H, int nqb, int T, TextLens lens,
    int varlen, int R, int64_t Ut) {
    __shared__ __attribute__((aligned(1024))) uint8_t st0[2 * kKTile];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[2 * kKTile];

    // XCD-aware order: each XCD gets a contiguous run of items and tail units (neighbouring items
    // share K and V, and the XCD's workgroups walk them in step)
    int g = blockIdx.x;
    const int G = gridDim.x;
    if ((G & 7) == 0) g = (g & 7) * (G >> 3) + (g >> 3);
    const int Hn = H * nqb;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int D = H * kD;

    // fragment read offsets.  K rows t4*16 + lr: chunk (ks*4 + lg) ^ lr = 4 (ks ^ (lr >> 2)) + (lg ^ (lr & 3)),
    // so ks = 4 u + m reads at kb[m] + u * 256.  V^T rows dt*16 + lr: chunk (h2*4 + lg) ^ ((lr >> 1) & 7).
    int kb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) kb[m] = lr * 512 + ((lg ^ (lr & 3)) << 4) + ((m ^ (lr >> 2)) << 6);
    const int x = (lr >> 1) & 7;
    const int csw = (lg ^ (x & 3)) << 4;
    const int vb0 = lr * 128 + csw + ((x >> 2) << 6);        // keys 0..31 of the tile
    const int vb1 = lr * 128 + csw + ((1 ^ (x >> 2)) << 6);  // keys 32..63

    // row sums of P^T come from the matrix cores: a constant A fragment whose first row is all
    // ones (row 0 of the A operand lives in lanes 0, 16, 32, 48) turns O^T += V^T P^T into l += 1^T P^T, summing exactly the
    // fp16 weights that O accumulates; lane l (l < 16) holds query column l in lacc[qt][0]
    f16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (_Float16)(lr == 0 ? 1.0f : 0.0f);
    const float cs = 0.0625f * 1.4426950408889634f;  // 1/sqrt(256) * log2(e)

    // segments: first whole items r G + g (r < R), then this workgroup's range of the tail units
    int r = 0;
    const int64_t u_end = Ut * (g + 1) / G;
    for (int64_t u = Ut * g / G;;) {
        // the segment: tiles [e0, e1) of item (b, h, qb)
        int b, it, e0, e1;
        if (r < R) {
            const int I = r * G + g;
            ++r;
            b = I / Hn;
            it = I - b * Hn;
            e0 = 0;
            e1 = KeyWalk(L, T, varlen ? lens.len[b] : T).nkt;
        } else if (u < u_end) {
            const UnitPos pos = locate_tail(u, R * G, Hn, L, T, lens, varlen);
            b = pos.b;
            it = pos.it;
            e0 = (int)(u - pos.first);
            e1 = (int)(min(u_end, pos.first + KeyWalk(L, T, varlen ? lens.len[b] : T).nkt) - pos.first);
            u = pos.first + e1;
        } else {
            break;
        }
        const int h = it / nqb, qb = it % nqb, bh = b * H + h;
        const int Tb = varlen ? lens.len[b] : T;  // this sample's text rows; keys [Tb, T) are padding
        const KeyWalk kw(L, T, Tb);

        const uint16_t* Qh = q + (int64_t)bh * Lp * kD;
        const int q0 = qb * kQB + wave * 16;

        Loader ld;
        ld.rk = __builtin_amdgcn_make_buffer_rsrc((void*)(k + (int64_t)bh * Lp * kD), 0, Lp * kD * 2, kRsrcWord3);
        ld.rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vt + (int64_t)bh * kD * Lp), 0, kD * Lp * 2, kRsrcWord3);
        ld.Lp2 = Lp * 2;
        ld.lds0 = (uint32_t)wave * 1024;
        {
            // K tile: 1 KiB block (wave + 12 i) holds rows 2 wave + (lane >> 5) + 24 i (relative to the
            // tile), physical chunk lane & 31 = logical chunk ^ (row & 15)
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                const int r = 2 * wave + (lane >> 5);
                ld.kvoff[i] = (uint32_t)(r * 512 + (((lane & 31) ^ ((r + 24 * i) & 15)) * 16));
            }
            ld.nblk = wave < 8 ? 3 : 2;
            // V^T tile: 1 KiB block (wave + 12 i) holds rows 8 wave + (lane >> 3) + 96 i, physical chunk
            // lane & 7 = logical chunk ^ ((row >> 1) & 7) = logical ^ ((4 (wave & 1) + (lane >> 4)) & 7),
            // which does not depend on i
            const int vrow = 8 * wave + (lane >> 3);
            ld.vvoff = (uint32_t)(vrow * Lp * 2 + (((lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7)) * 16));
        }

        // q fragments (B operand of S^T): rows q0 + qt*16 + lr, dims ks*32 + 8*lg .. +8 (the last item's
        // rows past Lp read row Lp - 1; their results are not stored)
        constexpr int NQT = 1;
        bf16x8 qf[NQT][8];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                qf[qt][ks] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(Qh + (int64_t)min(q0 + qt * 16 + lr, Lp - 1) * kD + ks * 32 + 8 * lg));

        v4f oacc[NQT][16];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int dt = 0; dt < 16; ++dt) oacc[qt][dt] = v4f{0.f, 0.f, 0.f, 0.f};
        float mrun[NQT];
        for (int qt = 0; qt < NQT; ++qt) mrun[qt] = -1e30f;
        v4f lacc[NQT];
        for (int qt = 0; qt < NQT; ++qt) lacc[qt] = v4f{0.f, 0.f, 0.f, 0.f};

        auto compute = [&](const uint8_t* stg, int key0) {
            const uint8_t* kl = stg;
            const uint8_t* vl = stg + kKTile;
            // S^T tile: s[qt][t4][r] = score(key = t4*16 + 4*lg + r, query = qt*16 + lr)
            v4f s[NQT][4];
    #pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
    #pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) s[qt][t4] = v4f{0.f, 0.f, 0.f, 0.f};
            bf16x8 kf[2][4];
            auto load_kf = [&](int slot, int ks) {
                const int base = kb[ks & 3] + (ks >> 2) * 256;
    #pragma unroll
                for (int t4 = 0; t4 < 4; ++t4)
                    kf[slot][t4] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kl + base + t4 * 8192));
            };
            __builtin_amdgcn_s_setprio(1);
            load_kf(0, 0);
    #pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                if (ks + 1 < 8) load_kf((ks + 1) & 1, ks + 1);
    #pragma unroll
                for (int t4 = 0; t4 < 4; ++t4)
    #pragma unroll
                    for (int qt = 0; qt < NQT; ++qt)
                        s[qt][t4] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks & 1][t4], qf[qt][ks], s[qt][t4], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            // mask keys >= L (ragged last tile) and the sample's text padding [Tb, T)
            if (key0 + kKB > L || (Tb < T && key0 < T && key0 + kKB > Tb)) {
    #pragma unroll
                for (int t4 = 0; t4 < 4; ++t4)
    #pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (const int key = key0 + t4 * 16 + 4 * lg + r; key >= L || (key >= Tb && key < T))
    #pragma unroll
                            for (int qt = 0; qt < NQT; ++qt) s[qt][t4][r] = -INFINITY;
            }

            __builtin_amdgcn_s_setprio(0);
            // online softmax (exp2 domain), P^T packed as the B operand of O^T += V^T P^T
            f16x8 pf[NQT][2];
    #pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                float mx = fmaxf(fmaxf(s[qt][0][0], s[qt][0][1]), fmaxf(s[qt][0][2], s[qt][0][3]));
    #pragma unroll
                for (int t4 = 1; t4 < 4; ++t4)
                    mx = fmaxf(mx, fmaxf(fmaxf(s[qt][t4][0], s[qt][t4][1]), fmaxf(s[qt][t4][2], s[qt][t4][3])));
                mx = col_max(mx);
                const float mnew = fmaxf(mrun[qt], mx * cs);
                if (__builtin_amdgcn_ballot_w64(mnew > mrun[qt] + 8.0f) != 0) {
                    const float alpha = exp2f(mrun[qt] - mnew);
                    mrun[qt] = mnew;
                    lacc[qt] *= alpha;
    #pragma unroll
                    for (int dt = 0; dt < 16; ++dt) oacc[qt][dt] *= alpha;
                }
                const float mref = mrun[qt];
    #pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    // v_exp_f32 directly: results below 2^-126 flush to zero, which a
                    // softmax weight relative to a max of at least 1 can ignore
                    float p[8];
    #pragma unroll
                    for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(s[qt][2 * h2 + (e >> 2)][e & 3] * cs - mref);
                    f16x8 ph;
    #pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const f16x2 hp = __builtin_convertvector(f32x2{p[e], p[e + 1]}, f16x2);
                        ph[e] = hp[0];
                        ph[e + 1] = hp[1];
                    }
                    pf[qt][h2] = ph;
                }
            }

            // O^T[d][query] += sum_key V^T[d][key] P^T[key][query]; V^T fragments one group of four
            // d-tiles ahead (two register slots), like the K fragments of S^T (one step ahead)
            f16x8 vf[2][4];
            auto load_vf = [&](int slot, int g) {  // g = 0..7: h2 = g >> 2, d-tiles 4 (g & 3) .. +3
                const int base = (g >> 2) ? vb1 : vb0;
    #pragma unroll
                for (int u = 0; u < 4; ++u)
                    vf[slot][u] =
                        __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(vl + base + (4 * (g & 3) + u) * 2048));
            };
            __builtin_amdgcn_s_setprio(1);
            load_vf(0, 0);
    #pragma unroll
            for (int g = 0; g < 8; ++g) {
                if (g + 1 < 8) load_vf((g + 1) & 1, g + 1);
                const int h2 = g >> 2;
    #pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int dt = 4 * (g & 3) + u;
    #pragma unroll
                    for (int qt = 0; qt < NQT; ++qt)
                        oacc[qt][dt] =
                            __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[g & 1][u], pf[qt][h2], oacc[qt][dt], 0, 0, 0);
                }
                if ((g & 3) == 3)
    #pragma unroll
                    for (int qt = 0; qt < NQT; ++qt)
                        lacc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[qt][h2], lacc[qt], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // Two LDS stages: tile e0 + t lives in stage t & 1; the loads of tile t + 1 run during the
        // compute of tile t; one barrier per tile.
        const int n = e1 - e0;
        // a wave whose 16 queries all lie past L (the last block when L is no multiple of 192) still
        // issues its share of the loads and meets every barrier, but computes nothing
        const bool active = q0 < L;
        ld.issue(st0, kw.key(e0));
        // the q fragments must have arrived here, before the barrier (otherwise the compiler moves
        // their loads behind it and the two latencies add up)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(qf[0][ks]));
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int t = 0; t < n; t += 2) {
            if (t + 1 < n) ld.issue(st1, kw.key(e0 + t + 1));
            if (active) compute(st0, kw.key(e0 + t));
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (t + 1 >= n) break;
            if (t + 2 < n) ld.issue(st0, kw.key(e0 + t + 2));
            if (active) compute(st1, kw.key(e0 + t + 1));
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }

        if (e0 == 0 && e1 == kw.nkt) {
            // the whole item: normalise and write o[b*L + query][h*256 + d]
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const float l = __shfl(lacc[qt][0], lr, 64);
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
        } else {
            // a piece: slot 2 g if it starts inside the item, else 2 g + 1 (it ends inside it)
            float* pb = part + (size_t)(2 * g + (e0 > 0 ? 0 : 1)) * kPartFloats;
            const float l = __shfl(lacc[0][0], lr, 64);
            const float inv = 1.0f / l;
#pragma unroll
            for (int dt = 0; dt < 16; ++dt) {
                const v4f v = oacc[0][dt] * inv;
                const f16x2 a = __builtin_convertvector(f32x2{v[0], v[1]}, f16x2);
                const f16x2 c = __builtin_convertvector(f32x2{v[2], v[3]}, f16x2);
                *reinterpret_cast<u32x2*>(pb + ((wave * 16 + dt) * 64 + lane) * 2) =
                    u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, c)};
            }
            if (lane < 16) *reinterpret_cast<f32x2*>(pb + kPartO + (wave * 16 + lane) * 2) = f32x2{mrun[0], l};
        }
    }
}

// Tail items split between neighbouring ranges: the boundary u_j = j Ut / G that lies inside an
// item and is that item's first inner boundary combines the item's pieces: the end piece of range j - 1 (slot 2 (j - 1) + 1) and the start
// pieces of the non-empty ranges j, j + 1, ... that begin inside the item (slots 2 j', in order).
// O = sum_s O_s 2^(m_s - m), l = sum_s l_s 2^(m_s - m), m = max_s m_s; o = O / l (each piece
// stores O_s / l_s).
// The boundaries j that merge an item: u_j lies inside the item and is its first inner boundary.
struct MergeList {
    uint16_t j[kAttnMaxGrid];
};
__host__ __device__ inline bool merges_at(int j, int G, int R, int64_t Ut, int Hn, int L, int T, const TextLens& lens,
                                          int varlen) {
    if (j < 1) return false;
    const int64_t uj = Ut * j / G;
    if (uj >= Ut) return false;
    const UnitPos pos = locate_tail(uj, R * G, Hn, L, T, lens, varlen);
    return uj != pos.first && Ut * (j - 1) / G <= pos.first;
}

// One 64-thread block per (merging boundary, wave slice of 16 queries): blockIdx.x indexes the
// list of merging boundaries, blockIdx.y is the slice.
__global__ __launch_bounds__(64) void attn_merge_kernel(const float* __restrict__ part, uint16_t* __restrict__ o,
                                                        int L, int H, int nqb, int T, TextLens lens, int varlen,
                                                        int R, int64_t Ut, int G, MergeList ml) {
    const int j = ml.j[blockIdx.x];
    const int64_t uj = Ut * j / G;
    const UnitPos pos = locate_tail(uj, R * G, H * nqb, L, T, lens, varlen);
    const int64_t item_end = pos.first + KeyWalk(L, T, varlen ? lens.len[pos.b] : T).nkt;

    const int lane = threadIdx.x, wave = blockIdx.y;
    const int lr = lane & 15, lg = lane >> 4;
    // the pieces: slot 2 (j - 1) + 1, then 2 j' for the non-empty ranges j' >= j starting inside the
    // item; combined in one pass with a running max, the next piece's loads issued before the
    // current one is added
    int jj = j;
    auto next_piece = [&]() -> const float* {
        while (jj < G && Ut * jj / G < item_end) {
            const int c = jj++;
            if (Ut * (c + 1) / G > Ut * c / G) return part + (size_t)(2 * c) * kPartFloats;
        }
        return nullptr;
    };
    struct Piece {
        f32x2 ml;
        u32x2 v[16];
    };
    auto load = [&](const float* pb, Piece& p) {
        p.ml = *reinterpret_cast<const f32x2*>(pb + kPartO + (wave * 16 + lr) * 2);
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) p.v[dt] = *reinterpret_cast<const u32x2*>(pb + ((wave * 16 + dt) * 64 + lane) * 2);
    };
    Piece cur, nxt;
    load(part + (size_t)(2 * (j - 1) + 1) * kPartFloats, cur);
    v4f acc[16];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) acc[dt] = v4f{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;
    for (bool more = true; more;) {
        const float* pn = next_piece();
        more = pn != nullptr;
        if (more) load(pn, nxt);
        // the piece holds O_s / l_s: it adds 2^(m_s - m) l_s times that to O
        const float mn = fmaxf(m, cur.ml[0]);
        const float a = exp2f(m - mn), w = exp2f(cur.ml[0] - mn) * cur.ml[1];
        m = mn;
        l = l * a + w;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
            // (through scalars: hipcc's bit_cast of a vector component reads component 0)
            const uint32_t bx = cur.v[dt].x, by = cur.v[dt].y;
            const f16x2 x = __builtin_bit_cast(f16x2, bx), y = __builtin_bit_cast(f16x2, by);
            const v4f v = {(float)x[0], (float)x[1], (float)y[0], (float)y[1]};
            acc[dt] = acc[dt] * a + w * v;
        }
        if (more) cur = nxt;
    }
    const int h = pos.it / nqb, qb = pos.it % nqb;
    const int qi = qb * kQB + wave * 16 + lr;
    if (qi < L) {
        const float inv = 1.0f / l;
        uint16_t* orow = o + ((int64_t)pos.b * L + qi) * (H * kD) + h * kD;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
            u32x2 w;
            w.x = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
            w.y = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
            *reinterpret_cast<u32x2*>(orow + dt * 16 + 4 * lg) = w;
        }
    }
}

}  // namespace

size_t attention_part_bytes() { return (size_t)2 * kAttnMaxGrid * kPartFloats * sizeof(float); }

hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* vt, uint16_t* o, int B, int L,
                            int H, int T, const TextLens* lens, float* part, int grid, hipStream_t st) {
    if (L == 0) return hipSuccess;
    if (grid < 0 || grid > kAttnMaxGrid) return hipErrorInvalidValue;
    const int Lp = padded_len(L);
    const int nqb = (L + kQB - 1) / kQB;

    TextLens tl{};
    if (lens) tl = *lens;
    const int Hn = H * nqb, items = B * Hn;
    if (grid == 0) {
        // one workgroup per item (no pieces)
        hipLaunchKernelGGL(attn_kernel, dim3(items), dim3(64 * kWaves), 0, st, q, k, vt, o, part, L, Lp, H, nqb, T, tl,
                           lens ? 1 : 0, 1, (int64_t)0);
        return hipGetLastError();
    }
    // R whole rounds of G items, then the Ut tile units of the remaining items split evenly
    const int R = items >= grid ? items / grid : 0;
    const int I0 = R * grid;
    int64_t Ut = 0;
    for (int b = I0 / Hn; b < B; ++b)
        Ut += (int64_t)(b == I0 / Hn ? (b + 1) * Hn - I0 : Hn) * KeyWalk(L, T, lens ? tl.len[b] : T).nkt;
    const int G = R > 0 ? grid : (int)std::min<int64_t>(grid, Ut);
    hipLaunchKernelGGL(attn_kernel, dim3(G), dim3(64 * kWaves), 0, st, q, k, vt, o, part, L, Lp, H, nqb, T, tl, lens ? 1 : 0,
                       R, Ut);
    if (G > 1 && Ut > 0) {
        MergeList ml;
        int nm = 0;
        for (int j = 1; j < G; ++j)
            if (merges_at(j, G, R, Ut, Hn, L, T, tl, lens ? 1 : 0)) ml.j[nm++] = (uint16_t)j;
        if (nm > 0)
            hipLaunchKernelGGL(attn_merge_kernel, dim3(nm, kWaves), dim3(64), 0, st, part, o, L, H, nqb, T, tl,
                               lens ? 1 : 0, R, Ut, G, ml);
    }
    return hipGetLastError();
}

}  // namespace sfm
