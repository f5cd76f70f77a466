// Internal declarations of the gfx950 DiT library: the context, device helpers
// shared by the kernels, and the host launchers each kernel file exports.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/sfm.h"

struct sfm_context {
    sfm_dims dims;
    int device;
    int max_pos;          // rows of the rotary tables: max_text + 128 image positions
    float* rope_cos;      // device [max_pos][64] fp32
    float* rope_sin;      // device [max_pos][64] fp32
    float nf4_code[16];   // NF4 codebook (fp32), passed to kernels by value
    int attn_grid = 0;    // attention workgroups: the device's compute units, at most 256
    float* attn_part = nullptr;  // partial results of the standalone attention calls
    void* scratch = nullptr;     // device address of the library's static scratch on `device`
    // the two passes of a CFG step run on these streams at once (default priority);
    // the fork / join events order them against the caller's stream, and the lock
    // keeps concurrent steps on one context from interleaving their use of them
    hipStream_t side[2] = {nullptr, nullptr};
    hipEvent_t fork = nullptr;
    hipEvent_t join[2] = {nullptr, nullptr};
    // host-streamed block weights: layer copies run on `copy` into two device
    // slots; copied[s] marks slot s filled, consumed[s] its block computed
    hipStream_t copy = nullptr;
    hipEvent_t copied[2] = {nullptr, nullptr};
    hipEvent_t consumed[2] = {nullptr, nullptr};
    hipEvent_t done = nullptr;
    std::mutex step_lock;
};

namespace sfm {

struct Nf4Code {
    float v[16];
};

// ------------------------------------------------------------------ device helpers
#if defined(__HIPCC__)

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Two fp32 -> two OCP E4M3 codes in the low (word 0) or high (word 1) half of
// `old`, hardware round-to-nearest-even.  Callers clamp to +-448 first.
template <bool HI>
__device__ __forceinline__ uint32_t cvt_fp8x2(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Sum over the 64 lanes of a wave without LDS: DPP rotations inside each
// row of 16 lanes, then the cross-row swaps (rows 0<->1, 2<->3, then halves).
__device__ __forceinline__ float dpp_ror(float x, int n) {
    switch (n) {
        case 8: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
        case 4: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, false));
        case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xF, 0xF, false));
        default: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xF, 0xF, false));
    }
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
    x += dpp_ror(x, 8);
    x += dpp_ror(x, 4);
    x += dpp_ror(x, 2);
    x += dpp_ror(x, 1);
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Reduction over a workgroup of NW waves through `red` (NW floats of LDS).
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) t += red[i];
    return t;
}

template <int NW>
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) red[w] = v;
    __syncthreads();
    float t = red[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) t = fmaxf(t, red[i]);
    return t;
}

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }

// Rotary position of row l of a sample whose text prefix has T rows, the first Tb of them
// real text, on one axis (0 t, 1 h, 2 w): text (and padding) rows l -> l on every axis,
// image token i = l - T at (Tb, Tb + i / gw, Tb + i % gw).
__device__ __forceinline__ int axis_pos(int l, int T, int Tb, int gw, int axis) {
    if (l < T) return l;
    const int i = l - T;
    if (axis == 0) return Tb;
    if (axis == 1) return Tb + i / gw;
    return Tb + i % gw;
}

// Position of token t (0..31, inside its group of 32) in the attention kernel's V^T rows:
// the stored order of a group is [4g..4g+3, 16+4g..16+4g+3] for g = 0..3.
__device__ __forceinline__ int vt_slot(int t) { return 8 * ((t & 15) >> 2) + 4 * (t >> 4) + (t & 3); }

#endif  // __HIPCC__

inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
inline int padded_len(int L) { return (int)round_up(L, 128); }

// Per-sample text lengths of a batch whose text prefixes are padded to T rows
// in memory: sample b's text is rows [0, len[b]) of its prefix, rows
// [len[b], T) are padding (masked as keys; their own outputs are unspecified)
// and its image positions start at len[b].  Passed to kernels by value.
constexpr int kMaxVarlenBatch = 64;
struct TextLens {
    int32_t len[kMaxVarlenBatch];
};

// Records a printf-style message for sfm_last_error (thread-local) and returns code.
int fail(int code, const char* fmt, ...);

// ------------------------------------------------------------------ launchers
// All launchers enqueue on `st` and return hipError_t of the launch.

// k_norm.hip
// out[b][n] = sum_k w[n][k] act(in[b][k]) + bias[n] (act SiLU when act_silu); B <= 8, k % 8 == 0
hipError_t launch_gemv(const float* in, int act_silu, const uint16_t* w, const float* bias, float* out, int B,
                       int n_out, int k, hipStream_t st);
// The same product for `layers` weight sets at once (one launch): layer l reads p.w[l], p.bias[l]
// (bias may be NULL) and writes out + l * out_stride.
constexpr int kGemvMaxLayers = 64;
struct GemvLayers {
    const uint16_t* w[kGemvMaxLayers];
    const float* bias[kGemvMaxLayers];
};
hipError_t launch_gemv_layers(const float* in, int act_silu, const GemvLayers& p, int layers, float* out,
                              int64_t out_stride, int B, int n_out, int k, hipStream_t st);
hipError_t launch_adaln_fp8(const uint16_t* x, int64_t rows_per_batch_in, int64_t row_off, int rows_per_batch,
                            const float* scale, int64_t scale_stride, uint8_t* hq, float* hs, int B, int D, float eps,
                            hipStream_t st);
hipError_t launch_adaln_bf16(const uint16_t* x, int64_t rows_per_batch_in, int64_t row_off, int rows_per_batch,
                             const float* scale, int64_t scale_stride, uint16_t* h, int B, int D, float eps,
                             hipStream_t st);
hipError_t launch_quant_rows(const uint16_t* a, int rows, int cols, uint8_t* q, float* s, hipStream_t st);
// h = bf16(x / sqrt(mean(x^2) + eps) * w) per fp32 row, then E4M3 codes + alpha/448; cols % 4 == 0, <= 65536
hipError_t launch_rmsnorm_f32_quant(const float* x, int rows, int cols, const uint16_t* w, uint8_t* q, float* s,
                                    float eps, hipStream_t st);
hipError_t launch_timestep_embed(float t, float* e, int B, int dim, hipStream_t st);

// k_gemm_fp8.hip
// shared: another pass's kernels run on the GPU at the same time and fill the last round of
// tiles, so the tile shape is chosen by main-loop efficiency alone (else by whole rounds too)
hipError_t launch_gemm_fp8(int epi, const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                           uint16_t* out, const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N,
                           int K, int L, hipStream_t st, bool shared = false);
// MXFP4 weights: w packed E2M1 nibbles [N][K/2] (element 2i in the low nibble), wexp E8M0
// exponents [N][K/32]; FP8 activation codes as for launch_gemm_fp8; K % 256 == 0
hipError_t launch_gemm_mx(int epi, const uint8_t* a, const float* sa, const uint8_t* w, const uint8_t* wexp,
                          uint16_t* out, const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N,
                          int K, int L, hipStream_t st, bool shared = false);
// Split-K FP8 STORE projection for few rows and long K (few output tiles): splitk_parts(M, N, K)
// parts of fp32 partial sums in `part` ([parts][M][N]), then a reduce applying sa, sw and the
// bf16 rounding.  1 part means the plain launch would fill the chip as well.
int splitk_parts(int M, int N, int K);
hipError_t launch_gemm_fp8_splitk(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* out,
                                  int M, int N, int K, float* part, hipStream_t st);

// QKV projection whose epilogue applies QK-RMSNorm (weights qn, kn) and the rotary
// embedding and writes q, k [B][H][Lp][256] (bf16) and V^T [B][H][256][Lp] (fp16, keys in the
// stored order of vt_slot) directly, in place of the STORE projection + launch_qk_norm_rope.
// N = 3 H 256 (q heads, k heads, v heads); rows past each sample's L are not written.
struct RopeArgs {
    uint16_t* q;
    uint16_t* k;
    uint16_t* vt;
    const uint16_t* qn;
    const uint16_t* kn;
    const float* cos_t;
    const float* sin_t;
    int T, gw, Lp, H;
    float eps;
    int varlen;
    TextLens lens;
};
hipError_t launch_gemm_fp8_qkv_rope(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, int M,
                                   int K, int L, const RopeArgs& ra, hipStream_t st);

// k_gemm_nf4.hip
hipError_t launch_gemm_nf4(int epi, const uint16_t* a, const uint8_t* w, const float* absmax, const Nf4Code& code,
                           uint16_t* out, const uint16_t* resid, const float* gate, int64_t gate_stride, int M, int N,
                           int K, int L, hipStream_t st);
// The NF4 QKV projection (bf16 activation a [M][K]) with the same fused QK-RMSNorm + rotary
// epilogue and outputs as launch_gemm_fp8_qkv_rope.
hipError_t launch_gemm_nf4_qkv_rope(const uint16_t* a, const uint8_t* w, const float* absmax, const Nf4Code& code,
                                    int M, int K, int L, const RopeArgs& ra, hipStream_t st);

// k_rope.hip
// lens: per-sample text lengths (image positions start at len[b]), or NULL when every sample has T
hipError_t launch_qk_norm_rope(const uint16_t* qkv, const uint16_t* qn, const uint16_t* kn, const float* cos_t,
                               const float* sin_t, uint16_t* q, uint16_t* k, uint16_t* vt, int B, int T, int gh,
                               int gw, int H, float eps, const TextLens* lens, hipStream_t st);
// Zeroes the padding rows [L, Lp) of q and k and the padding columns of V^T (nothing when
// Lp == L): the attention kernel multiplies V^T's padding by zero weights, so it must be finite.
hipError_t launch_attn_pad_zero(uint16_t* q, uint16_t* k, uint16_t* vt, int B, int L, int H, hipStream_t st);

// k_attn.hip
// Attention runs as `grid` persistent workgroups (at most kAttnMaxGrid; one per compute unit)
// that split the work evenly; items shared between workgroups leave partial results in `part`
// (attention_part_bytes() bytes, private to the launch's stream until the launch completes).
// grid 0: one workgroup per (batch, head, query block), no partial results.
constexpr int kAttnMaxGrid = 256;
size_t attention_part_bytes();
// lens: per-sample text lengths of the T-row text prefixes (keys [len[b], T) masked), or NULL for none
hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* vt, uint16_t* o, int B, int L,
                            int H, int T, const TextLens* lens, float* part, int grid, hipStream_t st);

// k_misc.hip
hipError_t launch_euler_cfg(const float* z, const float* vc, const float* vu, float* zo, float* vo, int64_t n,
                            float g, float dt, hipStream_t st);
hipError_t launch_dequant_fp8(const uint8_t* q, const float* s, void* out, int out_bf16, int n, int k,
                              hipStream_t st);
hipError_t launch_dequant_mx(const uint8_t* q, const uint8_t* ex, void* out, int out_bf16, int n, int k,
                             hipStream_t st);
hipError_t launch_dequant_nf4(const uint8_t* q, const float* absmax, const Nf4Code& code, void* out, int out_bf16,
                              int n, int k, hipStream_t st);
// out[m][n] = sum_k a[m][k] w[n][k] + bias[n]; a fp32 or bf16, w bf16, out bf16 or fp32.
// Row m of `a` is read at a_row(m) = (m / a_rpb) * a_bstride + a_off + m % a_rpb, same for out.
hipError_t launch_small_linear(const void* a, int a_bf16, int64_t a_rpb, int64_t a_bstride, int64_t a_off,
                               const uint16_t* w, const float* bias, void* out, int out_bf16, int64_t o_rpb,
                               int64_t o_bstride, int64_t o_off, int M, int N, int K, hipStream_t st);
hipError_t launch_copy_rows(const uint16_t* src, int64_t src_rpb, uint16_t* dst, int64_t dst_rpb, int B,
                            int rows, int cols, hipStream_t st);

}  // namespace sfm
