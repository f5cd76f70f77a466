/*
 * sfm.h - C ABI of the MI355X (gfx950) Ideogram-4 single-stream DiT library.
 *
 * The library computes the forward pass of one single-stream DiT block on the
 * joint [text | image-latent] token sequence, the 34-block velocity model, and
 * one Euler flow-matching step with asymmetric classifier-free guidance
 * (Ideogram 4.0 research note, "Model architecture" and "Training method").
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned device memory (for example from a
 *     PyTorch tensor's data_ptr()).  Host pointers are marked "host".
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.  All
 *     device work is enqueued asynchronously on that stream; nothing blocks
 *     the host.  The caller synchronises before reading results.
 *   - Return value: SFM_OK (0) or a negative sfm_status.  Every argument,
 *     shape, alignment and workspace check runs before the first enqueue, so an
 *     error leaves no partial work behind.  sfm_last_error() gives a
 *     thread-local message for the last failure.
 *   - Device pointers must be 16-byte aligned.
 *   - The library allocates no device memory per call.  Workspaces are passed
 *     in; size them with the *_workspace_bytes() queries.  Calls that share a
 *     workspace must be ordered on one stream.
 *   - bf16 tensors are passed as uint16_t bit patterns; FP8 tensors as uint8_t
 *     OCP E4M3FN codes (bias 7, max 448, no infinities).
 *
 * Row-major layouts throughout.  Notation: B batch, T text tokens, gh x gw
 * image grid, L = T + gh*gw, M = B*L, D = emb_dim, H = num_heads, d = 256,
 * F = intermediate, A = adaln_dim, C = latent channels.
 */
#ifndef SFM_H
#define SFM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sfm_status {
    SFM_OK = 0,
    SFM_E_INVALID_ARG = -1, /* null pointer, unknown enum value, bad scalar */
    SFM_E_SHAPE = -2,       /* dims or sequence shape outside the supported set */
    SFM_E_WORKSPACE = -3,   /* workspace missing or smaller than required */
    SFM_E_ARCH = -4,        /* device is not gfx950 */
    SFM_E_ALIGN = -5,       /* a device pointer is not 16-byte aligned */
    SFM_E_DEVICE = -6       /* a HIP runtime call failed */
} sfm_status;

/* Model shape.  Ideogram 4.0 research note, "Model architecture", spec table:
 * emb_dim 4608, 18 heads of 256, SwiGLU intermediate 12288, adaln_dim 512,
 * rope_theta 5e6, mrope_section (24, 20, 20), 128 latent channels, text up to
 * 2048 tokens.  rope_dims is the number of rotated dims per head (the first
 * 128 as 64 pairs); eps is the RMSNorm epsilon (1e-6). */
typedef struct sfm_dims {
    int32_t emb_dim, num_heads, head_dim, intermediate, adaln_dim, latent_ch;
    int32_t rope_dims, mrope_section[3], max_text;
    float rope_theta, eps;
} sfm_dims;

/* The spec-table shape, and the tiny shape (emb 512 = 2 x 256, F 1536) used by
 * quick tests.  Pure host functions. */
sfm_dims sfm_dims_ideogram4(void);
sfm_dims sfm_dims_tiny(void);

typedef struct sfm_context sfm_context;

/* Create a context on HIP device `device`: checks that the device is gfx950
 * (else SFM_E_ARCH), and uploads the constant tables - the MRoPE cos/sin
 * table for every integer position the shape limits allow, built on the host
 * in double precision and rounded to fp32, and the NF4 codebook.  Only
 * emb_dim = num_heads * 256 with head_dim 256, rope_dims 128 and
 * mrope_section (24, 20, 20) are supported (else SFM_E_SHAPE).  It also creates
 * the two streams and three events on which sfm_cfg_step runs its two passes
 * side by side.  The tables never change afterwards and the context may be
 * shared by threads. */
int sfm_context_create(const sfm_dims* dims, int device, sfm_context** out);
void sfm_context_destroy(sfm_context* ctx);

/* Host-only shape check (no HIP call): T in [0, max_text]; gh, gw in [1, 128];
 * for the spec shape also gh, gw >= 16 (256 px) and max/min aspect <= 6
 * (research note spec table: 256-2048 px per side, multiples of 16, aspect up
 * to 6:1); B >= 1.  Returns SFM_OK or SFM_E_SHAPE. */
int sfm_check_shape(const sfm_dims* dims, int B, int T, int gh, int gw);

/* Host helper: MRoPE positions for the joint sequence into pos_host[L][3]
 * (t, h, w).  Text token i -> (i, i, i); image token (r, c), row-major ->
 * (T, T + r, T + c) (research note, "Model architecture": 1-D text positions
 * broadcast to three axes, image tokens at (t, h, w)). */
int sfm_positions(int T, int gh, int gw, int32_t* pos_host);

/* ---------------------------------------------------------------- weights */

typedef enum sfm_wfmt {
    SFM_W_FP8_E4M3 = 1, /* q: uint8 E4M3 codes [n][k]; scale: fp32 [n] per output channel */
    SFM_W_NF4_B64 = 2,  /* q: uint8 [n][k/2] nibbles (element 2i = high nibble of byte i);
                           scale: fp32 absmax [n*k/64], one per 64 consecutive elements */
    SFM_W_MXFP4 = 3     /* q: uint8 [n][k/2] E2M1 nibbles (element 2i = LOW nibble of byte i);
                           scale: uint8 E8M0 exponents [n][k/32], one per 32 consecutive elements */
} sfm_wfmt;

/* A quantised weight W[n][k] (out x in).  FP8: w = decode(q) * scale[n]
 * (deployment post, section 2: original release FP8 E4M3).  NF4: w =
 * fp32(code[q] * absmax[block]) with the 16-level normal-quantile codebook
 * (deployment post, section 2.1: NF4, block size 64).  MXFP4: w = e2m1(q) *
 * 2^(e - 127), the OCP microscaling form of the 4-bit float FFN weights of the
 * deployment post's mixed scheme (section 2.2); its products run on FP8 x FP4
 * matrix cores with the activation quantised per token to E4M3, as for FP8.
 * `scale` points to fp32 values for FP8 and NF4 and to uint8 exponents for
 * MXFP4. */
typedef struct sfm_qweight {
    int32_t fmt, n, k;
    const void* q;
    const void* scale;
} sfm_qweight;

/* One block's weights.  qkv [3D][D] (rows: q heads, k heads, v heads, head h
 * at rows h*256..h*256+255 of each part); o [D][D]; gate_up [2F][D] (gate rows
 * [0, F), up rows [F, 2F)); down [D][F].  All four in one format, or "mixed"
 * (deployment post, section 2.2): qkv and o FP8, gate_up and down MXFP4.  q_norm,
 * k_norm: bf16 [256] QK-RMSNorm weights shared by the heads.  mod_w bf16
 * [4D][A], mod_b fp32 [4D]: AdaLN map from the timestep embedding to
 * (scale_attn, gate_attn, scale_mlp, gate_mlp). */
typedef struct sfm_block_weights {
    sfm_qweight qkv, o, gate_up, down;
    const uint16_t* q_norm;
    const uint16_t* k_norm;
    const uint16_t* mod_w;
    const float* mod_b;
} sfm_block_weights;

/* Velocity-model weights.  blocks: host array of num_layers block weights,
 * FP8 or mixed (FP8 attention projections, MXFP4 FFN; every layer with the
 * FFN format of layer 0).  x_w bf16 [D][C], x_b fp32 [D]: latent-to-token embedding.  t_w1,
 * t_w2 bf16 [A][A], t_b1, t_b2 fp32 [A]: timestep MLP.  f_mod_w bf16 [D][A],
 * f_mod_b fp32 [D]: final-layer AdaLN scale.  f_w bf16 [C][D], f_b fp32 [C]:
 * projection back to latent channels. */
typedef struct sfm_model_weights {
    int32_t num_layers;
    const sfm_block_weights* blocks;
    const uint16_t* x_w;
    const float* x_b;
    const uint16_t* t_w1;
    const float* t_b1;
    const uint16_t* t_w2;
    const float* t_b2;
    const uint16_t* f_mod_w;
    const float* f_mod_b;
    const uint16_t* f_w;
    const float* f_b;
} sfm_model_weights;

/* ------------------------------------------------------- step-level entry points */

/* Modulation (research note, "Model architecture": the timestep embedding
 * generates per-block scale and gate): mod[b][n] = sum_j w[n][j] *
 * SiLU(c[b][j]) + bias[n].  w bf16 [n_out][A], bias fp32 [n_out], c fp32
 * [B][A], mod fp32 [B][n_out]. */
int sfm_modulation(const sfm_context* ctx, const uint16_t* w, const float* bias, const float* c,
                   float* mod, int B, int n_out, void* stream);

/* AdaLN RMSNorm (research note, AdaLN modulates the residual paths):
 * h = bf16(x / sqrt(mean(x^2) + eps) * (1 + scale[b])) per row of x bf16
 * [B*L][D]; scale[b] = mod + b*mod_batch_stride (D fp32 values).
 * FP8 form: writes the per-token E4M3 quantisation of h - codes hq [B*L][D]
 * and hs[m] = amax(h[m]) / 448 (fp32) - as the next FP8 GEMM's input.
 * bf16 form: writes h itself (bf16 [B*L][D]) for the NF4 path. */
int sfm_adaln_norm_fp8(const sfm_context* ctx, const uint16_t* x, const float* scale, int64_t mod_batch_stride,
                       uint8_t* hq, float* hs, int B, int L, void* stream);
int sfm_adaln_norm_bf16(const sfm_context* ctx, const uint16_t* x, const float* scale, int64_t mod_batch_stride,
                        uint16_t* h, int B, int L, void* stream);

/* Per-token E4M3 quantisation of bf16 rows a [rows][cols]: alpha = max|a|,
 * q = e4m3_rne_sat(fp32(a * fp32(448 / alpha))), s = alpha / 448; zero rows
 * give zero codes and s = 0.  cols % 8 == 0. */
int sfm_quant_rows_fp8(const uint16_t* a, int rows, int cols, uint8_t* q, float* s, void* stream);

typedef enum sfm_epilogue {
    SFM_EPI_STORE = 0,      /* out bf16 [M][n] = bf16(y) */
    SFM_EPI_RESID_GATE = 1, /* out bf16 [M][n] = bf16(resid + gate[b] * y); out may equal resid */
    SFM_EPI_SWIGLU = 2      /* out bf16 [M][n/2] = bf16(silu(y[:, :n/2]) * y[:, n/2:]) */
} sfm_epilogue;

/* Projection y = A W^T with a fused epilogue (research note block internals:
 * QKV / output projections, SwiGLU MLP, gated residual).
 * FP8 weights: a = E4M3 codes [M][k] with per-row scale a_scale [M] (as made by
 * sfm_adaln_norm_fp8 / sfm_quant_rows_fp8); y = (sum dec(a) dec(q)) *
 * a_scale[m] * w.scale[n], FP8 x FP8 matrix cores, fp32 accumulation.
 * NF4 weights: a = bf16 [M][k], a_scale unused; y = a * bf16(w)^T on bf16
 * matrix cores, the NF4 decode fused into the weight-operand load.
 * gate: fp32, row b of the batch at gate + b*gate_batch_stride (n values);
 * L gives the batch of a row (b = m / L); with the gated residual and rows in
 * more than one batch (M > L), L >= 128.  k % 256 == 0, n % 256 == 0 and
 * n * k < 2^31 (SFM_E_SHAPE otherwise); M is limited only by int range. */
int sfm_linear(const sfm_context* ctx, int epilogue, const void* a, const float* a_scale, const sfm_qweight* w,
               uint16_t* out, const uint16_t* resid, const float* gate, int64_t gate_batch_stride, int M, int L,
               void* stream);

/* Padded sequence length used by the attention layouts: L rounded up to 128. */
int sfm_padded_len(int L);

/* QK-RMSNorm + 3-D MRoPE (research note block internals: QK-RMSNorm and MRoPE
 * with mrope_section (24, 20, 20), rope_theta 5e6).  Input qkv bf16
 * [B*L][3D] as written by the QKV projection.  Per token and head:
 * u = u / sqrt(mean(u^2) + eps) * gamma, then pairs (j, j+64), j < 64, rotate
 * by pos[axis(j)] * theta^(-j/64) with axis t for j < 24, h for j < 44, w
 * otherwise; dims 128..255 pass through; result rounded to bf16.
 * Outputs (Lp = sfm_padded_len(L)): q, k bf16 [B][H][Lp][256]; vt fp16
 * [B][H][256][Lp] (v transposed; the bf16 values of v are exact in fp16 down
 * to 2^-17, values beyond +-65504 saturate).  Inside every aligned group of 32
 * tokens vt stores the tokens in the order 4g..4g+3, 16+4g..16+4g+3 for
 * g = 0..3 (the attention kernel's operand order).  Padding rows / columns are
 * written as zeros. */
int sfm_qk_norm_rope(const sfm_context* ctx, const uint16_t* qkv, const uint16_t* q_norm, const uint16_t* k_norm,
                     uint16_t* q, uint16_t* k, uint16_t* vt, int B, int T, int gh, int gw, void* stream);

/* The QKV projection and sfm_qk_norm_rope in one kernel: the projection of a
 * by w ([3D][D]: q, k, v heads of 256), each output rounded to bf16 as
 * sfm_linear's STORE epilogue would, then QK-RMSNorm with q_norm / k_norm and
 * the 3-D MRoPE
 * exactly as sfm_qk_norm_rope defines them (research note block internals),
 * written straight to q, k [B][H][Lp][256] (bf16) and vt [B][H][256][Lp]
 * (fp16, sfm_qk_norm_rope's stored key order); padding rows / columns are
 * written as zeros.  text_lens: host array of B per-sample text lengths in
 * [0, T] (the positions of sfm_qk_norm_rope_varlen), or NULL when every sample
 * has T.  The row's sum of squares adds in another order than the separate
 * kernel's, so q and k can differ from sfm_linear + sfm_qk_norm_rope in the
 * last bf16 place; v is the same bit for bit.  Weight formats: FP8 (a: E4M3
 * codes [B*L][D] with row scales a_scale [B*L]) or NF4 block 64 (deployment
 * post, section 2.1: a is bf16 [B*L][D], a_scale is ignored and may be NULL).
 * Errors as sfm_linear and sfm_qk_norm_rope (w must be FP8 or NF4 with
 * n = 3 emb_dim, k = emb_dim). */
int sfm_qkv_rope(const sfm_context* ctx, const void* a, const float* a_scale, const sfm_qweight* w,
                 const uint16_t* q_norm, const uint16_t* k_norm, uint16_t* q, uint16_t* k, uint16_t* vt, int B, int T,
                 int gh, int gw, const int32_t* text_lens, void* stream);

/* Full bidirectional softmax attention over the joint sequence, scale 1/16, no
 * mask (research note: one shared self-attention over text + image tokens).
 * q, k bf16 [B][H][Lp][256], vt fp16 [B][H][256][Lp] as made by
 * sfm_qk_norm_rope; o bf16 [B*L][D], head h at columns h*256.. .  Scores in
 * fp32 from bf16 q k^T; the P V product in fp16 with fp32 accumulation.
 * The (batch, head, 128-query block, 64-key tile) units are split evenly over
 * one workgroup per compute unit; a query block shared by two workgroups is
 * finished by a second kernel from fp32 partial results that this call keeps
 * in a buffer owned by the context, so sfm_attention / sfm_attention_varlen
 * calls on one context must not overlap in time (the block, model and step
 * calls keep theirs in the caller's workspace instead). */
int sfm_attention(const sfm_context* ctx, const uint16_t* q, const uint16_t* k, const uint16_t* vt, uint16_t* o,
                  int B, int L, void* stream);

/* Euler update with asymmetric CFG (research note, "Training method": Euler
 * integration z_{t-dt} = z_t + v dt; deployment post 1.3: CFG scale 4.0):
 * v = v_u + guidance * (v_c - v_u); z_out = z + dt * v, fp32, n elements.
 * z_out may equal z; v_out may be NULL. */
int sfm_euler_cfg(const float* z, const float* v_c, const float* v_u, float* z_out, float* v_out, int64_t n,
                  float guidance, float dt, void* stream);

/* Dequantise a weight to out [n][k]: out_dtype 0 = fp32, 1 = bf16 (RNE of the
 * fp32 value).  FP8: fp32(decode(q) * scale[n]); NF4: fp32(code[q] *
 * absmax[block]); MXFP4: e2m1(q) * 2^(e - 127) (exact in fp32 and bf16).
 * Bit-exact by definition. */
int sfm_dequant(const sfm_context* ctx, const sfm_qweight* w, void* out, int out_dtype, void* stream);

/* --------------------------------------------------------- block / model / step */

/* Workspace bytes for sfm_block_forward with the given shape and weight format. */
size_t sfm_block_workspace_bytes(const sfm_context* ctx, int B, int T, int gh, int gw, int wfmt);

/* One DiT block (research note block internals), in place allowed
 * (x_out may equal x_in):
 *   mod = W_mod SiLU(c) + b_mod;                      (scale_a, gate_a, scale_m, gate_m)
 *   h = AdaLN(x, scale_a); q,k,v = h W_qkv^T; q,k = MRoPE(QKNorm(q,k));
 *   o = attention(q, k, v); x1 = x + gate_a * (o W_o^T);
 *   h2 = AdaLN(x1, scale_m); s = silu(h2 W_g^T) * (h2 W_u^T); x2 = x1 + gate_m * (s W_d^T)
 * with bf16 storage of every activation.  x bf16 [B][L][D], c fp32 [B][A]. */
int sfm_block_forward(const sfm_context* ctx, const sfm_block_weights* w, const uint16_t* x_in, uint16_t* x_out,
                      const float* c, int B, int T, int gh, int gw, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for sfm_model_velocity / sfm_cfg_step. */
size_t sfm_step_workspace_bytes(const sfm_context* ctx, int B, int T, int gh, int gw);

/* Velocity of the single-stream DiT (research note, "Training method": the
 * DiT predicts the flow-matching velocity).  text bf16 [B][T][D] (projected
 * 4608-d features; NULL when T == 0), latent fp32 [B][gh*gw][C], t host
 * scalar time for the whole batch.  c = W2 SiLU(W1 e(t) + b1) + b2 with
 * e(t) = [cos(1000 t f_i), sin(1000 t f_i)], f_i = 10000^(-i/(A/2));
 * x = [text | bf16(latent W_x^T + b_x)]; num_layers blocks; v = bf16(RMSNorm(x_img)
 * (1 + W_fm SiLU(c) + b_fm)) W_f^T + b_f.  v_out fp32 [B][gh*gw][C]. */
int sfm_model_velocity(const sfm_context* ctx, const sfm_model_weights* mw, const uint16_t* text,
                       const float* latent, float t, float* v_out, int B, int T, int gh, int gw, void* ws,
                       size_t ws_bytes, void* stream);

/* One guided Euler step: v_c from the conditional model on [text | image],
 * v_u from the separate unconditional model on the image tokens only (T = 0,
 * positions (0, r, c)) (research note, "Training method": asymmetric CFG drops
 * the text tokens from the unconditional pass), then sfm_euler_cfg.
 * z_out may equal z; v_c_out / v_u_out may be NULL (then workspace is used).
 * The two passes are independent and run at the same time on two streams the
 * context owns; events order them after the work already on `stream` and the
 * Euler update after both, so the call behaves as if it ran on `stream` alone.
 * Calls on one context from several threads enqueue one after the other. */
int sfm_cfg_step(const sfm_context* ctx, const sfm_model_weights* cond, const sfm_model_weights* uncond,
                 const uint16_t* text, const float* z, float* z_out, float t, float dt, float guidance, int B,
                 int T, int gh, int gw, float* v_c_out, float* v_u_out, void* ws, size_t ws_bytes, void* stream);

/* sfm_cfg_step with launch timing, for measuring the matrix kernels inside a
 * timed step.  ev_begin[i] / ev_end[i] are HIP events (hipEvent_t, created and
 * owned by the caller) recorded on `stream` immediately before and after the
 * i-th matrix launch of the step, for i < n_events; later launches are not
 * bracketed.  Every block contributes five launches in this order: QKV
 * projection, attention, output projection, gate/up projection, down
 * projection; the conditional pass's layers come first, then the
 * unconditional pass's (pair (p * layers + l) * 5 + j for pass p, layer l,
 * launch j).  The two passes run one after the other on `stream` here, so
 * that each bracketed launch has the GPU to itself, and every kernel takes the
 * launch shape it uses when it runs alone (as in sfm_block_forward: attention
 * on one persistent workgroup per compute unit, projection tiles chosen by
 * whole rounds of workgroups); sfm_cfg_step's concurrent passes instead take
 * the shapes that share the GPU best.  *n_recorded (if not NULL) receives the number of
 * pairs recorded.  Errors as sfm_cfg_step, plus SFM_E_INVALID_ARG for NULL
 * events. */
int sfm_cfg_step_timed(const sfm_context* ctx, const sfm_model_weights* cond, const sfm_model_weights* uncond,
                       const uint16_t* text, const float* z, float* z_out, float t, float dt, float guidance, int B,
                       int T, int gh, int gw, float* v_c_out, float* v_u_out, void* ws, size_t ws_bytes, void* stream,
                       void* const* ev_begin, void* const* ev_end, int n_events, int* n_recorded);

/* ---------------------------------------------------------------- host-streamed weights */

/* Workspace bytes of sfm_model_velocity_streamed: a velocity-model workspace
 * plus two device slots for one block's FP8 weights each (~274 MB at the spec
 * dims); a slot also holds a mixed block (its MXFP4 FFN weights are smaller),
 * of which only the block's own bytes are copied. */
size_t sfm_streamed_workspace_bytes(const sfm_context* ctx, int B, int T, int gh, int gw);

/* sfm_model_velocity with the blocks' weights in host memory (SimpleTuner
 * Ideogram 4 quick start, "Validation": the unconditional transformer can be
 * kept in CPU memory and its layers streamed to the accelerator on every
 * forward pass, trading speed for device memory).  Every pointer of
 * mw->blocks[i] points to host memory, pinned (hipHostMalloc) for the copies
 * to overlap the computation; the other weights of mw are device memory.
 * Blocks may be FP8 or mixed (MXFP4 FFN), all layers alike.
 * Block i + 1's weights are copied into one of two workspace slots on a
 * context-owned copy stream while block i computes from the other; results
 * equal sfm_model_velocity's bitwise.  Calls on one context are serialised.
 * Errors as sfm_model_velocity. */
int sfm_model_velocity_streamed(const sfm_context* ctx, const sfm_model_weights* mw, const uint16_t* text,
                                const float* latent, float t, float* v_out, int B, int T, int gh, int gw, void* ws,
                                size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- variable text lengths */

/* Batches of prompts with different text lengths.  The text prefixes are
 * padded to T rows in memory ([B][T + gh*gw][D] as everywhere); text_lens is
 * a host array of B values in [0, T] (B <= 64): sample b's text is rows
 * [0, text_lens[b]) of its prefix, rows [text_lens[b], T) are padding.  Each
 * sample's text and image rows come out as if the sample ran alone with its
 * own text_lens[b] text tokens: its image positions start at text_lens[b]
 * (research note, "Model architecture": image tokens at (t, h, w) after the
 * 1-D text positions) and attention masks the padding keys (key tiles wholly
 * inside the padding are skipped).  Padding rows' own outputs are unspecified
 * (finite for finite inputs).  Errors as the uniform calls, plus SFM_E_SHAPE
 * for a length outside [0, T] or B > 64 and SFM_E_INVALID_ARG for NULL
 * text_lens.  Workspaces are those of the uniform calls. */
int sfm_qk_norm_rope_varlen(const sfm_context* ctx, const uint16_t* qkv, const uint16_t* q_norm,
                            const uint16_t* k_norm, uint16_t* q, uint16_t* k, uint16_t* vt, int B, int T,
                            const int32_t* text_lens, int gh, int gw, void* stream);
/* L = T + image tokens per sample; requires T < L. */
int sfm_attention_varlen(const sfm_context* ctx, const uint16_t* q, const uint16_t* k, const uint16_t* vt, uint16_t* o,
                         int B, int L, int T, const int32_t* text_lens, void* stream);
int sfm_block_forward_varlen(const sfm_context* ctx, const sfm_block_weights* w, const uint16_t* x_in,
                             uint16_t* x_out, const float* c, int B, int T, const int32_t* text_lens, int gh, int gw,
                             void* ws, size_t ws_bytes, void* stream);
int sfm_model_velocity_varlen(const sfm_context* ctx, const sfm_model_weights* mw, const uint16_t* text,
                              const int32_t* text_lens, const float* latent, float t, float* v_out, int B, int T,
                              int gh, int gw, void* ws, size_t ws_bytes, void* stream);
/* The lengths apply to the conditional pass; the unconditional pass has no text. */
int sfm_cfg_step_varlen(const sfm_context* ctx, const sfm_model_weights* cond, const sfm_model_weights* uncond,
                        const uint16_t* text, const int32_t* text_lens, const float* z, float* z_out, float t, float dt,
                        float guidance, int B, int T, int gh, int gw, float* v_c_out, float* v_u_out, void* ws,
                        size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- text conditioning */

/* Workspace bytes of sfm_text_project for M tokens of k_raw features (with
 * room for the fp32 partial sums of a split-K projection when M is small). */
size_t sfm_text_project_workspace_bytes(const sfm_context* ctx, int M, int k_raw);

/* Projected text conditioning from raw text-encoder features (SimpleTuner
 * Ideogram 4 quick start, "Text embed cache": the text encoder concatenates 13
 * Qwen hidden states, 13 * 4096 = 53,248 fp32 values per token, and the
 * transformer's frozen llm_cond_norm and llm_cond_proj project them to the
 * conditioning the blocks consume).  text_out[m] = bf16(FP8 linear(bf16(
 * raw[m] / sqrt(mean(raw[m]^2) + eps) * norm_w))): RMSNorm with a weight,
 * then a projection without bias, its input quantised per token to E4M3 like
 * every FP8 projection.  raw fp32 [M][k] (row-major), norm_w bf16 [k],
 * proj FP8 [emb_dim][k] with per-channel scales, text_out bf16 [M][emb_dim].
 * k = proj->k must be a multiple of 256 in [256, 65536].  M rows are
 * independent (batch and tokens flattened).  With few rows (a prompt) the
 * projection splits K over up to 8 workgroups per output tile and reduces the
 * fp32 partial sums before the scales and the bf16 rounding.  Errors: SFM_E_INVALID_ARG (NULL
 * or non-FP8 weight), SFM_E_SHAPE, SFM_E_WORKSPACE, SFM_E_ALIGN, SFM_E_DEVICE. */
int sfm_text_project(const sfm_context* ctx, const float* raw, const uint16_t* norm_w, const sfm_qweight* proj,
                     uint16_t* text_out, int M, void* ws, size_t ws_bytes, void* stream);

/* sfm_text_project for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The E4M3 codes, row scales and split-K partial sums live in a fixed device
 * scratch of 128 MiB that the library holds on each GPU it runs on until the
 * process ends; its device address is looked up once per device when a
 * context is created.  Accepts every (M, k) whose
 * sfm_text_project_workspace_bytes is at most 128 MiB (any prompt of up to
 * 2048 tokens at 53,248 features); larger: SFM_E_WORKSPACE before any enqueue.
 * Allocates nothing and calls no allocating routine.  The scratch keeps the
 * last call's contents and every call on one GPU uses it: calls that overlap
 * in time on one GPU (different streams or threads) race and give undefined
 * results, so order them on one stream.  Results equal sfm_text_project's
 * bitwise (the same kernels).  Errors as sfm_text_project, plus SFM_E_DEVICE
 * when the context holds no scratch address. */
int sfm_text_project_noalloc(const sfm_context* ctx, const float* raw, const uint16_t* norm_w,
                             const sfm_qweight* proj, uint16_t* text_out, int M, void* stream);

/* ---------------------------------------------------------------- sampler */

/* Time grid of the logit-normal schedule (research note, "Training method":
 * logit-normal noise schedule with parameters (mu, std), mu shifted by
 * 0.5 * ln(num_pixels / 512^2) with the image size).  Writes n_steps + 1 host
 * doubles t_out[i] = sigmoid(mu' + std * Phi^-1(1 - i / n_steps)): t_out[0] = 1
 * (noise), t_out[n_steps] = 0 (clean), strictly decreasing (the quantiles of
 * the shifted distribution at evenly spaced probabilities; the pages name the
 * distribution, not the grid).  Host only.  SFM_E_INVALID_ARG for n_steps < 1,
 * NULL t_out, num_pixels < 1, non-finite mu / std or std <= 0. */
int sfm_time_grid(int n_steps, double mu, double std_dev, int64_t num_pixels, double* t_out);

/* Presets of the research note, "Infra": steps, the number at the main
 * guidance weight (the rest are polish steps at the lower weight), and the
 * schedule's (mu, std). */
enum {
    SFM_PRESET_V4_QUALITY_48 = 0, /* 48 steps: 45 at 7, 3 at 3; mu 0.0, std 1.5 */
    SFM_PRESET_V4_DEFAULT_20 = 1, /* 20 steps: 18 at 7, 2 at 3; mu 0.0, std 1.75 */
    SFM_PRESET_V4_TURBO_12 = 2    /* 12 steps: 11 at 7, 1 at 3; mu 0.5, std 1.75 */
};
typedef struct sfm_preset_info {
    int32_t n_steps, n_main;
    float guidance_main, guidance_polish;
    double mu, std_dev;
} sfm_preset_info;
int sfm_preset(int preset, sfm_preset_info* out);

/* A preset at an image size: t_out[0 .. n] (sfm_time_grid with the preset's
 * mu / std and height_px * width_px pixels) and guidance_out[0 .. n - 1]
 * (main weight, then the polish weight), both host arrays with room for
 * `capacity` >= n steps.  Returns n > 0, or a negative SFM_E_* status. */
int sfm_preset_schedule(int preset, int height_px, int width_px, double* t_out, float* guidance_out, int capacity);

/* n_steps guided Euler steps (research note, "Training method": Euler
 * integration z_{t - dt} = z_t + v dt with a per-step guidance weight): step i
 * is sfm_cfg_step at t = (float)t[i], dt = (float)(t[i] - t[i + 1]), guidance
 * guidance[i], reading z for the first step and z_out afterwards (z_out may
 * equal z).  t (n_steps + 1) and guidance (n_steps) are host arrays; t must be
 * finite and strictly decreasing.  Workspace: sfm_step_workspace_bytes.  All
 * checks run before the first step is enqueued; errors as sfm_cfg_step plus
 * SFM_E_INVALID_ARG for the arrays. */
int sfm_sample(const sfm_context* ctx, const sfm_model_weights* cond, const sfm_model_weights* uncond,
               const uint16_t* text, const float* z, float* z_out, const double* t, const float* guidance,
               int n_steps, int B, int T, int gh, int gw, void* ws, size_t ws_bytes, void* stream);
/* sfm_sample over sfm_cfg_step_varlen (per-sample text lengths, see above). */
int sfm_sample_varlen(const sfm_context* ctx, const sfm_model_weights* cond, const sfm_model_weights* uncond,
                      const uint16_t* text, const int32_t* text_lens, const float* z, float* z_out, const double* t,
                      const float* guidance, int n_steps, int B, int T, int gh, int gw, void* ws, size_t ws_bytes,
                      void* stream);

/* ---------------------------------------------------------------- errors */
const char* sfm_status_string(int status);
const char* sfm_last_error(void);

/* Debug mode for callers hunting an asynchronous failure: with on != 0 every
 * kernel launch of every entry point is followed by hipDeviceSynchronize and
 * hipGetLastError, and a failure there is returned as SFM_E_DEVICE by the
 * entry point whose launch caused it (with the launch named in
 * sfm_last_error()).  Process-wide; off by default, or on when the
 * environment holds SFM_SYNC_CHECK=1 as the library loads.  It serialises all
 * streams and must stay off under HIP graph capture.  Returns the previous
 * setting. */
int sfm_set_sync_check(int on);

#ifdef __cplusplus
}
#endif
#endif /* SFM_H */
