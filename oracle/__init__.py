"""Plain CPU oracle for the Ideogram-4 single-stream DiT block and the Euler /
asymmetric-CFG step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
anything in this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the GPU library
(no kernels, headers, helpers, tables or constant generators); the two meet only
through seeded inputs produced elsewhere.

Every function is a direct, slow transcription of the definition it cites, in
float64 between the storage points that the definition fixes (bf16 activations,
FP8-E4M3 / NF4 weight codes).  Citations name the source page and its section:

  [Note]     "Ideogram 4.0" research note (zhao9797.github.io), sections
             "Model architecture" (block internals and the model spec table) and
             "Training method" (flow matching, Euler, asymmetric CFG).
  [Deploy]   "Ideogram 4.0 free local deployment" blog post (post.smzdm.com),
             section 1.3 (asymmetric CFG, scale 4.0), section 2 (FP8 E4M3
             original weights), section 2.1 (NF4, block size 64, QLoRA) and
             section 2.2 (mixed scheme: 4-bit float FFN weights with block
             scales, attention projections in FP8; here in the OCP MXFP4 form).
  [Note]     also section "Infra" (sampling presets) for the sampler.
  [Tuner]    SimpleTuner Ideogram 4 quick-start, sections "Text embed cache"
             (4608-d projected text features) and "Validation" (separate
             image-only unconditional transformer).

What pins each function (tests/test_oracle_numerics.py, tests/test_oracle_dit.py):
  bf16_round / bits      torch's bfloat16 cast, ties-to-even cases
  e4m3_decode / encode   all 256 codes vs torch's float8_e4m3fn cast; brute-force
                         nearest-code search; saturation
  nf4_codebook           endpoints -1, 0, 1; levels are evenly spaced normal
                         quantiles (scipy's inverse CDF)
  nf4/fp8 dequant        brute force per element
  e2m1 / e8m0 / mxfp4    (tests/test_oracle_mxfp4.py) E2M1 table structure (sign,
                         bias-1 binades, top value 6); brute-force nearest encode
                         with ties to even; E8M0 vs torch's float8_e8m0fnu; nibble
                         order; exact round trip of representable blocks; error
                         bound incl. saturation; mxfp4_linear equals fp8_linear on
                         weights both formats hold exactly; per-block scales; the
                         mixed block equals the FP8 block on such weights
  silu, timestep_embedding   closed forms
  modulation             (tests/test_oracle_block_pins.py) unit-vector weights: SiLU of
                         c plus bias, chunk-major order (scale_a, gate_a, scale_m, gate_m)
  timestep_mlp           identity-like weights against the closed form with SiLU
  rms_normalize, adaln_norm  invariants (unit RMS, scale invariance, scale -1 -> 0)
  quantize_rows_e4m3, fp8_linear  identity on representable rows, brute-force
                         matmul when quantisation is exact, zero rows, power-of-two
                         scaling, bounded quantisation error
  positions, mrope_*     layout written out, closed-form angles, pair norms,
                         identity at position 0, relative-position property,
                         one axis moves one section; a unit pair turns to
                         (cos, sin) (RoFormer's rotation direction)
  qk_norm_rope           +-1 rows with power-of-two gamma give +-gamma; a random row
                         with gamma != 1 against a hand loop
  nf4_linear             brute force with torch's fp32 product and bf16 cast of the
                         dequantised weight
  attention              brute force on tiny sequences, special cases
  block_forward          gate 0 and scale -1 identities, row-subset and batch
                         consistency; each branch switched off by its own chunk
                         (gate_a = 0 with scale_m = -1 and the converse); an
                         MLP-only update computed by hand (SwiGLU operand order,
                         scale_m / gate_m wiring); attention half then MLP half
                         equals the block (the MLP reads x1); value rows and the
                         output projection's orientation by hand
  model_velocity         zero-layer reduction to the final layer of the embedding
  euler_cfg, cfg_step    closed forms; uncond ignores text; guidance 1 gives cond
  param_count            the ~9.3B of the spec table
  text_projection        feature width of the cache page; exact scale invariance
                         (eps 0); the textbook product when quantisation is exact
  sampler.time_grid      endpoints, order, closed-form median sigmoid(log 2) = 2/3,
                         symmetry without shift, scipy's normal quantile
  sampler presets        the research note's preset table (tests/golden)
  sampler.euler_loop / sample   constant velocity telescopes to z + v, the linear
                         ODE's product form, chaining of the guided steps
tests/oracle_mutations.py plants 22 plausible single-line mistakes in a scratch copy of
dit.py; each one fails at least one of the pins above.
Parity unpinned: the whole model against a real checkpoint (none exists here).
The modulation chunk order, the timestep MLP and the final layer are readings
of prose: the pins fix that the oracle computes exactly those readings, not
that a trained Ideogram 4 uses them.
"""

from . import numerics, dit, sampler  # noqa: F401
