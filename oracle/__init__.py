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
             original weights) and section 2.1 (NF4, block size 64, QLoRA).
  [Tuner]    SimpleTuner Ideogram 4 quick-start, sections "Text embed cache"
             (4608-d projected text features) and "Validation" (separate
             image-only unconditional transformer).

Parity status per function is listed in ``oracle/PINS.md``.
"""

from . import numerics, dit  # noqa: F401
