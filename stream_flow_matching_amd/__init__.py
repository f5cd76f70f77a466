"""MI355X (gfx950) library for the Ideogram-4 single-stream DiT block and the
Euler / asymmetric-CFG denoising step.

The compute path is libsfm.so (hand-written HIP kernels behind the C ABI in
include/sfm.h); ``stream_flow_matching_amd.sfm`` is its ctypes binding and
``stream_flow_matching_amd.synth`` makes seeded synthetic inputs.  Importing the
package loads nothing; the library is loaded on first use.
"""
