"""Writes tests/golden/cfg_step_1024.npz: the oracle's conditional and
unconditional velocities for one guided Euler step of the full 34-layer model
at 1024 x 1024 (512 projected text tokens + 64 x 64 image tokens for the
conditional model, the image tokens alone for the separate unconditional
model; both FP8 weight sets, the latent and t drawn by the seeded generators
in stream_flow_matching_amd/synth.py, keys (0, "cond") and (0, "uncond")), at
the step's t and at t moved by one float32 ulp (*_tulp: the oracle's own
response to a rounding-level change of one input).

Only the oracle computes here.  Each pass walks its 34 blocks with the block
weights drawn one layer at a time, so a pass holds one layer's weights at
once; the four passes run in four processes.  Every eighth image token's
velocity row (512 rows x 128 channels, fp32) is stored with t, dt and the row
indices.  Run from the repository root:  python tests/golden/make_cfg_step_1024.py
(about 80 minutes on 8 cores in float64).
"""

import os
import sys
from multiprocessing import get_context

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
os.environ.setdefault("OPENBLAS_NUM_THREADS", "2")      # four passes share the cores

import numpy as np  # noqa: E402

OUT = os.path.join(HERE, "cfg_step_1024.npz")
ROWS = np.arange(0, 4096, 8)


def task(args):
    name, ulp = args
    from stream_flow_matching_amd import synth
    from tests.golden import oracle_runs as R
    w = synth.WORKLOADS["cfg_step_1024"]
    v = R.velocity(w, w.layers, (0, name), name == "cond", ulp)
    return ("v_c_rows" if name == "cond" else "v_u_rows") + ("_tulp" if ulp else ""), v[ROWS].astype(np.float32)


def main():
    from stream_flow_matching_amd import synth
    _, _, t, dt = synth.step_inputs(synth.WORKLOADS["cfg_step_1024"])
    tasks = [(n, u) for u in (False, True) for n in ("cond", "uncond")]
    with get_context("spawn").Pool(4) as pool:
        out = dict(pool.map(task, tasks))
    np.savez_compressed(OUT, rows=ROWS, t=np.float64(t), dt=np.float64(dt), **out)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
