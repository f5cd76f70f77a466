"""Build libsfm.so (gfx950) in-tree with hipcc.

Every .hip source under csrc/ is compiled to an object in parallel and linked
into stream_flow_matching_amd/libsfm.so.  Packed-fp32 instruction selection is
turned off for device code (the library does not rely on v_pk_*_f32).
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsfm.so")
BUILD = os.path.join(os.path.dirname(HERE), "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Per-source code-generation options.  The attention kernel keeps its O
# accumulators in the VGPR form of the MFMA instructions: the default mixed
# VGPR/AGPR assignment moves them between the two register files every tile;
# no operand of its max reductions can be a NaN, so the canonicalising moves
# around the cross-lane swaps are dropped.
FILE_FLAGS = {
    "k_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
}


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    return obj, warn


def build(verbose=False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    if verbose:
        for (_, w), s in zip(results, srcs):
            if w:
                print(f"[{os.path.basename(s)}]\n{w}", file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


# A second copy of the library whose host code carries AddressSanitizer and
# UndefinedBehaviorSanitizer instrumentation: the sources holding the C ABI's
# argument, shape and workspace checks and the sampler's host schedules are
# recompiled with the host-only sanitizer options; the kernel objects of the
# normal build are linked unchanged (device code is never instrumented).  The
# copy is loaded only by processes that preload the sanitizer runtime.
SAN_SOURCES = ("sfm_api.hip", "sfm_sampler.hip")
SAN_FLAGS = ("-O1 -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
             "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer").split()
SAN_LINK = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -shared-libsan".split()
SAN_OUT = os.path.join(HERE, "libsfm_asan.so")


def sanitizer_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (to preload)."""
    import glob
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang", "*",
                                         "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so next to hipcc")
    return hits[-1]


def build_sanitized() -> str:
    """Build libsfm_asan.so from the objects of build() and host-instrumented
    copies of SAN_SOURCES."""
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in sources()]
    if not all(os.path.exists(o) for o in objs):
        build()
    san_dir = os.path.join(BUILD, "asan")
    os.makedirs(san_dir, exist_ok=True)
    plain = [f for f in FLAGS if f != "-O3"]
    linked = []
    for src in sources():
        name = os.path.basename(src)
        if name not in SAN_SOURCES:
            linked.append(os.path.join(BUILD, name + ".o"))
            continue
        obj = os.path.join(san_dir, name + ".o")
        r = subprocess.run([HIPCC, *plain, *SAN_FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (sanitized) failed for {src}:\n{r.stderr}")
        linked.append(obj)
    tmp = SAN_OUT + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_LINK, "-o", tmp, *linked],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    os.replace(tmp, SAN_OUT)
    return SAN_OUT


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_sanitized())
