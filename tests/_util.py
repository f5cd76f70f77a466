"""Glue between the seeded inputs, the oracle and the GPU binding (tests only)."""

from __future__ import annotations

import numpy as np
import torch

from oracle import dit as O


def np64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a (CPU or device) float / bf16 tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def npu8(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").numpy().astype(np.uint8)


def oracle_weight(fmt, pair):
    q, s = pair
    if s.dtype == torch.uint8:                     # MXFP4: E8M0 exponents [n][k/32]
        n, k2 = q.shape
        return O.Mxfp4Weight(npu8(q), npu8(s), n, 2 * k2)
    if fmt in ("fp8", "mixed"):
        return O.Fp8Weight(npu8(q), s.detach().cpu().numpy().astype(np.float32))
    n, k2 = q.shape
    return O.Nf4Weight(npu8(q), s.detach().cpu().numpy().astype(np.float32), n, 2 * k2)


def oracle_block(p) -> O.BlockWeights:
    return O.BlockWeights(oracle_weight(p.fmt, p.qkv), oracle_weight(p.fmt, p.o), oracle_weight(p.fmt, p.gate_up),
                          oracle_weight(p.fmt, p.down), np64(p.q_norm), np64(p.k_norm), np64(p.mod_w),
                          p.mod_b.detach().cpu().numpy().astype(np.float32))


def oracle_model(p) -> O.ModelWeights:
    f32 = lambda t: t.detach().cpu().numpy().astype(np.float32)
    return O.ModelWeights([oracle_block(b) for b in p.blocks], np64(p.x_w), f32(p.x_b), np64(p.t_w1), f32(p.t_b1),
                          np64(p.t_w2), f32(p.t_b2), np64(p.f_mod_w), f32(p.f_mod_b), np64(p.f_w), f32(p.f_b))


def to_device(obj, device="cuda"):
    """Copy every tensor field of a synth dataclass (recursively) to the device."""
    import dataclasses
    if isinstance(obj, torch.Tensor):
        return obj.to(device)
    if isinstance(obj, tuple):
        return tuple(to_device(x, device) for x in obj)
    if isinstance(obj, list):
        return [to_device(x, device) for x in obj]
    if dataclasses.is_dataclass(obj):
        return dataclasses.replace(obj, **{f.name: to_device(getattr(obj, f.name), device)
                                           for f in dataclasses.fields(obj)})
    return obj


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def vt_order(n):
    """Token stored at each position of the attention kernel's V^T rows: inside
    every group of 32, positions 8g .. 8g+7 hold tokens 4g..4g+3, 16+4g..16+4g+3."""
    idx = np.empty(n, np.int64)
    for j in range(0, n, 32):
        for g in range(4):
            for e in range(8):
                idx[j + 8 * g + e] = j + 4 * g + (e if e < 4 else 12 + e)
    return idx


def check_rel(tag, got, ref, bar) -> float:
    """rel-L2 of got against ref, reported with its bar (stderr, and one JSON line
    appended to the file named by SFM_MARGINS when set), then asserted < bar."""
    import json
    import os
    import sys
    err = rel_l2(got, ref)
    print(f"[margin] {tag}: rel-L2 {err:.3e} (bar {bar:.1e})", file=sys.stderr, flush=True)
    path = os.environ.get("SFM_MARGINS")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"test": tag, "rel_l2": err, "bar": bar}) + "\n")
    assert err < bar, f"{tag}: rel-L2 {err:.3e} >= {bar}"
    return err


def check_spread(tag, got, ref, ref_alt, factor) -> float:
    """rel-L2 of got against the oracle's ref, bounded by `factor` times the
    oracle's own spread: the rel-L2 between ref and ref_alt, the oracle run on
    an input moved at rounding level (t by one float32 ulp).  Past a depth at
    which such a change already moves the output by percents (per-token FP8
    codes flip at their rounding boundaries and the flips compound from block
    to block), an implementation that rounds differently cannot come closer to
    the oracle than the oracle comes to itself; a wrong term still lands far
    outside.  Reported like check_rel."""
    import json
    import os
    import sys
    err, spread = rel_l2(got, ref), rel_l2(ref_alt, ref)
    bar = factor * spread
    print(f"[margin] {tag}: rel-L2 {err:.3e} (oracle spread {spread:.3e}, bar {bar:.3e})", file=sys.stderr,
          flush=True)
    path = os.environ.get("SFM_MARGINS")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"test": tag, "rel_l2": err, "oracle_spread": spread, "bar": bar}) + "\n")
    assert err < bar, f"{tag}: rel-L2 {err:.3e} >= {factor} x oracle spread {spread:.3e}"
    return err
