"""Pins of the oracle's MXFP4 format (E2M1 elements, E8M0 scale per 32 elements
of a row) and of its linear layer.  [Deploy] section 2.2: 4-bit float FFN
weights with block scales (mixed scheme); the gfx950 form is OCP MXFP4."""

import numpy as np
import pytest
import torch

import oracle.dit as O
import oracle.numerics as N


def test_e2m1_codebook_structure():
    """The 8 magnitudes of a 1-sign, 2-exponent (bias 1), 1-mantissa minifloat:
    0, a subnormal half of the smallest normal, then three binades of two
    values each, each binade twice the last, the top value 6."""
    v = N.e2m1_decode(np.arange(16))
    mag = v[:8]
    assert mag[0] == 0.0
    assert np.all(np.diff(mag) > 0)
    assert mag[1] == mag[2] / 2                       # subnormal step = half of 1.0
    for e in range(1, 4):                              # binade e: codes 2e, 2e + 1
        lo, hi = mag[2 * e], mag[2 * e + 1]
        assert hi == lo * 1.5                          # one mantissa bit
        if e > 1:
            assert lo == 2 * mag[2 * (e - 1)]
    assert mag[7] == 6.0
    assert np.array_equal(v[8:], -mag)                 # sign bit


def _brute_force_encode(x):
    """Nearest of the 15 distinct E2M1 values; on a tie the code with the even
    mantissa bit; beyond 6 saturate."""
    vals = N.e2m1_decode(np.arange(16))
    out = []
    for xi in np.asarray(x, np.float64):
        d = np.abs(vals - np.clip(xi, -6, 6))
        best = np.flatnonzero(d == d.min())
        # among ties (and +-0), prefer an even mantissa bit, then the sign of x
        best = sorted(best, key=lambda c: ((c & 1), (c >= 8) != (xi < 0)))
        out.append(vals[best[0]])
    return np.array(out)


def test_e2m1_encode_brute_force():
    grid = np.concatenate([np.linspace(-7.5, 7.5, 6001),
                           # every midpoint between neighbouring values (the ties) and just around them
                           *[np.array([m - 1e-9, m, m + 1e-9]) * s
                             for m in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0) for s in (1, -1)]])
    got = N.e2m1_decode(N.e2m1_encode(grid))
    assert np.array_equal(np.abs(got), np.abs(_brute_force_encode(grid)))
    assert np.array_equal(np.sign(got[got != 0]), np.sign(grid[got != 0]))


def test_e8m0_against_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float32).double().numpy()
    got = N.e8m0_decode(codes.numpy())
    assert np.array_equal(got[:255], ref[:255])
    assert np.isnan(got[255]) and np.isnan(ref[255])


def test_mxfp4_pack_layout():
    """Element 2i in the low nibble of byte i (the order the matrix cores read)."""
    c = np.array([[1, 2, 15, 0]], np.uint8)
    p = N.mxfp4_pack(c)
    assert p.tolist() == [[0x21, 0x0F]]
    r = np.random.default_rng(0).integers(0, 16, (3, 64)).astype(np.uint8)
    assert np.array_equal(N.mxfp4_unpack(N.mxfp4_pack(r), 3, 64), r)


def test_mxfp4_representable_roundtrip():
    """Blocks of E2M1 values times a power of two come back exactly."""
    rng = np.random.default_rng(1)
    n, k = 6, 128
    codes = rng.integers(0, 16, (n, k))
    s = rng.integers(-10, 3, (n, k // 32))
    w = N.e2m1_decode(codes) * np.exp2(np.repeat(s, 32, axis=1))
    q, e = N.mxfp4_quantize(w)
    d = N.mxfp4_dequant_f32(N.mxfp4_pack(q), e, n, k)
    assert np.array_equal(d.astype(np.float64), w)


def test_mxfp4_error_bound():
    """Per element: half a grid step of its binade in the block's scale, or the
    saturation excess above 6 * scale."""
    rng = np.random.default_rng(2)
    n, k = 8, 256
    w = rng.normal(0, 0.02, (n, k))
    q, e = N.mxfp4_quantize(w)
    d = N.mxfp4_dequant_f32(N.mxfp4_pack(q), e, n, k).astype(np.float64)
    scale = np.repeat(np.exp2(e.astype(np.float64) - 127), 32, axis=1)
    a = np.abs(w) / scale
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    bound = np.where(a <= 6, step / 2, a - 6) * scale
    assert np.all(np.abs(d - w) <= bound * (1 + 1e-12))
    # the block scale puts each block's largest magnitude in [4, 8) scale units
    amax = np.abs(w).reshape(n, k // 32, 32).max(axis=2) / np.exp2(e.astype(np.float64) - 127)
    assert np.all((amax >= 4) & (amax < 8))


def test_mxfp4_linear_matches_fp8_linear():
    """Weights that one exponent per row scales are also exact FP8 weights
    (E2M1 values are E4M3 values; the row's power of two is the per-channel
    scale): the MXFP4 and FP8 layers (the latter pinned against torch's E4M3)
    must give identical products."""
    rng = np.random.default_rng(3)
    n, k, m = 16, 96, 5
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    row_e = rng.integers(118, 124, n).astype(np.uint8)
    scales = np.repeat(row_e[:, None], k // 32, axis=1)
    a = N.bf16_round(rng.normal(0, 1, (m, k)))
    y_mx = O.mxfp4_linear(a, N.mxfp4_pack(codes), scales, n, k)
    fp8_codes = N.e4m3_encode(N.e2m1_decode(codes))
    y_f8 = O.fp8_linear(a, fp8_codes, np.exp2(row_e.astype(np.float64) - 127).astype(np.float32))
    assert np.array_equal(y_mx, y_f8)


def test_mxfp4_block_scales_apply_per_block():
    """One weight row with a different exponent in each 32-block: the product
    is the sum of the per-block products, each scaled by its own power of two."""
    rng = np.random.default_rng(4)
    k = 128
    codes = rng.integers(0, 16, (1, k)).astype(np.uint8)
    e = np.array([[120, 127, 130, 100]], np.uint8)
    a = N.bf16_round(rng.normal(0, 1, (3, k)))
    y = O.mxfp4_linear(a, N.mxfp4_pack(codes), e, 1, k)
    aq, alpha = O.quantize_rows_e4m3(a)
    parts = []
    for b in range(4):
        sl = slice(32 * b, 32 * b + 32)
        parts.append(N.e4m3_decode(aq[:, sl]) @ N.e2m1_decode(codes[0, sl]) * 2.0 ** (int(e[0, b]) - 127))
    ref = np.sum(parts, axis=0) * alpha / N.E4M3_MAX
    np.testing.assert_allclose(y[:, 0], ref, rtol=1e-15, atol=0)


def test_mixed_block_matches_fp8_block():
    """A block with MXFP4 gate/up and down weights (one exponent per row) equals
    the FP8 block holding the same weights as E4M3 codes with per-row scales."""
    from stream_flow_matching_amd import synth
    from _util import oracle_block
    w = synth.Workload("tiny_mx", synth.TINY, 1, 4, 4, 4)
    p = synth.block_params(w.shape, (0, "mx_pin"), "mixed")
    x, c = synth.block_inputs(w)
    ob = oracle_block(p)
    for name in ("gate_up", "down"):
        mw = getattr(ob, name)
        row_e = mw.scales[:, :1].copy()
        mw.scales[:] = row_e                               # one exponent per row
        codes = N.mxfp4_unpack(mw.packed, mw.n, mw.k)
        f8 = O.Fp8Weight(N.e4m3_encode(N.e2m1_decode(codes)),
                         np.exp2(row_e[:, 0].astype(np.float64) - 127).astype(np.float32))
        setattr(ob, name + "_f8", f8)
    ob_f8 = O.BlockWeights(ob.qkv, ob.o, ob.gate_up_f8, ob.down_f8, ob.q_norm, ob.k_norm, ob.mod_w, ob.mod_b)
    xs = x.double().numpy()
    cs = c.double().numpy()
    y_mx = O.block_forward(xs, cs, ob, w.T, w.gh, w.gw, O.TINY)
    y_f8 = O.block_forward(xs, cs, ob_f8, w.T, w.gh, w.gw, O.TINY)
    assert np.array_equal(y_mx, y_f8)
