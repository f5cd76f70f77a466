"""The synthetic MXFP4 weight recipe: its stored frequencies are those that OCP MX
quantisation of N(0, 0.02^2) weights produces, and the generator follows them.

Recomputed here from the normal distribution (scipy): a block's shared exponent
is floor(log2 amax) - 2 (+127), so the block maximum of 32 draws picks the
exponent; an element's E2M1 code is the nearest value, so the normal mass
between neighbouring midpoints (in units of the block scale) gives the code
frequencies."""

import numpy as np
import torch
from scipy.stats import norm

from stream_flow_matching_amd import synth

SIGMA = 0.02
MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])   # between the E2M1 magnitudes 0 .. 6


def _amax_cdf(a):
    return (2 * norm.cdf(a / SIGMA) - 1) ** 32


def test_exponent_probabilities_match_the_block_maximum():
    # exponent e holds blocks whose maximum lies in [2^(e-125), 2^(e-124))
    p = [_amax_cdf(2.0 ** (e - 124)) - _amax_cdf(2.0 ** (e - 125)) for e in (119, 120, 121)]
    assert sum(p) > 0.9999                           # the other exponents are negligible
    np.testing.assert_allclose(synth._MX_EXP_P, p, atol=1e-4)


def test_code_frequencies_match_the_normal_mass_between_midpoints():
    for row, e in zip(synth._MX_CODE_P, (119, 120, 121)):
        scale = 2.0 ** (e - 127)
        cdf = 2 * norm.cdf(MIDPOINTS * scale / SIGMA) - 1
        p = np.diff(np.r_[0.0, cdf, 1.0])
        # stored to 4 decimals, the last entry absorbing the rounding so that a
        # row sums to 1: within 1.5e-4 of the exact masses
        np.testing.assert_allclose(row, p, atol=1.5e-4)
        assert abs(sum(row) - 1) < 1e-9


def test_generated_weights_follow_the_tables():
    n, k = 512, 4096
    packed, ex = synth.mxfp4_weight(n, k, ("recipe",))
    q = torch.stack([packed & 15, packed >> 4], dim=-1).view(n, k).numpy()
    e = ex.numpy()
    assert set(np.unique(e)) <= {119, 120, 121}
    np.testing.assert_allclose(np.bincount(e.ravel() - 119, minlength=3) / e.size, synth._MX_EXP_P, atol=5e-3)
    # every block holds its forced +-6; the other codes of exponent-120 blocks follow that row
    blocks = q.reshape(n * k // 32, 32)
    assert np.all((blocks & 7).max(axis=1) == 7)
    mag = (blocks[e.ravel() == 120] & 7).ravel()
    freq = np.bincount(mag, minlength=8) / mag.size
    expect = np.array(synth._MX_CODE_P[1]) * 31 / 32
    expect[7] += 1 / 32
    np.testing.assert_allclose(freq, expect, atol=3e-3)
    # signs are balanced
    assert abs((q >= 8).mean() - 0.5) < 5e-3
    # weight rms of the recipe: 0.020, as the FP8 recipe's N(0, 0.02^2)
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])[q & 7] * np.exp2(np.repeat(e, 32, axis=1).astype(float) - 127)
    assert abs(np.sqrt(np.mean(vals ** 2)) - 0.020) < 0.0015
