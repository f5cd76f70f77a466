"""Pins for the oracle's number formats: bf16 rounding, FP8-E4M3 decode/encode,
the NF4 codebook and the two dequantisers.  Each pin is independent of the
oracle's own code: a library routine (torch's float8_e4m3fn / bfloat16 casts,
scipy's normal CDF), brute force over all codes, or a page's stated fact."""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.stats import norm

from oracle import numerics as N

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- E4M3

def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_all_codes_match_library():
    ours = N.e4m3_decode(np.arange(256, dtype=np.uint8))
    ref = _torch_decode_all()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])


def test_e4m3_decode_special_codes():
    v = N.e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x7E, 0xFE, 0x7F, 0xFF, 0x80], np.uint8))
    assert v[0] == 0.0 and v[1] == 2.0 ** -9 and v[2] == 7 * 2.0 ** -9
    assert v[3] == 2.0 ** -6 and v[4] == 1.0
    assert v[5] == 448.0 and v[6] == -448.0
    assert math.isnan(v[7]) and math.isnan(v[8])
    assert v[9] == 0.0
    pos = N.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)              # 127 non-negative finite values strictly increasing
    assert np.sum(~np.isnan(N.e4m3_decode(np.arange(256, dtype=np.uint8)))) == 254


def test_e4m3_encode_roundtrip_all_finite():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], np.uint8)
    assert np.array_equal(N.e4m3_encode(N.e4m3_decode(codes)), codes)


def _brute_encode(x):
    """Nearest finite E4M3 magnitude by exhaustive search over codes 0..126,
    ties to the even code, saturating at 448; the sign bit is added after."""
    codes = np.arange(0, 127, dtype=np.int64)
    vals = N.e4m3_decode(codes.astype(np.uint8))
    out = []
    for xi in x:
        a = min(abs(xi), 448.0)
        d = np.abs(vals - a)
        cand = codes[d == np.min(d)]
        c = int(cand[0]) if len(cand) == 1 else int(cand[(cand & 1) == 0][0])
        out.append(c | (0x80 if xi < 0 else 0))
    return np.array(out, np.uint8)


def test_e4m3_encode_matches_brute_force():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.normal(0, 50, 3000), rng.normal(0, 0.01, 1000), rng.uniform(-500, 500, 1000),
    ]).astype(np.float32).astype(np.float64)
    # exact midpoints between neighbouring codes (ties)
    pos = N.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.concatenate([x, mids, -mids, [448.0, 460.0, 464.0, 1e6, -1e6]])
    ours = N.e4m3_encode(x)
    ref = _brute_encode(x)
    # the sign of a result that rounds to zero is a don't-care
    same = (ours == ref) | (((ours & 0x7F) == 0) & ((ref & 0x7F) == 0))
    assert np.all(same), x[~same][:10]


def test_e4m3_encode_matches_library_in_range():
    rng = np.random.default_rng(2)
    x = rng.normal(0, 60, 20000).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(N.e4m3_encode(x.astype(np.float64)), ref)


def test_e4m3_encode_saturates():
    assert list(N.e4m3_encode(np.array([1e4, -1e4, 449.0, 480.0, np.nan]))) == [0x7E, 0xFE, 0x7E, 0x7E, 0x7F]


# --------------------------------------------------------------------------- bf16

def test_bf16_round_matches_library():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.normal(0, 1, 50000), rng.normal(0, 1e-3, 1000), rng.normal(0, 1e4, 1000)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(N.bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_ties_to_even():
    # every bf16 upper half with the low half exactly at the midpoint 0x8000
    hi = np.arange(0, 0x7F80, 7, dtype=np.uint32)
    bits = (hi << 16) | 0x8000
    x = bits.view(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(N.bf16_round(x.astype(np.float64)), ref)
    # and the ones just above / below the tie
    for low in (0x7FFF, 0x8001):
        x = ((hi << 16) | low).view(np.float32)
        ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
        assert np.array_equal(N.bf16_round(x.astype(np.float64)), ref)


def test_bf16_bits_roundtrip():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)
    assert np.array_equal(N.float_to_bf16_bits(N.bf16_bits_to_float(bits)), bits)


# --------------------------------------------------------------------------- NF4

def test_nf4_codebook_shape_and_endpoints():
    cb = N.nf4_codebook()
    assert cb.dtype == np.float32 and cb.shape == (16,)
    assert cb[0] == -1.0 and cb[7] == 0.0 and cb[15] == 1.0
    assert np.all(np.diff(cb) > 0)
    assert np.sum(cb < 0) == 7 and np.sum(cb > 0) == 8


def test_nf4_codebook_levels_are_evenly_spaced_normal_quantiles():
    """Mapping the levels back through the normal CDF (scipy, independent of the
    oracle's quantile routine) must give evenly spaced probabilities: step
    (delta - 1/2)/8 on the positive side and (delta - 1/2)/7 on the negative."""
    cb = N.nf4_codebook().astype(np.float64)
    delta = 0.5 * ((1 - 1 / 32) + (1 - 1 / 30))
    top = norm.ppf(delta)
    p_pos = norm.cdf(cb[8:] * top)                # 8 positive levels, ascending
    p_neg = norm.cdf(-cb[:7] * top)               # 7 negative levels, |.| descending
    assert np.allclose(np.diff(p_pos), (delta - 0.5) / 8, atol=1e-6)
    assert np.allclose(np.diff(p_neg[::-1]), (delta - 0.5) / 7, atol=1e-6)
    assert abs(p_pos[-1] - delta) < 1e-7 and abs(p_pos[0] - (0.5 + (delta - 0.5) / 8)) < 1e-6


def test_nf4_page_list_is_rejected():
    page = json.load(open(os.path.join(GOLD, "nf4_page_list.json")))
    lv = np.array(page["levels"])
    assert page["block_size"] == 64 and len(lv) == 16
    assert lv.max() > 1.0                           # cannot be an absmax-normalised code
    assert not np.allclose(lv, N.nf4_codebook(), atol=1e-3)


def test_nf4_dequant_brute_force():
    rng = np.random.default_rng(4)
    n, k = 3, 128
    q = rng.integers(0, 16, (n, k))
    packed = ((q[:, 0::2] << 4) | q[:, 1::2]).astype(np.uint8)
    absmax = rng.uniform(0.01, 0.1, n * k // 64).astype(np.float32)
    cb = N.nf4_codebook()
    out = N.nf4_dequant_f32(packed, absmax, n, k)
    for i in range(n):
        for j in range(k):
            want = np.float32(cb[q[i, j]]) * np.float32(absmax[(i * k + j) // 64])
            assert out[i, j] == np.float32(want)


def test_fp8_dequant_brute_force():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (4, 9)).astype(np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    s = rng.uniform(1e-5, 1e-3, 4).astype(np.float32)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * torch.from_numpy(s)[:, None]
    assert np.array_equal(N.fp8_dequant_f32(codes, s), ref.numpy())
