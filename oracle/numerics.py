"""Number formats used at the storage points of the path (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

* bf16: the pipeline runs in bfloat16 ([Note] "Infra", Diffusers pipeline in
  bf16).  ``bf16_round`` rounds a real value to the nearest bfloat16,
  ties to even, in one step from float64.
* FP8 E4M3: the released weights are FP8 E4M3 ([Deploy] section 2).  The
  variant is the OCP E4M3FN one: exponent bias 7, no infinities, NaN only at
  S.1111.111, largest finite 448, subnormals m * 2**-9.
* MXFP4: [Deploy] section 2.2 describes a mixed scheme with the FFN layers in
  4-bit floats (torch.float4_e2m1fn elements, block scales) and the attention
  projections kept in FP8.  The gfx950 form here is OCP MXFP4: E2M1 elements,
  one E8M0 power-of-two scale per 32 consecutive elements of a row.
* NF4: [Deploy] section 2.1 names QLoRA's NormalFloat-4 with block size 64.
  The codebook printed there (ending at 1.6368) cannot be an absmax-scaled
  code (its values exceed 1), so the codebook here is rebuilt from the QLoRA
  construction the page cites: normal quantiles at evenly spaced
  probabilities, 8 on the positive side and 7 on the negative side plus an
  exact zero, normalised so that the extreme codes are -1 and +1.
"""

from __future__ import annotations

import math
import statistics

import numpy as np

E4M3_MAX = 448.0


# --------------------------------------------------------------------------- bf16

def bf16_round(x) -> np.ndarray:
    """Round real values (any float array) to the nearest bf16, ties to even.

    bf16 keeps 8 significant bits and fp32's exponent range.  The value is
    written as m * 2**e with 0.5 <= |m| < 1 (np.frexp is exact); the quantum at
    that binade is 2**(e-8), clamped at the subnormal quantum 2**-133.
    Overflow past the largest finite bf16 gives +-inf.  Result is float64.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[finite])
    e = np.maximum(e, -125)                      # below 2**-126: fixed subnormal quantum
    quantum = np.ldexp(1.0, e - 8)
    r = np.rint(x[finite] / quantum) * quantum   # np.rint: half to even
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > big, np.copysign(np.inf, r), r)
    out[finite] = r
    return out


def bf16_bits_to_float(bits) -> np.ndarray:
    """Decode raw bf16 bit patterns (uint16) to float64: the upper half of fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def float_to_bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of values that are already bf16-representable."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------- E4M3

def e4m3_decode(codes) -> np.ndarray:
    """Value of each OCP E4M3FN code (uint8) as float64.

    Fields: sign s = bit 7, exponent E = bits 6..3, mantissa M = bits 2..0.
    E == 0: (-1)**s * M/8 * 2**-6 (subnormal).  E > 0: (-1)**s * (1 + M/8) *
    2**(E-7).  E == 15 and M == 7 is NaN; there is no infinity.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 0x7
    normal = (1.0 + M / 8.0) * np.ldexp(1.0, E - 7)
    sub = (M / 8.0) * 2.0 ** -6
    v = s * np.where(E == 0, sub, normal)
    v = np.where((E == 15) & (M == 7), np.nan, v)
    return v


def e4m3_encode(x) -> np.ndarray:
    """Round values to the nearest E4M3FN code, ties to even, saturating.

    Inputs are clamped to [-448, 448] first (saturating conversion), so no
    finite input becomes NaN; NaN inputs give 0x7F.  The input is taken as an
    exact real number (callers pass fp32 values).
    """
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), E4M3_MAX)
    sign = (np.signbit(np.where(nan, 0.0, x))).astype(np.int64)
    # subnormal range: |x| < 2**-6, quantum 2**-9; code = rint(|x| / 2**-9)
    # (a result of 8 is code 0x08 = 2**-6, the smallest normal, so it is consistent)
    sub_code = np.rint(a / 2.0 ** -9).astype(np.int64)
    # normal range: |x| = f * 2**e, f in [1, 2)
    _, e2 = np.frexp(np.where(a > 0, a, 1.0))  # a = m * 2**e2, m in [0.5, 1)
    e = e2 - 1
    q = np.rint(a / np.ldexp(1.0, e) * 8.0).astype(np.int64)  # 8..16
    carry = q == 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 8, q)
    norm_code = ((e + 7) << 3) | (q - 8)
    code = np.where(a < 2.0 ** -6, sub_code, norm_code)
    code = code | (sign << 7)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------- NF4

def nf4_codebook() -> np.ndarray:
    """The 16 NF4 code values, computed in float64 and returned as float32.

    Construction (QLoRA "4-bit NormalFloat"; [Deploy] section 2.1 names it and
    the block size 64): take the probability offset
    delta = ((1 - 1/32) + (1 - 1/30)) / 2.  Positive side: the standard normal
    quantiles at 9 evenly spaced probabilities from delta down to 1/2, keeping
    the first 8 (the 1/2 end is the zero).  Negative side: the negated quantiles
    at 8 evenly spaced probabilities from delta down to 1/2, keeping the first
    7.  Add an exact zero, sort, divide everything by the largest magnitude
    (the quantile at delta).  Result: code[0] = -1, code[7] = 0, code[15] = +1.
    """
    nd = statistics.NormalDist()
    delta = 0.5 * ((1.0 - 1.0 / 32.0) + (1.0 - 1.0 / 30.0))
    pos_p = [delta + (0.5 - delta) * i / 8.0 for i in range(8)]
    neg_p = [delta + (0.5 - delta) * i / 7.0 for i in range(7)]
    pos = [nd.inv_cdf(p) for p in pos_p]
    neg = [-nd.inv_cdf(p) for p in neg_p]
    vals = sorted(pos + neg + [0.0])
    top = max(abs(v) for v in vals)
    return np.array([v / top for v in vals], dtype=np.float64).astype(np.float32)


def nf4_unpack(packed: np.ndarray, n: int, k: int) -> np.ndarray:
    """Nibble indices [n, k] from packed bytes [n, k/2].

    Element 2i of a row sits in the high nibble of byte i, element 2i+1 in the
    low nibble (the layout chosen for this library's NF4 weights).
    """
    p = np.asarray(packed, dtype=np.uint8).reshape(n, k // 2)
    out = np.empty((n, k), dtype=np.uint8)
    out[:, 0::2] = p >> 4
    out[:, 1::2] = p & 0xF
    return out


def nf4_dequant_f32(packed, absmax, n: int, k: int) -> np.ndarray:
    """fp32 weight w[n, k] = fp32(code[q[n, k]] * absmax[(n*k + k) // 64]).

    Blocks are 64 consecutive elements of the row-major [n, k] weight; the
    product is one fp32 multiply (IEEE, round to nearest even).
    """
    if k % 64:
        raise ValueError("NF4 blocks of 64 need k % 64 == 0")
    q = nf4_unpack(packed, n, k)
    code = nf4_codebook()
    am = np.asarray(absmax, dtype=np.float32).reshape(n, k // 64)
    am_full = np.repeat(am, 64, axis=1)
    return (code[q].astype(np.float32) * am_full).astype(np.float32)


# --------------------------------------------------------------------------- MXFP4

def e2m1_decode(codes) -> np.ndarray:
    """Value of 4-bit E2M1 codes (float64).

    Code bits s.ee.m: sign s, exponent field e (bias 1), one mantissa bit m.
    e = 0 is the subnormal binade, value m * 2**-1; e > 0 gives
    (1 + m/2) * 2**(e - 1).  The largest finite magnitude is 6; there are no
    infinities or NaNs.  ([Deploy] section 2.2 names torch.float4_e2m1fn as the
    element type of the 4-bit layers.)
    """
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


def e2m1_encode(x) -> np.ndarray:
    """Nearest E2M1 code, ties to the even mantissa bit, |x| > 6 saturating to 6.

    Implemented by rounding |x| on the uniform grid of its binade: the grid
    step is 0.5 below 2, 1 in [2, 4) and 2 in [4, 8).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 6.0)
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    q = a / step
    r = np.floor(q)
    frac = q - r
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2) == 1))
    v = (r + up) * step                       # may step into the next binade (exact)
    v = np.minimum(v, 6.0)
    # code from the value: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 are codes 0..7
    mag_code = np.where(v < 2.0, np.round(v * 2.0), np.where(v < 4.0, v + 2.0, v / 2.0 + 4.0)).astype(np.int64)
    sign = ((x < 0) & (mag_code > 0)).astype(np.int64)
    return (sign << 3 | mag_code).astype(np.uint8)


def e8m0_decode(codes) -> np.ndarray:
    """E8M0 block scale 2**(code - 127) (float64); code 255 is NaN."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def mxfp4_quantize(w, block=32):
    """(codes uint8 [n, k], scale exponents uint8 [n, k/block]) of w [n, k].

    OCP Microscaling, FP4 (E2M1) elements: each block of 32 consecutive
    elements of a row shares the scale 2**X with X = floor(log2(amax)) - 2
    (2 is the largest E2M1 exponent, so amax / 2**X lies in [4, 8) and values
    above 6 saturate); elements are e2m1_encode(w / 2**X).  An all-zero block
    gets exponent code 0.  This is the gfx950 analogue of the 4-bit FFN layers
    of the mixed scheme in [Deploy] section 2.2 (NVIDIA's variant: E4M3 scales
    over other block sizes).
    """
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    if k % block:
        raise ValueError("k must be a multiple of the block size")
    wb = w.reshape(n, k // block, block)
    amax = np.abs(wb).max(axis=2)
    with np.errstate(divide="ignore"):
        X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2.0, -127.0)
    X = np.clip(X, -127.0, 127.0)
    codes = e2m1_encode(wb / np.exp2(X)[:, :, None]).reshape(n, k)
    return codes, (X + 127.0).astype(np.uint8)


def mxfp4_pack(codes) -> np.ndarray:
    """Bytes [n, k/2] of codes [n, k]: element 2i in the low nibble of byte i, 2i+1 in the high
    nibble (the order the gfx950 matrix cores read 4-bit operands)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def mxfp4_unpack(packed, n: int, k: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(n, k // 2)
    out = np.empty((n, k), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def mxfp4_dequant_f32(packed, scales, n: int, k: int) -> np.ndarray:
    """fp32 weight w[n, k] = e2m1(q[n, k]) * 2**(e[n, k // 32] - 127); exact in fp32 (a 2-bit
    significand times a power of two no smaller than 2**-128)."""
    if k % 32:
        raise ValueError("MXFP4 blocks of 32 need k % 32 == 0")
    q = mxfp4_unpack(packed, n, k)
    sc = np.repeat(e8m0_decode(np.asarray(scales, np.uint8).reshape(n, k // 32)), 32, axis=1)
    return (e2m1_decode(q) * sc).astype(np.float32)


def fp8_dequant_f32(codes, scale) -> np.ndarray:
    """fp32 weight w[n, k] = fp32(decode(q[n, k]) * s[n]) (per-output-channel scale)."""
    dec = e4m3_decode(codes).astype(np.float32)
    s = np.asarray(scale, dtype=np.float32)[:, None]
    return (dec * s).astype(np.float32)


def ulp_distance_f32(a, b) -> np.ndarray:
    """Distance in fp32 units-in-last-place (for diagnostics only)."""
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, np.int64(-(2 ** 31)) - ai, ai)
    bi = np.where(bi < 0, np.int64(-(2 ** 31)) - bi, bi)
    return np.abs(ai - bi)


def rel_l2(a, b) -> float:
    """||a - b||_2 / ||b||_2 in float64."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = math.sqrt(float(np.sum(b * b)))
    num = math.sqrt(float(np.sum((a - b) ** 2)))
    return num / den if den > 0 else num
