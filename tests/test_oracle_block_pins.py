"""Pins for the parts of the oracle's block and model that the identity pins in
test_oracle_dit.py cannot see: which modulation chunk feeds which branch, the
SiLU of the modulation and of the timestep MLP, the SwiGLU operand order, the
bf16 rounding of the NF4 weight operand, the direction of the rotary rotation
and the QK-norm weight.

Every expected value here is a closed form or a hand computation with Python
floats (math.exp, math.cos, explicit loops), independent of the oracle's own
formulas; a plausible one-line slip in any of those parts changes at least one
of them.

Sources: [Note] "Ideogram 4.0" research note, "Model architecture" (AdaLN
scale/gate on both residual paths, SwiGLU with a SiLU gate, QK-RMSNorm, MRoPE);
[Deploy] "Ideogram 4.0 NF4 deployment" post, section 2.1 (NF4 weights); the
rotation of a pair follows the RoFormer paper's rotary matrix
[[cos, -sin], [sin, cos]] (Su et al., 2021, section 3.2).
"""

import math

import numpy as np
import pytest
import torch

from oracle import dit as O
from oracle import numerics as N

D, H, F = 512, 2, 1536


def _silu(v):
    return v / (1.0 + math.exp(-v))


def _bf16(v):
    """bf16 rounding of one Python float through torch (independent of the oracle)."""
    return float(torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).to(torch.float64))


# --------------------------------------------------------------------------- modulation and timestep MLP

def test_modulation_applies_silu_and_splits_chunks_in_order():
    """W_mod rows are unit vectors: mod[b, i, j] = SiLU(c[b, r % 512]) + b_mod[r]
    with r = i*D + j (chunk-major order: scale_a, gate_a, scale_m, gate_m)."""
    Dm = 8                                   # four chunks of 8 rows
    rng = np.random.default_rng(101)
    c = rng.normal(0, 2, (2, 512))
    w = np.zeros((4 * Dm, 512))
    for r in range(4 * Dm):
        w[r, (7 * r + 3) % 512] = 1.0
    b = np.array([0.25 * r for r in range(4 * Dm)])
    mod = O.modulation(w, b, c)
    assert mod.shape == (2, 4, Dm)
    for bb in range(2):
        for i in range(4):
            for j in range(Dm):
                r = i * Dm + j
                want = _silu(float(c[bb, (7 * r + 3) % 512])) + 0.25 * r
                assert mod[bb, i, j] == pytest.approx(want, rel=1e-14, abs=1e-14)


def test_timestep_mlp_closed_form_with_identity_weights():
    """W1 = 2 I, b1 = -1, W2 = I, b2 = 0.5: c_i = SiLU(2 e_i - 1) + 0.5 with e the
    sinusoidal embedding written out with math.cos / math.sin."""
    I = np.eye(512)
    mw = O.ModelWeights([], None, None, 2 * I, -np.ones(512), I, np.full(512, 0.5), None, None, None, None)
    for t in (0.0, 0.37):
        c = O.timestep_mlp([t], mw)[0]
        for i in range(512):
            f = 10000.0 ** (-(i % 256) / 256.0)
            e = math.cos(1000.0 * t * f) if i < 256 else math.sin(1000.0 * t * f)
            assert c[i] == pytest.approx(_silu(2.0 * e - 1.0) + 0.5, rel=1e-13, abs=1e-14)
    # t = 0: cosine half is 1 -> SiLU(1) + 0.5, sine half 0 -> SiLU(-1) + 0.5
    c0 = O.timestep_mlp([0.0], mw)[0]
    assert c0[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)) + 0.5, rel=1e-15)
    assert c0[300] == pytest.approx(-1.0 / (1.0 + math.e) + 0.5, rel=1e-15)


# --------------------------------------------------------------------------- block: chunk -> branch, SwiGLU order

def _codes(n, k, rng):
    c = rng.integers(0, 0x7E, (n, k)).astype(np.uint8) | (rng.integers(0, 2, (n, k)) << 7).astype(np.uint8)
    return O.Fp8Weight(c, np.full(n, 0.02 * 3 / 448, np.float32))


def _block_with_mod(rng, chunks, gate_up=None, down=None):
    """Random FP8 block whose modulation is the constant vector chunks[i] per chunk
    (W_mod = 0, b_mod = chunk values), so mod does not depend on c."""
    mod_b = np.concatenate([np.full(D, v, np.float32) for v in chunks])
    return O.BlockWeights(_codes(3 * D, D, rng), _codes(D, D, rng),
                          gate_up if gate_up is not None else _codes(2 * F, D, rng),
                          down if down is not None else _codes(D, F, rng),
                          N.bf16_round(1 + rng.normal(0, 0.02, 256)), N.bf16_round(1 + rng.normal(0, 0.02, 256)),
                          np.zeros((4 * D, 512)), mod_b)


@pytest.mark.parametrize("chunks", [(0.7, 0.0, -1.0, 0.5),     # gate_a = 0, scale_m = -1
                                    (-1.0, 0.5, 0.7, 0.0)])    # scale_a = -1, gate_m = 0
def test_block_identity_needs_the_right_chunk_in_each_branch(chunks):
    """Each branch is switched off by a different chunk, the other branch by its
    own scale -1 (a zero row quantises to zero).  Output == input only if
    scale_a feeds the attention norm, gate_a the attention residual, scale_m the
    MLP norm and gate_m the MLP residual; the other chunk of each pair is
    non-trivial, so any swap adds a non-zero update."""
    rng = np.random.default_rng(102)
    w = _block_with_mod(rng, chunks)
    x = N.bf16_round(rng.normal(0, 1, (1, 2 + 4, D)))
    c = rng.normal(0, 1, (1, 512))
    assert np.array_equal(O.block_forward(x, c, w, 2, 2, 2, O.TINY), x)


def test_block_mlp_only_update_by_hand():
    """gate_a = 0 switches the attention branch off; the MLP is built so that its
    result is a closed form: x = 1 everywhere normalises (eps 1e-6) to
    1 / sqrt(1 + 1e-6), which times (1 + scale_m) = 1 rounds to exactly 1 in
    bf16 and quantises exactly (alpha 1, code 448).  The gate row 0 and up row 0
    read only k = 0, with codes +1 and -1 and channel scales 2 and 1, so g = 2
    and u = -1 there and 0 elsewhere; s = bf16(SiLU(g) * u).  Every down row
    reads s[0] with weight 1, and gate_m = 0.5, so every output element is
    bf16(1 + 0.5 * s0).  scale_a = 0.75 is non-zero so that a norm reading the
    wrong scale changes the result, and g*SiLU(u) instead of SiLU(g)*u gives a
    different s0."""
    rng = np.random.default_rng(103)
    gu = np.zeros((2 * F, D), np.uint8)
    gu[0, 0] = 0x38                      # +1.0
    gu[F, 0] = 0xB8                      # -1.0
    gs = np.ones(2 * F, np.float32)
    gs[0] = 2.0
    dn = np.zeros((D, F), np.uint8)
    dn[:, 0] = 0x38
    w = _block_with_mod(rng, (0.75, 0.0, 0.0, 0.5), gate_up=O.Fp8Weight(gu, gs),
                        down=O.Fp8Weight(dn, np.ones(D, np.float32)))
    L = 2 + 4
    x = np.ones((1, L, D))
    out = O.block_forward(x, rng.normal(0, 1, (1, 512)), w, 2, 2, 2, O.TINY)
    s0 = _bf16(_silu(2.0) * -1.0)
    assert s0 == -1.7578125
    want = _bf16(1.0 + 0.5 * s0)
    assert np.all(out == want)
    assert want == 0.12109375


# --------------------------------------------------------------------------- NF4 operand

def test_nf4_linear_rounds_the_dequantised_weight_to_bf16():
    """Brute force with torch: w = bf16(fp32(code) * fp32(absmax)), then a
    float64 sum of products with the bf16 activation.  The absmax values are
    chosen so that code * absmax is rarely a bf16 value."""
    rng = np.random.default_rng(104)
    n, k, m = 3, 128, 2
    q = rng.integers(0, 16, (n, k))
    packed = ((q[:, 0::2] << 4) | q[:, 1::2]).astype(np.uint8)
    absmax = rng.uniform(0.011, 0.013, n * k // 64).astype(np.float32)
    a = N.bf16_round(rng.normal(0, 1, (m, k)))
    code = torch.tensor(N.nf4_codebook(), dtype=torch.float32)
    w = torch.empty(n, k, dtype=torch.float64)
    for i in range(n):
        for j in range(k):
            prod = code[int(q[i, j])] * torch.tensor(absmax[(i * k + j) // 64], dtype=torch.float32)
            w[i, j] = prod.to(torch.bfloat16).to(torch.float64)
    assert not torch.equal(w, torch.tensor(N.nf4_dequant_f32(packed, absmax, n, k), dtype=torch.float64))
    y = O.nf4_linear(a, packed, absmax, n, k)
    for i in range(m):
        for j in range(n):
            acc = sum(float(a[i, t]) * float(w[j, t]) for t in range(k))
            assert y[i, j] == pytest.approx(acc, rel=1e-13, abs=1e-13)


# --------------------------------------------------------------------------- rotary and QK norm

def test_mrope_rotates_a_unit_pair_counterclockwise():
    """(u_j, u_{j+64}) = (1, 0) at position p goes to (cos(p w_j), sin(p w_j)),
    w_j = 5e6**(-j/64), and (0, 1) to (-sin, cos) (RoFormer's rotary matrix)."""
    d = O.IDEOGRAM4
    pos = np.array([[7, 11, 13]])
    for j, p in ((0, 7), (10, 7), (30, 11), (50, 13)):
        u = np.zeros((1, 1, 256))
        u[0, 0, j] = 1.0
        ang = p * 5e6 ** (-j / 64.0)
        r = O.apply_mrope(u, *O.mrope_cos_sin(pos, d), d)[0, 0]
        assert r[j] == pytest.approx(math.cos(ang), abs=1e-7)
        assert r[j + 64] == pytest.approx(math.sin(ang), abs=1e-7)
        u = np.zeros((1, 1, 256))
        u[0, 0, j + 64] = 1.0
        r = O.apply_mrope(u, *O.mrope_cos_sin(pos, d), d)[0, 0]
        assert r[j] == pytest.approx(-math.sin(ang), abs=1e-7)
        assert r[j + 64] == pytest.approx(math.cos(ang), abs=1e-7)


def test_qk_norm_multiplies_by_gamma():
    """At position 0 the rotation is the identity; a row of +-1 normalises to
    +-1/sqrt(1 + 1e-6), which times a power-of-two gamma rounds to +-gamma in
    bf16.  A second case with a non-power-of-two gamma is checked by hand."""
    d = O.IDEOGRAM4
    rng = np.random.default_rng(105)
    u = np.where(rng.random((1, 2, 256)) < 0.5, -1.0, 1.0)
    gamma = 2.0 ** rng.integers(-3, 3, 256).astype(np.float64)
    c, s = O.mrope_cos_sin(np.zeros((1, 3), np.int64), d)
    out = O.qk_norm_rope(u, gamma, c, s, d)
    assert np.array_equal(out, u * gamma[None, None, :])
    g2 = N.bf16_round(1 + rng.normal(0, 0.1, 256))
    x = N.bf16_round(rng.normal(0, 1, (1, 1, 256)))
    out = O.qk_norm_rope(x, g2, c, s, d)[0, 0]
    r = math.sqrt(sum(float(v) ** 2 for v in x[0, 0]) / 256.0 + 1e-6)
    for t in range(256):
        assert out[t] == _bf16(float(x[0, 0, t]) / r * float(g2[t]))


# --------------------------------------------------------------------------- block: residual chaining, V and O wiring

def test_block_is_the_attention_half_then_the_mlp_half():
    """The MLP branch reads x1, the output of the attention branch: one block with
    chunks (sa, ga, sm, gm) equals the block with the MLP switched off
    (sm = -1) followed by the block with the attention switched off (sa = -1),
    with the same projection weights."""
    rng = np.random.default_rng(106)
    proj = _block_with_mod(rng, (0, 0, 0, 0))
    chunks = (0.3, 0.6, -0.2, 0.8)

    def with_mod(ch):
        return O.BlockWeights(proj.qkv, proj.o, proj.gate_up, proj.down, proj.q_norm, proj.k_norm, proj.mod_w,
                              np.concatenate([np.full(D, v, np.float32) for v in ch]))

    x = N.bf16_round(rng.normal(0, 1, (1, 2 + 4, D)))
    c = rng.normal(0, 1, (1, 512))
    one = O.block_forward(x, c, with_mod(chunks), 2, 2, 2, O.TINY)
    half = O.block_forward(x, c, with_mod((chunks[0], chunks[1], -1.0, 0.0)), 2, 2, 2, O.TINY)
    two = O.block_forward(half, c, with_mod((-1.0, 0.0, chunks[2], chunks[3])), 2, 2, 2, O.TINY)
    assert not np.array_equal(half, x) and not np.array_equal(two, half)
    assert np.array_equal(one, two)


def test_block_value_rows_and_output_projection_by_hand():
    """x = 1 everywhere and scale_a = 0 give h = 1 (quantised exactly).  The v
    rows of the QKV weight read only k = 0, so every token's v is the row of
    code values dec(c_n), identical across tokens: attention returns it
    unchanged whatever the scores.  One code is 448, so o quantises exactly.
    Output row j of W_o reads o[perm(j)] with weight 1, gate_a = 0.5 and the
    MLP is off (scale_m = -1): x1[j] = bf16(1 + 0.5 dec(c_perm(j)))."""
    rng = np.random.default_rng(107)
    vc = (rng.integers(0, 0x7E, D) | (rng.integers(0, 2, D) << 7)).astype(np.uint8)
    vc[5] = 0x7E
    qkv = _codes(3 * D, D, rng)
    qkv.codes[2 * D:] = 0
    qkv.codes[2 * D:, 0] = vc
    qkv.scale[2 * D:] = 1.0
    perm = rng.permutation(D)
    oc = np.zeros((D, D), np.uint8)
    oc[np.arange(D), perm] = 0x38
    w = _block_with_mod(rng, (0.0, 0.5, -1.0, 0.0))
    w = O.BlockWeights(qkv, O.Fp8Weight(oc, np.ones(D, np.float32)), w.gate_up, w.down, w.q_norm, w.k_norm,
                       w.mod_w, w.mod_b)
    out = O.block_forward(np.ones((1, 6, D)), rng.normal(0, 1, (1, 512)), w, 2, 2, 2, O.TINY)
    dec = [float(torch.tensor([int(v)], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)[0])
           for v in vc]
    want = np.array([_bf16(1.0 + 0.5 * dec[perm[j]]) for j in range(D)])
    assert np.all(out == want[None, None, :])
