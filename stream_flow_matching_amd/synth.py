"""Seeded synthetic inputs and weights for the DiT block / CFG-step workloads.

This module holds no arithmetic of the method itself: it only draws random
numbers and packs them into the storage formats the library consumes (bf16
activations, FP8-E4M3 codes with a per-output-channel fp32 scale, NF4 nibbles
with a per-64-block fp32 absmax).  Both the GPU library's callers and the CPU
checker take their inputs from here, so the two always see identical bytes.

Every tensor is drawn from its own ``torch.Generator`` whose seed is a stable
hash of a key tuple (workload, weight set, layer, tensor name), so any single
layer can be regenerated on its own.  CPU and GPU generators produce different
streams for the same seed; parity tests therefore draw on the CPU and copy.

Weight recipe (the released checkpoint is FP8 E4M3, per the deployment post's
quantisation section; NF4 block 64 per its NF4 subsection):
  * FP8: w ~ N(0, 0.02**2); s[n] = max_k |w[n, k]| / 448; codes = E4M3(w / s)
    via torch's float8_e4m3fn cast after clamping to +-448.
  * NF4: nibble codes uniform over the 16 levels (normal-quantile levels are
    near-equiprobable for normal weights), one element per 64-block forced to
    an extreme level (+-1, the absmax element), absmax = max |N(0, 0.02**2)|
    over 64 draws.
  * MXFP4 (the 4-bit FFN layers of the mixed scheme, deployment post section
    2.2): the code and scale frequencies that OCP MX quantisation of
    N(0, 0.02**2) weights produces (tables below, worked out offline from the
    normal distribution): each 32-block draws its E8M0 exponent (119, 120, 121
    with probability 0.0179, 0.9268, 0.0553), each element a magnitude code
    0..7 from that exponent's row and a random sign, and one element per block
    is forced to +-6 (the block maximum).  Weight rms 0.020, as for FP8.  The
    "mixed" block keeps QKV and the output projection in FP8 and puts gate/up
    and down in MXFP4.
  * small layers (latent embed, timestep MLP, final layer): N(0, 1/fan_in) in
    bf16; modulation weights N(0, 0.02**2) bf16 with zero bias; QK-norm
    weights 1 + N(0, 0.02**2) in bf16.
"""

from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import numpy as np
import torch

E4M3_LIMIT = 448.0


def seed_of(*key) -> int:
    """Stable 63-bit seed from a tuple of ints / strings."""
    ints = []
    for k in key:
        if isinstance(k, str):
            ints.append(zlib.crc32(k.encode()))
        else:
            ints.append(int(k) & 0xFFFFFFFF)
    ss = np.random.SeedSequence(ints)
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def _gen(key, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*key))
    return g


def randn(shape, key, std=1.0, device="cpu") -> torch.Tensor:
    """float32 N(0, std**2) tensor."""
    x = torch.randn(*shape, generator=_gen(key, device), device=device, dtype=torch.float32)
    return x.mul_(std) if std != 1.0 else x


def bf16_normal(shape, key, std=1.0, mean=0.0, device="cpu") -> torch.Tensor:
    x = randn(shape, key, std, device)
    if mean:
        x.add_(mean)
    return x.to(torch.bfloat16)


def fp8_weight(n, k, key, std=0.02, device="cpu"):
    """(codes uint8 [n, k], scale float32 [n]) per the FP8 recipe above."""
    w = randn((n, k), key, std, device)
    s = w.abs().amax(dim=1) / E4M3_LIMIT
    w.div_(s[:, None]).clamp_(-E4M3_LIMIT, E4M3_LIMIT)
    codes = w.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), s.contiguous()


def nf4_weight(n, k, key, std=0.02, device="cpu"):
    """(packed uint8 [n, k/2], absmax float32 [n*k/64]) per the NF4 recipe above.

    Element 2i of a row is the high nibble of byte i, 2i+1 the low nibble.
    """
    if k % 64:
        raise ValueError("k must be a multiple of 64 for NF4 blocks")
    g = _gen(key + ("codes",), device)
    q = torch.randint(0, 16, (n, k), generator=g, device=device, dtype=torch.int32)
    nb = n * k // 64
    where = torch.randint(0, 64, (nb,), generator=g, device=device)
    ext = torch.where(torch.rand(nb, generator=g, device=device) < 0.5, 0, 15).to(torch.int32)
    qb = q.view(nb, 64)
    qb.scatter_(1, where[:, None], ext[:, None])
    draws = randn((nb, 64), key + ("absmax",), std, device)
    absmax = draws.abs().amax(dim=1).contiguous()
    packed = ((q[:, 0::2] << 4) | q[:, 1::2]).to(torch.uint8).contiguous()
    return packed, absmax


# MXFP4 recipe tables: block exponents 119, 120, 121 and, per exponent, the
# frequencies of the magnitude codes 0..7
_MX_EXP_P = (0.0179, 0.9268, 0.0553)
_MX_CODE_P = ((0.0389, 0.0775, 0.0764, 0.0746, 0.1072, 0.1311, 0.1654, 0.3289),
              (0.0778, 0.1527, 0.1442, 0.1311, 0.1654, 0.1572, 0.1208, 0.0508),
              (0.1549, 0.2872, 0.2291, 0.1572, 0.1208, 0.0446, 0.0061, 0.0001))


def mxfp4_weight(n, k, key, device="cpu"):
    """(packed uint8 [n, k/2], exponents uint8 [n, k/32]) per the MXFP4 recipe above.

    Element 2i of a row is the low nibble of byte i, 2i+1 the high nibble.
    """
    if k % 32:
        raise ValueError("k must be a multiple of 32 for MXFP4 blocks")
    g = _gen(key + ("codes",), device)
    nb = n * k // 32
    ue = torch.rand(nb, generator=g, device=device)
    ei = (ue >= _MX_EXP_P[0]).to(torch.int32) + (ue >= _MX_EXP_P[0] + _MX_EXP_P[1]).to(torch.int32)
    cdf = torch.tensor(np.cumsum(_MX_CODE_P, axis=1)[:, :7], dtype=torch.float32, device=device)
    rows = cdf[ei.long()]                                   # [nb, 7]
    u = torch.rand(nb, 32, generator=g, device=device)
    q = torch.zeros(nb, 32, dtype=torch.int32, device=device)
    for j in range(7):
        q += (u >= rows[:, j:j + 1]).to(torch.int32)
    q = q.view(n, k)
    del rows, u
    q += 8 * torch.randint(0, 2, (n, k), generator=g, device=device, dtype=torch.int32)
    where = torch.randint(0, 32, (nb,), generator=g, device=device)
    ext = torch.where(torch.rand(nb, generator=g, device=device) < 0.5, 7, 15).to(torch.int32)
    q.view(nb, 32).scatter_(1, where[:, None], ext[:, None])
    e = (119 + ei).view(n, k // 32).to(torch.uint8)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).to(torch.uint8).contiguous()
    return packed, e.contiguous()


# --------------------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Shape:
    emb_dim: int
    num_heads: int
    intermediate: int
    adaln_dim: int = 512
    latent_ch: int = 128


FULL = Shape(4608, 18, 12288)
TINY = Shape(512, 2, 1536)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    B: int
    T: int
    gh: int
    gw: int
    wfmt: str = "fp8"          # "fp8" | "nf4"
    layers: int = 1
    describe: str = ""

    @property
    def L(self):
        return self.T + self.gh * self.gw


# The five workloads: sizes follow the spec table (1024^2 -> 64x64 tokens,
# text <= 2048, aspect up to 6:1), the 512-token projected text cache, and the
# 2048x352 extreme-aspect case.
WORKLOADS = {
    "tiny_block": Workload("tiny_block", TINY, 1, 16, 16, 16,
                           describe="emb 512 (2x256 heads), F 1536, 16 text + 16x16 image tokens"),
    "block_1024": Workload("block_1024", FULL, 1, 512, 64, 64,
                           describe="full-width block at 1024^2: 512 text + 64x64 image tokens (L 4608)"),
    "cfg_step_1024": Workload("cfg_step_1024", FULL, 1, 512, 64, 64, layers=34,
                              describe="34-layer cond (512 text + 4096 image) + image-only uncond, CFG 4.0"),
    "block_2048": Workload("block_2048", FULL, 1, 2048, 128, 128,
                           describe="full-width block at 2048^2: 2048 text + 128x128 image tokens (L 18432)"),
    "block_6to1_nf4": Workload("block_6to1_nf4", FULL, 4, 256, 128, 22, wfmt="nf4",
                               describe="batch 4 of 2048x352 (128x22 tokens) + 256 text, NF4 weights"),
}


@dataclass
class BlockParams:
    """Raw (CPU or device) tensors of one block's weights."""
    fmt: str
    qkv: tuple
    o: tuple
    gate_up: tuple
    down: tuple
    q_norm: torch.Tensor      # bf16 [256]
    k_norm: torch.Tensor      # bf16 [256]
    mod_w: torch.Tensor       # bf16 [4D, 512]
    mod_b: torch.Tensor       # f32 [4D]


TEXT_FEATURES = 13 * 4096   # raw text-encoder width: 13 hidden states of 4096


def text_proj_params(D, k, key, device="cpu"):
    """Text-conditioning projection: norm weight 1 + N(0, 0.02) (bf16) and FP8
    projection weights [D][k] from N(0, 0.02) with per-channel scales."""
    norm_w = bf16_normal((k,), key + ("norm",), 0.02, 1.0, device)
    wq, ws = fp8_weight(D, k, key + ("proj",), device=device)
    return norm_w, wq, ws


def text_raw(M, k, key, device="cpu"):
    """Raw text-encoder features, fp32 N(0, 1) [M][k]."""
    return randn((M, k), key + ("raw",), 1.0, device)


def block_params(shape: Shape, key, fmt="fp8", device="cpu") -> BlockParams:
    """fmt "fp8", "nf4", or "mixed" (QKV and output projection FP8, gate/up and down MXFP4)."""
    D, F = shape.emb_dim, shape.intermediate
    mk = fp8_weight if fmt in ("fp8", "mixed") else nf4_weight
    mk_ffn = (lambda n, k, key, device: mxfp4_weight(n, k, key, device)) if fmt == "mixed" else mk
    return BlockParams(
        fmt=fmt,
        qkv=mk(3 * D, D, key + ("qkv",), device=device),
        o=mk(D, D, key + ("o",), device=device),
        gate_up=mk_ffn(2 * F, D, key + ("gate_up",), device=device),
        down=mk_ffn(D, F, key + ("down",), device=device),
        q_norm=bf16_normal((256,), key + ("q_norm",), 0.02, 1.0, device),
        k_norm=bf16_normal((256,), key + ("k_norm",), 0.02, 1.0, device),
        mod_w=bf16_normal((4 * D, shape.adaln_dim), key + ("mod_w",), 0.02, device=device),
        mod_b=torch.zeros(4 * D, dtype=torch.float32, device=device),
    )


@dataclass
class ModelParams:
    blocks: list
    x_w: torch.Tensor
    x_b: torch.Tensor
    t_w1: torch.Tensor
    t_b1: torch.Tensor
    t_w2: torch.Tensor
    t_b2: torch.Tensor
    f_mod_w: torch.Tensor
    f_mod_b: torch.Tensor
    f_w: torch.Tensor
    f_b: torch.Tensor


def model_params(shape: Shape, layers, key, device="cpu", fmt="fp8", workers=1) -> ModelParams:
    """fmt: the blocks' weight format, "fp8" or "mixed".  workers > 1 draws the
    blocks in a thread pool (each tensor has its own generator, so the bytes
    are the same as with one worker)."""
    D, A, C = shape.emb_dim, shape.adaln_dim, shape.latent_ch
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            blocks = list(ex.map(lambda i: block_params(shape, key + ("layer", i), fmt, device), range(layers)))
    else:
        blocks = [block_params(shape, key + ("layer", i), fmt, device) for i in range(layers)]
    return ModelParams(
        blocks=blocks,
        x_w=bf16_normal((D, C), key + ("x_w",), C ** -0.5, device=device),
        x_b=randn((D,), key + ("x_b",), 0.02, device),
        t_w1=bf16_normal((A, A), key + ("t_w1",), A ** -0.5, device=device),
        t_b1=randn((A,), key + ("t_b1",), 0.02, device),
        t_w2=bf16_normal((A, A), key + ("t_w2",), A ** -0.5, device=device),
        t_b2=randn((A,), key + ("t_b2",), 0.02, device),
        f_mod_w=bf16_normal((D, A), key + ("f_mod_w",), 0.02, device=device),
        f_mod_b=torch.zeros(D, dtype=torch.float32, device=device),
        f_w=bf16_normal((C, D), key + ("f_w",), D ** -0.5, device=device),
        f_b=randn((C,), key + ("f_b",), 0.02, device),
    )


def block_inputs(w: Workload, seed=0, device="cpu"):
    """x [B, L, D] bf16 ~ N(0, 1) and the AdaLN input c [B, 512] ~ N(0, 1)."""
    D = w.shape.emb_dim
    x = bf16_normal((w.B, w.L, D), (seed, w.name, "x"), device=device)
    c = randn((w.B, w.shape.adaln_dim), (seed, w.name, "c"), device=device)
    return x, c


def step_inputs(w: Workload, seed=0, device="cpu"):
    """Inputs of one guided Euler step.

    text [B, T, D] bf16 ~ N(0, 1) (already-projected 4608-d features), latent z
    [B, gh*gw, 128] fp32 ~ N(0, 1), t = sigmoid(mu + std * n) with mu 0.0 and
    std 1.5 (logit-normal draw), t_next = max(0, t - 1/48), dt = t - t_next.
    """
    D = w.shape.emb_dim
    text = bf16_normal((w.B, w.T, D), (seed, w.name, "text"), device=device)
    z = randn((w.B, w.gh * w.gw, w.shape.latent_ch), (seed, w.name, "z"), device=device)
    n = float(randn((1,), (seed, w.name, "t"))[0])
    t = 1.0 / (1.0 + np.exp(-(0.0 + 1.5 * n)))
    t = float(np.float32(t))
    t_next = max(0.0, t - 1.0 / 48.0)
    dt = float(np.float32(t - t_next))
    return text, z, t, dt
