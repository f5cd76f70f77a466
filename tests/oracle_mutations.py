"""Mutation check of the oracle's CPU pins (run by hand: python tests/oracle_mutations.py).

Each entry plants one plausible single-line mistake in a scratch copy of oracle/dit.py
(the repository itself is not touched) and runs the oracle's CPU pins against that copy;
every mutation must make at least one pin fail.  The list covers the block's wiring
(modulation chunks, SiLU placement, SwiGLU order, gates), the numerics (NF4 operand
rounding, E4M3 scale, RMSNorm epsilon), MRoPE (direction, sections, frequencies, image
positions), attention's scale, the timestep embedding and MLP, the embedder and the final
layer, and the guided Euler update."""

import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_dit.py", "tests/test_oracle_block_pins.py", "tests/test_oracle_numerics.py",
        "tests/test_oracle_mxfp4.py", "tests/test_oracle_sampler.py"]

MUTATIONS = {
    "modulation without SiLU": ("mod = silu(c) @ w.T", "mod = c @ w.T"),
    "MLP norm takes the attention scale": ("h2 = adaln_norm(x1, mod[b, 2][None, :]", "h2 = adaln_norm(x1, mod[b, 0][None, :]"),
    "attention norm takes the MLP scale": ("h = adaln_norm(xb, mod[b, 0][None, :]", "h = adaln_norm(xb, mod[b, 2][None, :]"),
    "attention residual takes the MLP gate": ("x1 = bf16_round(xb[rb] + mod[b, 1][None, :]", "x1 = bf16_round(xb[rb] + mod[b, 3][None, :]"),
    "MLP residual takes the MLP scale": ("x2 = bf16_round(x1 + mod[b, 3][None, :]", "x2 = bf16_round(x1 + mod[b, 2][None, :]"),
    "SwiGLU as g * silu(u)": ("s = bf16_round(silu(g) * u)", "s = bf16_round(g * silu(u))"),
    "NF4 operand not rounded to bf16": ("w = bf16_round(nf4_dequant_f32(packed, absmax, n, k).astype(np.float64)) if",
                                        "w = nf4_dequant_f32(packed, absmax, n, k).astype(np.float64) if"),
    "rotation by -theta": ("out[..., :half] = a * c - b * s\n    out[..., half:dims.rope_dims] = b * c + a * s",
                           "out[..., :half] = a * c + b * s\n    out[..., half:dims.rope_dims] = b * c - a * s"),
    "QK-norm weight ignored": ("n = rms_normalize(u_bf16, dims.eps) * np.asarray(gamma_bf16, np.float64)",
                               "n = rms_normalize(u_bf16, dims.eps)"),
    "MRoPE sections h and w swapped": ("np.where(j < s0 + s1, 1, 2)", "np.where(j < s0 + s1, 2, 1)"),
    "rotary frequencies over the head dim": ("inv_freq = dims.rope_theta ** (-j / npairs)",
                                             "inv_freq = dims.rope_theta ** (-2 * j / dims.head_dim)"),
    "image positions without the text offset": ("pos[T:, 1] = T + r.reshape(-1)", "pos[T:, 1] = r.reshape(-1)"),
    "attention scale 1/d": ("scale = 1.0 / math.sqrt(d)", "scale = 1.0 / d"),
    "E4M3 scale amax/240": ("inv = (np.float32(E4M3_MAX) / safe)", "inv = (np.float32(240.0) / safe)"),
    "RMSNorm epsilon outside the root": ("return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
                                         "return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)"),
    "timestep MLP without SiLU": ("return silu(hdn) @ np.asarray(mw.t_w2", "return hdn @ np.asarray(mw.t_w2"),
    "timestep embedding sin/cos swapped": ("np.concatenate([np.cos(a), np.sin(a)], axis=1)",
                                           "np.concatenate([np.sin(a), np.cos(a)], axis=1)"),
    "timestep embedding without the 1000": ("a = 1000.0 * t[:, None] * f[None, :]", "a = t[:, None] * f[None, :]"),
    "embedder without bias": ("latent @ np.asarray(mw.x_w, np.float64).T + np.asarray(mw.x_b, np.float64)",
                              "latent @ np.asarray(mw.x_w, np.float64).T"),
    "final scale without 1 +": ("* (1.0 + scale_f[:, None, :])", "* (scale_f[:, None, :])"),
    "final projection without bias": ("return hf @ np.asarray(mw.f_w, np.float64).T + np.asarray(mw.f_b, np.float64)",
                                      "return hf @ np.asarray(mw.f_w, np.float64).T"),
    "guidance towards the unconditional velocity": ("v = v_u + guidance * (v_c - v_u)", "v = v_c + guidance * (v_u - v_c)"),
}


def main():
    src = open(os.path.join(ROOT, "oracle", "dit.py")).read()
    survived = []
    for name, (a, b) in MUTATIONS.items():
        assert src.count(a) == 1, f"{name}: the pattern must occur once in oracle/dit.py"
        with tempfile.TemporaryDirectory() as tmp:
            tree = os.path.join(tmp, "tree")
            shutil.copytree(ROOT, tree, ignore=shutil.ignore_patterns(".git", "_work", "gpurun_out", "_build", "*.so"))
            with open(os.path.join(tree, "oracle", "dit.py"), "w") as f:
                f.write(src.replace(a, b))
            r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                                *PINS], cwd=tree, capture_output=True, text=True)
        caught = r.returncode != 0
        print(f"{'caught  ' if caught else 'SURVIVED'} {name}", flush=True)
        if not caught:
            survived.append(name)
    sys.exit(1 if survived else 0)


if __name__ == "__main__":
    main()
