"""Oracle multi-step sampler: the logit-normal time grid with the resolution
shift, the V4 presets (step count, guidance with a polish tail, mu, std) and
the Euler loop over guided steps.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  [Note] "Training method": the noise schedule is logit-normal with parameters
         (mu, std); mu is shifted with the image size by
         0.5 * log(num_pixels / (512 * 512)); inference integrates the velocity
         ODE with Euler steps z_{t - dt} = z_t + v dt; the guidance weight may
         change along the trajectory, the last steps near t = 0 being "polish"
         steps at a lower weight.
  [Note] "Infra": the presets V4_QUALITY_48 (48 steps, 45 at guidance 7 then 3
         at 3, mu 0.0, std 1.5; the default), V4_DEFAULT_20 (20 steps, 18 + 2,
         mu 0.0, std 1.75) and V4_TURBO_12 (12 steps, 11 + 1, mu 0.5, std 1.75).

Readings (the pages give the distribution, not the grid):
  * log is the natural logarithm;
  * the N + 1 times are the quantiles of the shifted logit-normal distribution
    at evenly spaced probabilities: t_i = sigmoid(mu' + std * Phi^-1(1 - i/N)),
    so t_0 = 1 (pure noise) and t_N = 0 (the clean latent), and step i uses
    t = t_i, dt = t_i - t_{i+1} > 0;
  * a garbled sigma formula on another page ([Deploy] section 6) is not used.

All arithmetic is float64; the inverse normal CDF is Python's
statistics.NormalDist (a library primitive).
"""

from __future__ import annotations

import math
from statistics import NormalDist

from . import dit

# name: (steps, steps at the main guidance, main guidance, polish guidance, mu, std)
PRESETS = {
    "V4_QUALITY_48": (48, 45, 7.0, 3.0, 0.0, 1.5),
    "V4_DEFAULT_20": (20, 18, 7.0, 3.0, 0.0, 1.75),
    "V4_TURBO_12": (12, 11, 7.0, 3.0, 0.5, 1.75),
}


def shifted_mu(mu, num_pixels):
    """Resolution-adjusted location of the logit-normal schedule ([Note]
    "Training method")."""
    return mu + 0.5 * math.log(num_pixels / (512.0 * 512.0))


def time_grid(n, mu, std, num_pixels):
    """t_0 = 1 > t_1 > ... > t_N = 0: quantiles of sigmoid(N(mu', std^2)) at
    probabilities 1 - i/N."""
    m = shifted_mu(mu, num_pixels)
    nd = NormalDist()
    t = [1.0]
    for i in range(1, n):
        x = m + std * nd.inv_cdf(1.0 - i / n)
        t.append(1.0 / (1.0 + math.exp(-x)))
    t.append(0.0)
    return t


def guidance_schedule(preset):
    """Per-step guidance weights of a preset: the main weight, then the polish
    weight for the last steps."""
    n, n_main, g_main, g_polish, _, _ = PRESETS[preset]
    return [g_main] * n_main + [g_polish] * (n - n_main)


def preset_grid(preset, height_px, width_px):
    """(t grid, guidance list) of a preset at an image size in pixels."""
    n, _, _, _, mu, std = PRESETS[preset]
    return time_grid(n, mu, std, height_px * width_px), guidance_schedule(preset)


def euler_loop(step, z, t, guidance):
    """z after len(guidance) guided Euler steps: step(z, t_i, dt_i, w_i) returns
    the next latent; dt_i = t_i - t_{i+1}."""
    for i, w in enumerate(guidance):
        z = step(z, t[i], t[i] - t[i + 1], w)
    return z


def sample(text_bf16, z, t, guidance, cond, uncond, gh, gw, dims):
    """The full sampler over the oracle's guided step (dit.cfg_step)."""
    batch = len(z)

    def step(zc, ti, dti, w):
        return dit.cfg_step(text_bf16, zc, [ti] * batch, dti, w, cond, uncond, gh, gw, dims)[0]
    return euler_loop(step, z, t, guidance)
