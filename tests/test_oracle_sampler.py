"""Pins of the oracle sampler (oracle/sampler.py) against the pages' preset
table, closed forms of the logit-normal quantile grid, scipy's normal quantile
and exactly solvable ODEs."""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit, ndtri

from oracle import dit, sampler as S

HERE = os.path.dirname(__file__)


def test_presets_match_the_research_note():
    gold = json.load(open(os.path.join(HERE, "golden", "sampler_presets.json")))["presets"]
    assert set(gold) == set(S.PRESETS)
    for name, g in gold.items():
        n, n_main, g_main, g_pol, mu, std = S.PRESETS[name]
        assert (n, n_main, n - n_main) == (g["steps"], g["main_steps"], g["polish_steps"])
        assert (g_main, g_pol, mu, std) == (g["main_guidance"], g["polish_guidance"], g["mu"], g["std"])
        w = S.guidance_schedule(name)
        assert len(w) == n and w[:n_main] == [g_main] * n_main and w[n_main:] == [g_pol] * (n - n_main)


@pytest.mark.parametrize("n", [1, 2, 12, 20, 48])
def test_grid_endpoints_and_order(n):
    t = S.time_grid(n, 0.3, 1.5, 1024 * 1024)
    assert len(t) == n + 1 and t[0] == 1.0 and t[-1] == 0.0
    assert all(a > b for a, b in zip(t, t[1:]))


def test_resolution_shift_closed_form():
    assert S.shifted_mu(0.0, 512 * 512) == 0.0
    assert math.isclose(S.shifted_mu(0.25, 1024 * 1024), 0.25 + math.log(2.0), rel_tol=0, abs_tol=1e-15)
    assert math.isclose(S.shifted_mu(0.0, 2048 * 2048), 2.0 * math.log(2.0), rel_tol=0, abs_tol=1e-15)


def test_grid_median_is_the_sigmoid_of_the_shifted_mu():
    # Phi^-1(1/2) = 0, and sigmoid(log 2) = 2/3 exactly
    t = S.time_grid(48, 0.0, 1.5, 1024 * 1024)
    assert abs(t[24] - 2.0 / 3.0) < 1e-15


def test_grid_is_symmetric_without_shift():
    t = S.time_grid(20, 0.0, 1.75, 512 * 512)
    for i in range(21):
        assert abs(t[i] + t[20 - i] - 1.0) < 1e-15


@pytest.mark.parametrize("preset", sorted(S.PRESETS))
def test_grid_matches_scipy_quantiles(preset):
    n, _, _, _, mu, std = S.PRESETS[preset]
    for px in (256 * 256, 1024 * 1024, 2048 * 352):
        t = S.time_grid(n, mu, std, px)
        m = mu + 0.5 * np.log(px / 262144.0)
        ref = expit(m + std * ndtri(1.0 - np.arange(1, n) / n))
        assert np.max(np.abs(np.array(t[1:-1]) - ref)) < 1e-14


def test_larger_mu_moves_steps_toward_noise():
    a = S.time_grid(20, 0.0, 1.75, 1024 * 1024)
    b = S.time_grid(20, 0.5, 1.75, 1024 * 1024)
    assert all(y > x for x, y in zip(a[1:-1], b[1:-1]))


def test_euler_loop_constant_velocity_telescopes():
    z0 = np.linspace(-1.0, 1.0, 7)
    v = np.array([0.5, -2.0, 1.0, 0.0, 3.0, -1.0, 0.25])
    t = S.time_grid(48, 0.0, 1.5, 1024 * 1024)
    z = S.euler_loop(lambda z, ti, dt, w: z + dt * v, z0, t, S.guidance_schedule("V4_QUALITY_48"))
    assert np.max(np.abs(z - (z0 + v))) < 1e-13


def test_euler_loop_linear_ode_product_form_and_guidance_order():
    # dz = -z dt per step: z_N = z_0 prod(1 - dt_i); the weights arrive in preset order
    t = S.time_grid(12, 0.5, 1.75, 768 * 1024)
    seen = []

    def step(z, ti, dt, w):
        seen.append((ti, w))
        return z * (1.0 - dt)

    z = S.euler_loop(step, np.array([2.0]), t, S.guidance_schedule("V4_TURBO_12"))
    ref = 2.0 * np.prod([1.0 - (t[i] - t[i + 1]) for i in range(12)])
    assert abs(z[0] - ref) < 1e-15
    assert [w for _, w in seen] == [7.0] * 11 + [3.0]
    assert [ti for ti, _ in seen] == t[:-1]


def test_sample_chains_guided_steps_in_grid_order():
    from oracle import numerics as N
    from test_oracle_dit import _tiny_model
    rng = np.random.default_rng(31)
    cond, unc = _tiny_model(rng, 1), _tiny_model(rng, 1)
    z = rng.normal(0, 1, (1, 4, 128))
    text = N.bf16_round(rng.normal(0, 1, (1, 2, 512)))
    # one step over the whole interval is one guided step at t = 1, dt = 1
    z1 = S.sample(text, z, [1.0, 0.0], [4.0], cond, unc, 2, 2, dit.TINY)
    assert np.array_equal(z1, dit.cfg_step(text, z, [1.0], 1.0, 4.0, cond, unc, 2, 2, dit.TINY)[0])
    # two steps: the second starts from the first's latent at t_1 with its own weight
    t = [1.0, 0.4, 0.0]
    z2 = S.sample(text, z, t, [7.0, 3.0], cond, unc, 2, 2, dit.TINY)
    za = dit.cfg_step(text, z, [1.0], 0.6, 7.0, cond, unc, 2, 2, dit.TINY)[0]
    zb = dit.cfg_step(text, za, [0.4], 0.4, 3.0, cond, unc, 2, 2, dit.TINY)[0]
    assert np.array_equal(z2, zb)
