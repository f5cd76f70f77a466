// Multi-step sampler: the time grid, the presets and the loop of guided
// Euler steps.
//
// Research note, "Training method": the noise schedule is logit-normal with
// parameters (mu, std), mu shifted by 0.5 * log(num_pixels / 512^2) with the
// image size; inference integrates dz/dt = v with Euler steps z_{t - dt} =
// z_t + v dt; the guidance weight may change along the trajectory (a lower
// weight for the last, "polish" steps near t = 0).  Research note, "Infra":
// the presets V4_QUALITY_48 (48 steps, 45 at guidance 7 + 3 at 3, mu 0.0, std
// 1.5), V4_DEFAULT_20 (20, 18 + 2, mu 0.0, std 1.75) and V4_TURBO_12 (12,
// 11 + 1, mu 0.5, std 1.75).
//
// The grid (the pages give the distribution, not the grid): t_i =
// sigmoid(mu' + std * Phi^-1(1 - i/N)), i = 0..N, the quantiles of the
// shifted logit-normal distribution at evenly spaced probabilities, so t_0 = 1
// (noise) and t_N = 0 (clean); log is the natural logarithm.  Phi^-1 is found
// by bracketed Newton iteration on the upper-tail probability 0.5 erfc(y /
// sqrt 2), all in double.
//
// sfm_sample enqueues one sfm_cfg_step per grid interval on the caller's
// stream, the first from z into z_out and the rest in place on z_out; all
// checks run before the first step is enqueued.
#include <cmath>

#include "sfm_internal.h"

namespace {

// y >= 0 with 0.5 erfc(y / sqrt 2) = q, for q in (0, 0.5]
double upper_quantile(double q) {
    const double inv_sqrt2 = 0.70710678118654752440, inv_sqrt2pi = 0.39894228040143267794;
    double lo = 0.0, hi = 40.0, y = 1.0;
    for (int it = 0; it < 200; ++it) {
        const double f = 0.5 * std::erfc(y * inv_sqrt2) - q;  // decreasing in y
        if (f > 0)
            lo = y;
        else
            hi = y;
        const double d = inv_sqrt2pi * std::exp(-0.5 * y * y);
        double yn = y + f / d;
        if (!(yn > lo && yn < hi)) yn = 0.5 * (lo + hi);
        const bool done = std::fabs(yn - y) <= 1e-16 * (1.0 + y);
        y = yn;
        if (done || hi - lo <= 1e-300) break;
    }
    return y;
}

// Phi^-1(p), p in (0, 1)
double probit(double p) { return p < 0.5 ? -upper_quantile(p) : upper_quantile(1.0 - p); }

struct Preset {
    int steps, main_steps;
    float g_main, g_polish;
    double mu, std;
};
constexpr Preset kPresets[] = {
    {48, 45, 7.0f, 3.0f, 0.0, 1.5},   // SFM_PRESET_V4_QUALITY_48
    {20, 18, 7.0f, 3.0f, 0.0, 1.75},  // SFM_PRESET_V4_DEFAULT_20
    {12, 11, 7.0f, 3.0f, 0.5, 1.75},  // SFM_PRESET_V4_TURBO_12
};

}  // namespace

extern "C" {

int sfm_time_grid(int n_steps, double mu, double std_dev, int64_t num_pixels, double* t_out) {
    if (n_steps < 1) return sfm::fail(SFM_E_INVALID_ARG, "n_steps < 1");
    if (!t_out) return sfm::fail(SFM_E_INVALID_ARG, "t_out is NULL");
    if (num_pixels < 1) return sfm::fail(SFM_E_INVALID_ARG, "num_pixels < 1");
    if (!std::isfinite(mu) || !std::isfinite(std_dev) || std_dev <= 0)
        return sfm::fail(SFM_E_INVALID_ARG, "mu / std not finite or std <= 0");
    const double m = mu + 0.5 * std::log((double)num_pixels / (512.0 * 512.0));
    t_out[0] = 1.0;
    for (int i = 1; i < n_steps; ++i) {
        const double x = m + std_dev * probit(1.0 - (double)i / n_steps);
        t_out[i] = 1.0 / (1.0 + std::exp(-x));
    }
    t_out[n_steps] = 0.0;
    return SFM_OK;
}

int sfm_preset(int preset, sfm_preset_info* out) {
    if (preset < 0 || preset >= (int)(sizeof kPresets / sizeof kPresets[0]))
        return sfm::fail(SFM_E_INVALID_ARG, "unknown preset %d", preset);
    if (!out) return sfm::fail(SFM_E_INVALID_ARG, "out is NULL");
    const Preset& p = kPresets[preset];
    out->n_steps = p.steps;
    out->n_main = p.main_steps;
    out->guidance_main = p.g_main;
    out->guidance_polish = p.g_polish;
    out->mu = p.mu;
    out->std_dev = p.std;
    return SFM_OK;
}

int sfm_preset_schedule(int preset, int height_px, int width_px, double* t_out, float* guidance_out, int capacity) {
    sfm_preset_info info;
    if (const int st = sfm_preset(preset, &info); st != SFM_OK) return st;
    if (height_px < 1 || width_px < 1) return sfm::fail(SFM_E_INVALID_ARG, "image size < 1 px");
    if (!t_out || !guidance_out) return sfm::fail(SFM_E_INVALID_ARG, "t_out / guidance_out is NULL");
    if (capacity < info.n_steps) return sfm::fail(SFM_E_INVALID_ARG, "capacity %d < %d steps", capacity, info.n_steps);
    if (const int st = sfm_time_grid(info.n_steps, info.mu, info.std_dev, (int64_t)height_px * width_px, t_out);
        st != SFM_OK)
        return st;
    for (int i = 0; i < info.n_steps; ++i) guidance_out[i] = i < info.n_main ? info.guidance_main : info.guidance_polish;
    return info.n_steps;
}

}  // extern "C"

namespace {

int sample(const sfm_context* ctx, const sfm_model_weights* cond, const sfm_model_weights* uncond,
           const uint16_t* text, const int32_t* text_lens, const float* z, float* z_out, const double* t,
           const float* guidance, int n_steps, int B, int T, int gh, int gw, void* ws, size_t ws_bytes, void* stream) {
    if (n_steps < 1) return sfm::fail(SFM_E_INVALID_ARG, "n_steps < 1");
    if (!t || !guidance) return sfm::fail(SFM_E_INVALID_ARG, "t / guidance is NULL");
    for (int i = 0; i <= n_steps; ++i)
        if (!std::isfinite(t[i])) return sfm::fail(SFM_E_INVALID_ARG, "t[%d] not finite", i);
    for (int i = 0; i < n_steps; ++i) {
        if (!std::isfinite(guidance[i])) return sfm::fail(SFM_E_INVALID_ARG, "guidance[%d] not finite", i);
        if (!(t[i] > t[i + 1])) return sfm::fail(SFM_E_INVALID_ARG, "t not decreasing at %d", i);
    }
    for (int i = 0; i < n_steps; ++i) {
        const float* zi = i == 0 ? z : z_out;
        const float ti = (float)t[i], dti = (float)(t[i] - t[i + 1]);
        const int st = text_lens ? sfm_cfg_step_varlen(ctx, cond, uncond, text, text_lens, zi, z_out, ti, dti,
                                                       guidance[i], B, T, gh, gw, nullptr, nullptr, ws, ws_bytes,
                                                       stream)
                                 : sfm_cfg_step(ctx, cond, uncond, text, zi, z_out, ti, dti, guidance[i], B, T, gh,
                                                gw, nullptr, nullptr, ws, ws_bytes, stream);
        if (st != SFM_OK) return st;
    }
    return SFM_OK;
}

}  // namespace

extern "C" {

int sfm_sample(const sfm_context* ctx, const sfm_model_weights* cond, const sfm_model_weights* uncond,
               const uint16_t* text, const float* z, float* z_out, const double* t, const float* guidance,
               int n_steps, int B, int T, int gh, int gw, void* ws, size_t ws_bytes, void* stream) {
    return sample(ctx, cond, uncond, text, nullptr, z, z_out, t, guidance, n_steps, B, T, gh, gw, ws, ws_bytes,
                  stream);
}

int sfm_sample_varlen(const sfm_context* ctx, const sfm_model_weights* cond, const sfm_model_weights* uncond,
                      const uint16_t* text, const int32_t* text_lens, const float* z, float* z_out, const double* t,
                      const float* guidance, int n_steps, int B, int T, int gh, int gw, void* ws, size_t ws_bytes,
                      void* stream) {
    if (!text_lens) return sfm::fail(SFM_E_INVALID_ARG, "text_lens is NULL");
    return sample(ctx, cond, uncond, text, text_lens, z, z_out, t, guidance, n_steps, B, T, gh, gw, ws, ws_bytes,
                  stream);
}

}  // extern "C"
