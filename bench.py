"""Benchmark: one guided Euler flow-matching step of the 34-layer Ideogram-4
shaped DiT at 1024x1024 on one MI355X (conditional pass on 512 text + 4096
image tokens, separate image-only unconditional pass on 4096 tokens, CFG 4.0).

Prints ONE JSON line.  `value` is DiT block tokens/s over the whole step
(34 * (4608 + 4096) block-token passes per step).  The step's TFLOP/s and
fraction of the FP8 matrix peak, the single-block figures at the other
workload shapes, the roofline of the dominant kernel (the FP8 gate/up SwiGLU
projection) and the CPU oracle baseline are reported beside it, and so is the
time of one whole 1024x1024 image with the V4_TURBO_12 and V4_QUALITY_48
sampler presets (12 / 48 guided steps; outside the timed steps).

Inputs are synthetic and seeded (weights FP8 E4M3 from N(0, 0.02), latent and
text N(0, 1), t from the logit-normal draw); all of them are resident in HBM
before the timed region starts.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 matrix peak (datasheet)
BF16_PEAK_TFLOPS = 2500.0     # dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0


def block_flops(L, B, D=4608, F=12288):
    """Algorithmic FLOPs of one block: 2*(4D^2 + 3DF) per token for the four
    projections, 4*L^2*D per sequence for attention."""
    return B * L * 2 * (4 * D * D + 3 * D * F) + B * 4 * L * L * D


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the single-block workloads")
    ap.add_argument("--cpu-sample", default="block_1024", help="workload timed on the CPU oracle")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run only the dominant launch and a calibration copy (for rocprofv3 --pmc passes)")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                    help="print per-kernel counter tables and the traffic records from rocprofv3 --pmc passes "
                         "over --pmc-probe (one output directory per pass) and exit (no GPU needed)")
    ap.add_argument("--no-hbm", action="store_true", help="skip the bandwidth-bound kernels with flushed caches")
    ap.add_argument("--yardstick", action="store_true",
                    help="time the vendor libraries at this path's shapes (hipBLASLt FP8 through torch._scaled_mm, "
                         "bf16 torch.mm, torch's scaled_dot_product_attention) and exit; a context figure, not part "
                         "of the path")
    ap.add_argument("--block-probe", metavar="WORKLOAD",
                    help="run only a few forwards of one block of a named workload (e.g. block_6to1_nf4) and a "
                         "calibration copy (for rocprofv3 kernel-trace and --pmc passes) and exit")
    ap.add_argument("--block-summary", nargs="+", metavar="DIR",
                    help="per-kernel table (markdown) of the block_6to1_nf4 matrix launches from rocprofv3 output "
                         "directories of --block-probe (a kernel trace and/or --pmc passes) and exit (no GPU needed)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="print per-kernel tables (markdown) from a rocprofv3 --kernel-trace --stats output "
                         "directory of this script and exit (no GPU needed)")
    return ap.parse_args()


def time_gpu(fn, iters, warmup=1):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters / 1e3   # seconds per call


class ClockSampler:
    """The GPU's gfx clock (the mean over its XCDs) and socket power, read from the
    amdsmi GPU metrics every `period` seconds by a thread while a workload runs.
    ok is False when amdsmi is missing or the device cannot be identified."""

    def __init__(self, period=0.01):
        import threading
        self.ok, self.period, self.samples = False, period, []
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            self.smi = amdsmi
            amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
            handles = amdsmi.amdsmi_get_processor_handles()
            self.h = handles[0] if len(handles) == 1 else None
            self.ok = self.h is not None
        except Exception:
            self.ok = False

    def read(self):
        m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float))]
        clk = sum(clks) / len(clks) if clks else m.get("current_gfxclk")
        pw = m.get("current_socket_power")
        return (float(clk) if isinstance(clk, (int, float)) else None,
                float(pw) if isinstance(pw, (int, float)) else None)

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self.read())
            except Exception:
                pass
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()
        try:
            self.smi.amdsmi_shut_down()
        except Exception:
            pass
        return False

    def summary(self, what, keep_last=1.0):
        import statistics
        kept = self.samples[int(len(self.samples) * (1.0 - keep_last)):]
        clk = sorted(c for c, _ in kept if c)
        pw = sorted(p for _, p in kept if p)
        if not clk:
            return None
        return {"mhz_median": round(statistics.median(clk), 1), "mhz_min": round(clk[0], 1),
                "mhz_max": round(clk[-1], 1), "socket_power_w_median": round(statistics.median(pw), 1) if pw else None,
                "samples": len(clk), "source": "amdsmi GPU metrics: current gfx clock of each XCD (mean over XCDs), "
                                               f"read every {self.period * 1e3:.0f} ms during {what}"}


def cfg_step_bench(sfm, synth, ctx, steps, warmup, presets=()):
    """Times `steps` CFG steps between two synchronisations; the last timed step
    runs through sfm_cfg_step_timed, which records HIP events on the launch
    stream around the five matrix launches of every block (QKV, attention, O,
    gate/up, down), giving each kernel's launch durations inside the timed
    region (that step runs its two passes one after the other)."""
    import torch
    w = synth.WORKLOADS["cfg_step_1024"]
    cond = synth.model_params(w.shape, w.layers, (0, "cond"), device="cuda")
    unc = synth.model_params(w.shape, w.layers, (0, "uncond"), device="cuda")
    text, z, t, dt = synth.step_inputs(w, device="cuda")
    cm, um = sfm.ModelWeights(cond), sfm.ModelWeights(unc)
    ws = sfm.workspace(sfm.sfm_step_workspace_bytes(ctx, w.B, w.T, w.gh, w.gw))
    zo = torch.empty_like(z)
    nev = 2 * w.layers * len(KINDS)
    evb = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
    eve = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
    for ev in evb + eve:       # creates the HIP events
        ev.record()

    def step():
        sfm.sfm_cfg_step(ctx, cm, um, text, z, zo, t, dt, 4.0, w.B, w.T, w.gh, w.gw, ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the clock under this load: guided steps for about two seconds between the warm-up and
    # the timed steps, with the metrics read beside them (the timed step with events stays the
    # last); the metrics table refreshes far more slowly than it is read, so only the second
    # second's readings count
    clock = None
    sampler = ClockSampler()
    if sampler.ok:
        with sampler:
            t_end = time.perf_counter() + 2.0
            while time.perf_counter() < t_end:
                step()
                torch.cuda.synchronize()
        clock = sampler.summary("guided steps run for 2 s between the warm-up and the timed steps (readings of the "
                                "second second)", keep_last=0.5)
    t0 = time.perf_counter()
    for _ in range(steps - 1):
        step()
    rec = sfm.sfm_cfg_step_timed(ctx, cm, um, text, z, zo, t, dt, 4.0, w.B, w.T, w.gh, w.gw, ws, evb, eve)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    us = [evb[i].elapsed_time(eve[i]) * 1e3 for i in range(rec)]   # microseconds
    nk = len(KINDS)
    # pair (p * layers + l) * 5 + j: pass p (0 conditional, 1 unconditional), layer l, launch j
    launches = {kind: [[us[(p * w.layers + l) * nk + j] for l in range(w.layers) if (p * w.layers + l) * nk + j < rec]
                       for p in range(2)] for j, kind in enumerate(KINDS)}
    ok = bool(torch.isfinite(zo).all())
    # whole images with the sampler presets (outside the timed steps above)
    samples = {}
    for name, pid in presets:
        t_grid, g = sfm.sfm_preset_schedule(pid, 16 * w.gh, 16 * w.gw)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        sfm.sfm_sample(ctx, cm, um, text, z, zo, t_grid, g, w.B, w.T, w.gh, w.gw, ws)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        samples[name] = {"steps": len(g), "s_per_image": round(el, 4), "ms_per_step": round(el / len(g) * 1e3, 3),
                         "finite": bool(torch.isfinite(zo).all())}
    streamed = None
    if presets:
        streamed = {"fp8": streamed_bench(sfm, ctx, cond, cm, text, z, t, w)}
        del cond, unc, cm, um, ws
        torch.cuda.empty_cache()
        mixed = synth.model_params(w.shape, w.layers, (0, "cond"), device="cuda", fmt="mixed")
        streamed["mixed"] = streamed_bench(sfm, ctx, mixed, sfm.ModelWeights(mixed), text, z, t, w,
                                           weights="QKV and output projection FP8, gate/up and down MXFP4")
        del mixed
    torch.cuda.empty_cache()
    return sec, ok, launches, samples, streamed, clock


def streamed_bench(sfm, ctx, cond, cm, text, z, t, w, iters=2, weights="FP8"):
    """The conditional velocity pass (34 layers, 1024^2) with its block weights
    in pinned host memory, streamed layer by layer, against the same pass with
    resident weights.  H2D rate = block weight bytes copied per second."""
    import dataclasses
    import torch

    def pin(o):
        if isinstance(o, torch.Tensor):
            return o.cpu().pin_memory()
        if isinstance(o, tuple):
            return tuple(pin(x) for x in o)
        if dataclasses.is_dataclass(o):
            return dataclasses.replace(o, **{f.name: pin(getattr(o, f.name)) for f in dataclasses.fields(o)})
        return o

    host = dataclasses.replace(cond, blocks=[pin(b) for b in cond.blocks])
    mh = sfm.ModelWeights(host)
    v = torch.empty(w.B, w.gh * w.gw, w.shape.latent_ch, device="cuda")
    ws_s = sfm.workspace(sfm.lib().sfm_streamed_workspace_bytes(ctx.handle, w.B, w.T, w.gh, w.gw))
    ws_r = sfm.workspace(sfm.sfm_step_workspace_bytes(ctx, w.B, w.T, w.gh, w.gw))
    s_str = time_gpu(lambda: sfm.sfm_model_velocity_streamed(ctx, mh, text, z, t, v, w.B, w.T, w.gh, w.gw, ws_s),
                     iters)
    s_res = time_gpu(lambda: sfm.sfm_model_velocity(ctx, cm, text, z, t, v, w.B, w.T, w.gh, w.gw, ws_r), iters)
    blk = sum(x.numel() * x.element_size() for b in host.blocks
              for x in (b.qkv + b.o + b.gate_up + b.down + (b.q_norm, b.k_norm, b.mod_w, b.mod_b)))
    del host, mh, ws_s, ws_r
    return {"workload": "conditional pass, 34 layers at 1024^2, block weights in pinned host memory",
            "weights": weights, "ms_streamed": round(s_str * 1e3, 2), "ms_resident": round(s_res * 1e3, 2),
            "block_weight_bytes": blk, "h2d_gb_s": round(blk / s_str / 1e9, 2)}


def block_bench(sfm, synth, ctx, name, iters=5, fmt=None):
    """One block at a named workload; fmt overrides its weight format ("mixed":
    QKV and output projection FP8, gate/up and down MXFP4, priced against the
    FP8 peak since FP8 x FP4 products run at the FP8 rate)."""
    import torch
    w = synth.WORKLOADS[name]
    fmt = fmt or w.wfmt
    p = synth.block_params(w.shape, (0, w.name), fmt, device="cuda")
    bw = sfm.BlockWeights(p)
    x, c = synth.block_inputs(w, device="cuda")
    xo = torch.empty_like(x)
    ws = sfm.workspace(sfm.sfm_block_workspace_bytes(ctx, w.B, w.T, w.gh, w.gw, bw.fmt))
    sec = time_gpu(lambda: sfm.sfm_block_forward(ctx, bw, x, xo, c, w.B, w.T, w.gh, w.gw, ws), iters)
    fl = block_flops(w.L, w.B)
    peak = BF16_PEAK_TFLOPS if fmt == "nf4" else FP8_PEAK_TFLOPS
    return {"workload": w.describe, "ms": round(sec * 1e3, 4), "tokens_per_s": round(w.B * w.L / sec, 1),
            "tflops": round(fl / sec / 1e12, 2), "frac_matrix_peak": round(fl / sec / 1e12 / peak, 4),
            "weights": fmt}


def block_varlen_bench(sfm, synth, ctx, lens=(512, 77), iters=5):
    """Two 1024^2 prompts of different text lengths in one batch (text padded
    to 512 rows): the block with per-sample lengths.  Tokens counted are the
    real ones (text + image of each sample)."""
    import torch
    w = synth.Workload("block_1024_varlen", synth.FULL, len(lens), 512, 64, 64)
    p = synth.block_params(w.shape, (0, w.name), "fp8", device="cuda")
    bw = sfm.BlockWeights(p)
    x, c = synth.block_inputs(w, device="cuda")
    xo = torch.empty_like(x)
    ws = sfm.workspace(sfm.sfm_block_workspace_bytes(ctx, w.B, w.T, w.gh, w.gw, bw.fmt))
    sec = time_gpu(lambda: sfm.sfm_block_forward_varlen(ctx, bw, x, xo, c, w.B, w.T, list(lens), w.gh, w.gw, ws),
                   iters)
    real = sum(t + w.gh * w.gw for t in lens)
    fl = sum(block_flops(t + w.gh * w.gw, 1) for t in lens)
    return {"workload": f"batch of {len(lens)} at 1024^2 with text lengths {list(lens)} padded to 512",
            "ms": round(sec * 1e3, 4), "tokens_per_s": round(real / sec, 1), "tflops": round(fl / sec / 1e12, 2)}


def attention_bench(sfm, ctx, L, iters=20):
    """sfm_attention alone at one 1024^2 pass's shape (18 heads of 256, batch 1),
    unit-RMS bf16 q and k and N(0,1) V: the balanced persistent grid plus its
    merge of split query blocks.  4 L^2 256 H FLOP against the bf16 peak."""
    import torch
    H, d = 18, 256
    Lp = sfm.sfm_padded_len(L)
    g = torch.Generator(device="cuda").manual_seed(L)
    q = torch.zeros(1, H, Lp, d, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros_like(q)
    vt = torch.zeros(1, H, d, Lp, dtype=torch.float16, device="cuda")
    q[:, :, :L] = torch.randn(1, H, L, d, generator=g, device="cuda").to(torch.bfloat16)
    k[:, :, :L] = torch.randn(1, H, L, d, generator=g, device="cuda").to(torch.bfloat16)
    vt[:, :, :, :L] = torch.randn(1, H, d, L, generator=g, device="cuda").to(torch.float16)
    o = torch.empty(L, H * d, dtype=torch.bfloat16, device="cuda")
    sec = time_gpu(lambda: sfm.sfm_attention(ctx, q, k, vt, o, 1, L), iters)
    fl = 4.0 * L * L * d * H
    return {"workload": f"attention alone, L {L}, 18 heads of 256 (balanced persistent grid + merge)",
            "us": round(sec * 1e6, 1), "tflops": round(fl / sec / 1e12, 2),
            "frac_bf16_peak": round(fl / sec / 1e12 / BF16_PEAK_TFLOPS, 4)}


def text_project_bench(sfm, synth, ctx, M=512, iters=10):
    """The text-conditioning projection of one 512-token prompt: 53,248 raw
    features per token to 4608 (RMSNorm + E4M3 + FP8 GEMM, K 53,248)."""
    import torch
    k, D = synth.TEXT_FEATURES, 4608
    norm_w, wq, ws = synth.text_proj_params(D, k, ("bench_tp",), device="cuda")
    raw = synth.text_raw(M, k, ("bench_tp",), device="cuda")
    w = sfm.qweight(sfm.SFM_W_FP8_E4M3, wq, ws)
    out = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    wsp = sfm.workspace(sfm.lib().sfm_text_project_workspace_bytes(ctx.handle, M, k))
    sec = time_gpu(lambda: sfm.sfm_text_project(ctx, raw, norm_w, w, out, wsp), iters)
    fl = 2.0 * M * k * D
    return {"workload": f"{M} tokens x {k} raw features -> {D}", "us": round(sec * 1e6, 1),
            "tflops": round(fl / sec / 1e12, 2), "frac_fp8_peak": round(fl / sec / 1e12 / FP8_PEAK_TFLOPS, 4)}


KINDS = ("qkv", "attention", "o", "gate_up", "down")   # a block's matrix launches, in launch order
KIND_DESC = {
    "qkv": "gemm_fp8_kernel, QKV projection with QK-RMSNorm + MRoPE in the epilogue (q, k, V^T in the attention layouts), N 13824, K 4608",
    "attention": "attn_kernel on one persistent workgroup per compute unit, with attn_merge_kernel for the "
                 "query blocks split between workgroups (both inside the timed pair): joint attention, 18 heads "
                 "of 256",
    "o": "gemm_fp8_kernel, gated-residual epilogue: output projection, N 4608, K 4608",
    "gate_up": "gemm_fp8_kernel, SwiGLU epilogue: gate/up projection, N 24576, K 4608",
    "down": "gemm_fp8_kernel, gated-residual epilogue: down projection, N 4608, K 12288",
}
KIND_SOURCES = {k: ("stream_flow_matching_amd/csrc/k_gemm_fp8.hip", "stream_flow_matching_amd/csrc/gemm_common.h",
                    "stream_flow_matching_amd/csrc/epi_qkv_rope.h") for k in KINDS}
KIND_SOURCES["attention"] = ("stream_flow_matching_amd/csrc/k_attn.hip",)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "cfg_step_1024_counters.md")
COPY_BYTES = 256 << 20            # plain copy kernel used to calibrate the byte counters
FLUSH_BYTES = 512 << 20           # written before each HBM-bound launch: evicts the 256 MB MALL and the L2s


def kernel_work(kind, L, B=1, D=4608, F=12288):
    """(algorithmic FLOP, algorithmic HBM bytes) of one launch of a block's matrix kernel.
    GEMMs: 2 M N K; bytes = E4M3 activation codes + row scales + weight codes + column
    scales + bf16 output (+ the bf16 residual read for the gated residual).
    Attention: 4 L^2 D per sequence; bytes = q, k (bf16), v^T (fp16) read once, o written."""
    M = B * L
    if kind == "attention":
        return 4.0 * B * L * L * D, 4 * M * D * 2
    n, k = {"qkv": (3 * D, D), "o": (D, D), "gate_up": (2 * F, D), "down": (D, F)}[kind]
    out_cols = n // 2 if kind == "gate_up" else n
    nbytes = M * k + 4 * M + n * k + 4 * n + 2 * M * out_cols + (2 * M * n if kind in ("o", "down") else 0)
    return 2.0 * M * n * k, nbytes


def sources_digest(kind):
    import hashlib
    h = hashlib.sha256()
    for rel in KIND_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kind):
    """HBM bytes per conditional-pass launch of `kind` from the committed counter runs
    (FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for a plain copy of
    COPY_BYTES), or None when the kernel's sources changed since they were taken."""
    try:
        with open(COUNTERS_FILE) as f:
            recs = [json.loads(l.split("traffic-record:", 1)[1]) for l in f if "traffic-record:" in l]
    except (OSError, ValueError):
        return None
    for rec in recs:
        if rec.get("kind") == kind and rec.get("pass") == "cond":
            return rec.get("bytes_per_launch") if rec.get("sources_sha256_16") == sources_digest(kind) else None
    return None


def kernel_table(launches, w):
    """Per matrix kernel of the timed step: average launch time per pass (HIP events
    on the launch stream), algorithmic work, TFLOP/s and fraction of its peak (FP8
    for the projections, bf16 for attention), and its time per step."""
    Lc, Lu = w.T + w.gh * w.gw, w.gh * w.gw
    table = {}
    for kind in KINDS:
        c, u = launches[kind]
        if not c or not u:
            continue
        peak = BF16_PEAK_TFLOPS if kind == "attention" else FP8_PEAK_TFLOPS
        (fc, bc), (fu, _) = kernel_work(kind, Lc), kernel_work(kind, Lu)
        ac, au = sum(c) / len(c), sum(u) / len(u)
        table[kind] = {"kernel": KIND_DESC[kind], "avg_us_cond": round(ac, 2), "avg_us_uncond": round(au, 2),
                       "tflop_per_launch_cond": round(fc / 1e12, 4), "tflops_cond": round(fc / ac / 1e6, 1),
                       "frac_cond": round(fc / ac / 1e6 / peak, 4), "tflops_uncond": round(fu / au / 1e6, 1),
                       "frac_uncond": round(fu / au / 1e6 / peak, 4), "peak_tflops": peak,
                       "algorithmic_bytes_cond": bc, "ms_per_step": round((sum(c) + sum(u)) / 1e3, 3),
                       "launches": [len(c), len(u)]}
    return table


def roofline(table, w):
    """The dominant kernel (the largest time per step among the matrix kernels) at the
    conditional pass's shape: achieved = algorithmic FLOP per launch / average launch
    duration from the events of the timed step; peak = its dtype's dense matrix peak."""
    kind = max(table, key=lambda k: table[k]["ms_per_step"])
    t = table[kind]
    fc, bc = kernel_work(kind, w.T + w.gh * w.gw)
    return {"bound": "mfma", "achieved": t["tflops_cond"], "peak": t["peak_tflops"], "unit": "TFLOP/s",
            "frac": t["frac_cond"], "traffic": measured_traffic(kind), "kernel": t["kernel"],
            "shape": f"conditional pass, L {w.T + w.gh * w.gw}", "avg_launch_us": t["avg_us_cond"],
            "launches": t["launches"][0], "flop_per_launch": fc, "algorithmic_bytes_per_launch": bc,
            "per_kernel": table}


def hbm_kernels(sfm, synth, ctx, iters=5, warm=True):
    """The bandwidth-bound kernels at the 1024^2 conditional shape (M 4608), each
    launched alone after a FLUSH_BYTES write that evicts the Infinity Cache and the
    L2s, timed with HIP events on the launch stream.  Bytes are algorithmic: each
    input read once, each output written once."""
    import torch
    M, D, F, T, g = 4608, 4608, 12288, 512, 64
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    x = synth.bf16_normal((M, D), ("hbm", "x"), device="cuda")
    scale = synth.randn((4 * D,), ("hbm", "mod"), 0.1, device="cuda")
    hq = torch.empty(M, D, dtype=torch.uint8, device="cuda")
    hs = torch.empty(M, dtype=torch.float32, device="cuda")
    sF = synth.bf16_normal((M, F), ("hbm", "s"), device="cuda")
    qF = torch.empty(M, F, dtype=torch.uint8, device="cuda")
    qkv = synth.bf16_normal((M, 3 * D), ("hbm", "qkv"), device="cuda")
    qn = synth.bf16_normal((256,), ("hbm", "qn"), 0.02, 1.0, device="cuda")
    kn = synth.bf16_normal((256,), ("hbm", "kn"), 0.02, 1.0, device="cuda")
    H, Lp = 18, sfm.sfm_padded_len(M)
    q = torch.empty(1, H, Lp, 256, dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    vt = torch.empty(1, H, 256, Lp, dtype=torch.float16, device="cuda")
    n8, k8 = 24576, 4608
    w8 = synth.fp8_weight(n8, k8, ("hbm", "w8"), device="cuda")
    w4 = synth.nf4_weight(n8, k8, ("hbm", "w4"), device="cuda")
    wout = torch.empty(n8, k8, dtype=torch.float32, device="cuda")
    nz = g * g * 128
    z = synth.randn((nz,), ("hbm", "z"), device="cuda")
    vc, vu, zo = torch.randn_like(z), torch.randn_like(z), torch.empty_like(z)
    qw8, qw4 = sfm.qweight(sfm.SFM_W_FP8_E4M3, *w8), sfm.qweight(sfm.SFM_W_NF4_B64, *w4)
    cases = [
        ("adaln_kernel (AdaLN RMSNorm + E4M3 codes)", f"M {M}, D {D}", 3 * M * D + 4 * M + 4 * D,
         lambda: sfm.sfm_adaln_norm_fp8(ctx, x, scale, 4 * D, hq, hs, 1, M)),
        ("quant_rows_kernel (attention output o)", f"M {M}, cols {D}", 3 * M * D + 4 * M,
         lambda: sfm.sfm_quant_rows_fp8(x, hq, hs)),
        ("quant_rows_kernel (SwiGLU output s)", f"M {M}, cols {F}", 3 * M * F + 4 * M,
         lambda: sfm.sfm_quant_rows_fp8(sF, qF, hs)),
        ("qk_norm_rope_kernel (QK-RMSNorm + MRoPE + V^T)", f"T {T}, {g}x{g}, 18 heads", 12 * M * D + 1024,
         lambda: sfm.sfm_qk_norm_rope(ctx, qkv, qn, kn, q, k, vt, 1, T, g, g)),
        ("dequant_fp8_kernel (standalone, fp32 out)", f"{n8} x {k8}", 5 * n8 * k8 + 4 * n8,
         lambda: sfm.sfm_dequant(ctx, qw8, wout)),
        ("dequant_nf4_kernel (standalone, fp32 out)", f"{n8} x {k8}", n8 * k8 // 2 + n8 * k8 // 16 + 4 * n8 * k8,
         lambda: sfm.sfm_dequant(ctx, qw4, wout)),
        ("euler_cfg_kernel", f"{nz} latent values", 16 * nz,
         lambda: sfm.sfm_euler_cfg(z, vc, vu, zo, None, 4.0, 1.0 / 48)),
    ]
    out = []
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, shape, nbytes, fn in cases:
        if warm:
            fn()
        tot = 0.0
        for it in range(iters):
            flush.fill_(it & 0xFF)
            s.record()
            fn()
            e.record()
            e.synchronize()
            tot += s.elapsed_time(e)
        us = tot / iters * 1e3
        out.append({"kernel": name, "shape": shape, "us": round(us, 2), "algorithmic_bytes": nbytes,
                    "gb_s": round(nbytes / us / 1e3, 1), "frac_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)})
    return out


def pmc_probe(sfm, synth, ctx):
    """For the rocprofv3 --pmc passes: one guided step at 1024^2 in the timed
    (sequential) form with both 34-layer weight sets drawn on the device, the
    bandwidth-bound kernels alone after a cache flush, and a plain device copy of
    COPY_BYTES that calibrates the byte counters."""
    import torch
    w = synth.WORKLOADS["cfg_step_1024"]
    cond = synth.model_params(w.shape, w.layers, (0, "cond"), device="cuda")
    unc = synth.model_params(w.shape, w.layers, (0, "uncond"), device="cuda")
    text, z, t, dt = synth.step_inputs(w, device="cuda")
    cm, um = sfm.ModelWeights(cond), sfm.ModelWeights(unc)
    ws = sfm.workspace(sfm.sfm_step_workspace_bytes(ctx, w.B, w.T, w.gh, w.gw))
    zo = torch.empty_like(z)
    torch.cuda.synchronize()
    sfm.sfm_cfg_step_timed(ctx, cm, um, text, z, zo, t, dt, 4.0, w.B, w.T, w.gh, w.gw, ws, [], [])
    torch.cuda.synchronize()
    del cond, unc, cm, um, ws
    torch.cuda.empty_cache()
    hbm_kernels(sfm, synth, ctx, iters=1, warm=False)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_probe": "done", "copy_bytes": COPY_BYTES,
                      "sources_sha256_16": {k: sources_digest(k) for k in KINDS}}))


BLOCK_PROBE_CALLS = 4   # block forwards run by --block-probe (the first one warms up)


def block_probe(sfm, synth, ctx, name):
    """For rocprofv3 runs: BLOCK_PROBE_CALLS forwards of one block of workload `name`
    (weights drawn on the device), then a plain device copy of COPY_BYTES that
    calibrates the byte counters."""
    import torch
    w = synth.WORKLOADS[name]
    p = synth.block_params(w.shape, (0, w.name), w.wfmt, device="cuda")
    bw = sfm.BlockWeights(p)
    x, c = synth.block_inputs(w, device="cuda")
    xo = torch.empty_like(x)
    ws = sfm.workspace(sfm.sfm_block_workspace_bytes(ctx, w.B, w.T, w.gh, w.gw, bw.fmt))
    ms = []
    for _ in range(BLOCK_PROBE_CALLS):
        ms.append(time_gpu(lambda: sfm.sfm_block_forward(ctx, bw, x, xo, c, w.B, w.T, w.gh, w.gw, ws), 1, 0) * 1e3)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"block_probe": name, "weights": w.wfmt, "ms": [round(v, 3) for v in ms],
                      "copy_bytes": COPY_BYTES}))


def block_work(kind, M, wfmt, D=4608, F=12288):
    """(algorithmic FLOP, algorithmic HBM bytes) of one projection of a block with M token
    rows.  NF4 weights: bf16 activation in, packed nibbles + fp32 absmax per 64 weights,
    bf16 out (+ the bf16 residual read for the gated residual); FP8 as kernel_work."""
    if wfmt != "nf4":
        return kernel_work(kind, M)
    n, k = {"qkv": (3 * D, D), "o": (D, D), "gate_up": (2 * F, D), "down": (D, F)}[kind]
    out_cols = n // 2 if kind == "gate_up" else n
    nbytes = 2 * M * k + n * k // 2 + 4 * (n * k // 64) + 2 * M * out_cols + (2 * M * n if kind in ("o", "down") else 0)
    return 2.0 * M * n * k, nbytes


def _block_kinds(order):
    """Label the matrix launches of block forwards (dispatches in launch order): QKV,
    attention, O, gate/up, down; the first forward (the warm-up) is left out."""
    labels, last, n = {}, None, 0
    for r in order:
        k = _short(r["Kernel_Name"])
        kind = None
        if k.startswith("gemm_fp8_kernel<") or k.startswith("gemm_nf4_kernel<"):
            epi = k.split(",")[2].strip().rstrip(">")
            kind = {"0": "qkv", "4": "qkv", "2": "gate_up", "1": "down" if last == "gate_up" else "o"}.get(epi)
        elif k.startswith("attn_kernel"):
            kind = "attention"
        if kind:
            n += kind == "qkv"
            if n > 1:
                labels[r["Dispatch_Id"]] = kind
            last = kind
    return labels


def block_summary(dirs, name="block_6to1_nf4"):
    """Markdown table from rocprofv3 runs over --block-probe: per matrix launch kind of the
    block, durations from a kernel trace and counters averaged per dispatch from --pmc
    passes; FETCH_SIZE / WRITE_SIZE scaled by what they read for the calibration copy."""
    import csv
    import glob
    from collections import defaultdict
    from stream_flow_matching_amd import synth
    w = synth.WORKLOADS[name]
    M = w.B * w.L
    dur = defaultdict(list)
    vals = defaultdict(lambda: defaultdict(list))
    copy = defaultdict(list)
    names = {}
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
            rows = sorted(csv.DictReader(open(f)), key=lambda r: int(r["Start_Timestamp"]))
            for r in rows:
                r["Dispatch_Id"] = r.get("Dispatch_Id") or r["Correlation_Id"]
            lab = _block_kinds(rows)
            for r in rows:
                if r["Dispatch_Id"] in lab:
                    dur[lab[r["Dispatch_Id"]]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
                    names[lab[r["Dispatch_Id"]]] = _short(r["Kernel_Name"])
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            rows = list(csv.DictReader(open(f)))
            disp = {}
            for r in rows:
                disp.setdefault(r["Dispatch_Id"], r)
            lab = _block_kinds(sorted(disp.values(), key=lambda r: int(r["Dispatch_Id"])))
            for r in rows:
                if r["Dispatch_Id"] in lab:
                    vals[lab[r["Dispatch_Id"]]][r["Counter_Name"]].append(float(r["Counter_Value"]))
                    names[lab[r["Dispatch_Id"]]] = _short(r["Kernel_Name"])
                elif "copyBuffer" in r["Kernel_Name"]:
                    copy[r["Counter_Name"]].append(float(r["Counter_Value"]))
    mean = lambda v: sum(v) / len(v)
    scale = {c: COPY_BYTES / (mean(v) * 1024) for c, v in copy.items() if c in ("FETCH_SIZE", "WRITE_SIZE") and v}
    peak = BF16_PEAK_TFLOPS if w.wfmt == "nf4" else FP8_PEAK_TFLOPS
    print(f"Workload {name}: {w.describe}; M = {M} token rows; weights {w.wfmt}.")
    print()
    print("| kind | kernel | launches | avg us | TFLOP/s | % of matrix peak | MfmaUtil (%) "
          "| LDS conflict cycles / active | FETCH + WRITE (MB, scaled) | algorithmic (MB) |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for kind in KINDS:
        if kind not in names:
            continue
        if kind == "attention":
            fl, ab = 4.0 * w.B * w.L * w.L * 4608, 8 * M * 4608
        else:
            fl, ab = block_work(kind, M, w.wfmt)
        us = mean(dur[kind]) if dur.get(kind) else None
        pk = BF16_PEAK_TFLOPS if kind == "attention" else peak
        tf = f"{fl / us / 1e6:.1f}" if us else ""
        frac = f"{100 * fl / us / 1e6 / pk:.1f}" if us else ""
        cv = vals.get(kind, {})
        util = f"{mean(cv['MfmaUtil']):.1f}" if "MfmaUtil" in cv else ""
        conf = ""
        if "SQ_LDS_BANK_CONFLICT" in cv and "SQ_LDS_IDX_ACTIVE" in cv and mean(cv["SQ_LDS_IDX_ACTIVE"]) > 0:
            conf = f"{mean(cv['SQ_LDS_BANK_CONFLICT']) / mean(cv['SQ_LDS_IDX_ACTIVE']):.3f}"
        traffic = ""
        if "FETCH_SIZE" in cv and "WRITE_SIZE" in cv and "FETCH_SIZE" in scale and "WRITE_SIZE" in scale:
            tb = (mean(cv["FETCH_SIZE"]) * scale["FETCH_SIZE"] + mean(cv["WRITE_SIZE"]) * scale["WRITE_SIZE"]) * 1024
            traffic = f"{tb / 1e6:.1f}"
        n = len(dur.get(kind, [])) or max((len(v) for v in cv.values()), default=0)
        avg = f"{us:.1f}" if us else ""
        print(f"| {kind} | `{names[kind]}` | {n} | {avg} | {tf} | {frac} | {util} | {conf} | {traffic} "
              f"| {ab / 1e6:.1f} |")
    if scale:
        print()
        print("Byte-counter scales from the copy of %d MiB: %s." % (COPY_BYTES >> 20, ", ".join(
            f"{c} x {v:.4f} KiB -> bytes" for c, v in sorted(scale.items()))))


def _short(n):
    n = n.replace("sfm::(anonymous namespace)::", "").replace("sfm::", "")
    n = n[5:] if n.startswith("void ") else n
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):      # drop the argument list, keep template arguments
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    return n[:cut]


def _step_kinds(rows):
    """Label the matrix launches of one guided step (dispatches in launch order): per
    block QKV (STORE GEMM), attention, O (gated residual), gate/up (SwiGLU), down
    (gated residual after a SwiGLU); the conditional pass first."""
    labels, last = {}, None
    for r in rows:
        n = _short(r["Kernel_Name"])
        kind = None
        if n.startswith("gemm_fp8_kernel<"):
            epi = n.split(",")[2].strip()
            kind = {"0": "qkv", "4": "qkv", "2": "gate_up", "1": "down" if last == "gate_up" else "o"}.get(epi)
        elif n.startswith("attn_kernel"):
            kind = "attention"
        if kind:
            labels[r["Dispatch_Id"]] = kind
            last = kind
    return labels


def pmc_summary(dirs):
    """Per-kernel tables from rocprofv3 --pmc passes over --pmc-probe (one directory per
    pass, each with its counter_collection.csv): counters are averaged per dispatch
    over the launches of each (kernel kind, pass) of the guided step and over the
    standalone bandwidth-bound launches.  FETCH_SIZE / WRITE_SIZE are scaled by what
    they read for the plain copy of COPY_BYTES."""
    import csv
    import glob
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))     # (group) -> counter -> values
    copy = defaultdict(list)
    grids = {}
    for d in dirs:
        f = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
        if not f:
            sys.exit(f"no counter_collection.csv under {d}")
        rows = list(csv.DictReader(open(f[0])))
        disp = {}
        for r in rows:
            disp.setdefault(r["Dispatch_Id"], r)
        order = sorted(disp.values(), key=lambda r: int(r["Dispatch_Id"]))
        labels = _step_kinds(order)
        nsteps = sum(1 for v in labels.values() if v == "qkv")
        seen = defaultdict(int)
        group_of = {}
        last_step = max((int(d) for d in labels), default=-1)
        for r in order:
            did = r["Dispatch_Id"]
            if did in labels:
                kind = labels[did]
                seen[kind] += 1
                group_of[did] = (kind, "cond" if seen[kind] <= nsteps // 2 else "uncond")
            elif "copyBuffer" in r["Kernel_Name"]:
                group_of[did] = ("copy", "")
            elif "sfm::" in r["Kernel_Name"] and int(did) > last_step:
                wg = int(r["Grid_Size"]) // max(int(r["Workgroup_Size"]), 1)
                group_of[did] = (f"{_short(r['Kernel_Name'])} [{wg} wg]", "alone")
        for r in rows:
            g = group_of.get(r["Dispatch_Id"])
            if not g:
                continue
            grids[g] = int(r["Grid_Size"]) // max(int(r["Workgroup_Size"]), 1)
            if g[0] == "copy":
                copy[r["Counter_Name"]].append(float(r["Counter_Value"]))
            else:
                vals[g][r["Counter_Name"]].append(float(r["Counter_Value"]))
    mean = lambda v: sum(v) / len(v)
    scale = {c: COPY_BYTES / (mean(v) * 1024) for c, v in copy.items() if c in ("FETCH_SIZE", "WRITE_SIZE") and v}
    counters = sorted({c for g in vals.values() for c in g})
    print("| kernel | pass | workgroups | launches | " + " | ".join(counters) + " |")
    print("|---|---|---|---|" + "---|" * len(counters))
    for g, cv in sorted(vals.items()):
        n = max(len(v) for v in cv.values())
        print(f"| `{g[0]}` | {g[1]} | {grids[g]} | {n} | " +
              " | ".join(f"{mean(cv[c]):.4g}" if c in cv else "" for c in counters) + " |")
    if scale:
        print()
        print("Byte-counter scales from the copy of %d MiB: %s." % (COPY_BYTES >> 20, ", ".join(
            f"{c} x {v:.4f} KiB -> bytes" for c, v in sorted(scale.items()))))
    # derived per kernel: matrix-core utilisation, counted matrix FLOPs against the algorithmic
    # ones, LDS bank conflicts per LDS-active cycle, and bytes against the algorithmic bytes
    print()
    print("| kernel | pass | MfmaUtil (%) | matrix FLOP counted / algorithmic | LDS conflict cycles / active "
          "| FETCH + WRITE (MB, scaled) | algorithmic (MB) | ratio |")
    print("|---|---|---|---|---|---|---|---|")
    Lof = {"cond": 4608, "uncond": 4096}
    for g, cv in sorted(vals.items()):
        util = f"{mean(cv['MfmaUtil']):.1f}" if "MfmaUtil" in cv else ""
        flop_ratio = conf = traffic = alg = ratio = ""
        if g[0] in KINDS:
            fl, ab = kernel_work(g[0], Lof[g[1]])
            mops = sum(mean(cv[c]) for c in cv if c.startswith("SQ_INSTS_VALU_MFMA_MOPS_"))
            if mops:
                flop_ratio = f"{mops * 512 / fl:.3f}"
            alg = f"{ab / 1e6:.1f}"
        if "SQ_LDS_BANK_CONFLICT" in cv and "SQ_LDS_IDX_ACTIVE" in cv and mean(cv["SQ_LDS_IDX_ACTIVE"]) > 0:
            conf = f"{mean(cv['SQ_LDS_BANK_CONFLICT']) / mean(cv['SQ_LDS_IDX_ACTIVE']):.3f}"
        if "FETCH_SIZE" in cv and "WRITE_SIZE" in cv and "FETCH_SIZE" in scale and "WRITE_SIZE" in scale:
            tb = (mean(cv["FETCH_SIZE"]) * scale["FETCH_SIZE"] + mean(cv["WRITE_SIZE"]) * scale["WRITE_SIZE"]) * 1024
            traffic = f"{tb / 1e6:.1f}"
            if g[0] in KINDS:
                ratio = f"{tb / kernel_work(g[0], Lof[g[1]])[1]:.2f}"
        if util or flop_ratio or conf or traffic:
            print(f"| `{g[0]}` | {g[1]} | {util} | {flop_ratio} | {conf} | {traffic} | {alg} | {ratio} |")
    for g, cv in sorted(vals.items()):
        if g[0] in KINDS and "FETCH_SIZE" in cv and "WRITE_SIZE" in cv and "FETCH_SIZE" in scale:
            fb = mean(cv["FETCH_SIZE"]) * 1024 * scale["FETCH_SIZE"]
            wb = mean(cv["WRITE_SIZE"]) * 1024 * scale["WRITE_SIZE"]
            rec = {"kind": g[0], "pass": g[1], "bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb),
                   "write_bytes": round(wb), "sources_sha256_16": sources_digest(g[0])}
            print("traffic-record: " + json.dumps(rec))


def trace_summary(out_dir):
    """Markdown tables from rocprofv3's kernel_trace.csv / kernel_stats.csv under
    out_dir: every launch of this library's kernels grouped by (kernel, grid in
    workgroups), and the matrix launches of the last guided step (the one bench.py
    times with events) per kind and pass."""
    import csv
    import glob
    from collections import defaultdict
    trace = sorted(glob.glob(os.path.join(out_dir, "**", "*kernel_trace.csv"), recursive=True))
    if not trace:
        sys.exit(f"no kernel_trace.csv under {out_dir}")
    groups = defaultdict(list)
    rows = sorted(csv.DictReader(open(trace[0])), key=lambda r: int(r["Start_Timestamp"]))
    rows = [r for r in rows if "sfm::" in r["Kernel_Name"]]
    for r in rows:
        wg = 1
        for ax in "XYZ":
            wg *= int(r[f"Grid_Size_{ax}"]) // max(int(r[f"Workgroup_Size_{ax}"]), 1)
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups[(_short(r["Kernel_Name"]), wg)].append(us)
    total = sum(sum(v) for v in groups.values())
    print("| kernel | workgroups | launches | avg us | share of GPU time (%) |")
    print("|---|---|---|---|---|")
    for (name, wg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{name}` | {wg} | {len(v)} | {sum(v) / len(v):.1f} | {100 * sum(v) / total:.1f} |")
    # the last step: its 2 * 34 * 5 matrix launches are the last ones of their kinds
    for r in rows:
        r["Dispatch_Id"] = r.get("Dispatch_Id") or r["Correlation_Id"]
    labels = _step_kinds(rows)
    per = defaultdict(list)
    for r in rows:
        if r["Dispatch_Id"] in labels:
            per[labels[r["Dispatch_Id"]]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print()
    print("| matrix kernel (last step) | avg us cond | avg us uncond | ms per step |")
    print("|---|---|---|---|")
    for kind in KINDS:
        v = per.get(kind, [])[-68:]
        if len(v) == 68:
            c, u = v[:34], v[34:]
            print(f"| {kind} | {sum(c) / 34:.1f} | {sum(u) / 34:.1f} | {sum(v) / 1e3:.2f} |")
    stats = sorted(glob.glob(os.path.join(out_dir, "**", "*kernel_stats.csv"), recursive=True))
    if stats:
        print()
        print("| kernel (rocprofv3 --stats) | calls | avg us | % |")
        print("|---|---|---|---|")
        for r in csv.DictReader(open(stats[0])):
            if "sfm::" in r["Name"]:
                print(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                      f"{float(r['Percentage']):.2f} |")


def yardstick(iters=20):
    """Vendor-library timings at the step's shapes on this GPU, for context: hipBLASLt's FP8
    GEMM (torch._scaled_mm, per-tensor scales, bf16 out, no fused epilogue), torch's bf16 GEMM
    and torch's scaled_dot_product_attention at one pass's attention shape."""
    import torch
    out = {}
    for name, (M, N, K) in (("gate_up", (4608, 24576, 4608)), ("o", (4608, 4608, 4608)),
                            ("down", (4608, 4608, 12288)), ("qkv", (4608, 13824, 4608)),
                            ("square_8192", (8192, 8192, 8192))):
        a = (torch.randn(M, K, device="cuda") * 0.5).to(torch.float8_e4m3fn)
        b = (torch.randn(N, K, device="cuda") * 0.5).to(torch.float8_e4m3fn).t()
        one = torch.tensor(1.0, device="cuda")
        us = time_gpu(lambda: torch._scaled_mm(a, b, scale_a=one, scale_b=one, out_dtype=torch.bfloat16), iters) * 1e6
        ab = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        bb = torch.randn(K, N, device="cuda", dtype=torch.bfloat16)
        us16 = time_gpu(lambda: ab @ bb, iters) * 1e6
        fl = 2.0 * M * N * K
        out[name] = {"shape": [M, N, K], "fp8_scaled_mm_us": round(us, 1),
                     "fp8_frac": round(fl / us / 1e6 / FP8_PEAK_TFLOPS, 4), "bf16_mm_us": round(us16, 1),
                     "bf16_frac": round(fl / us16 / 1e6 / BF16_PEAK_TFLOPS, 4)}
    for L in (4608, 4096):
        q = torch.randn(1, 18, L, 256, device="cuda", dtype=torch.bfloat16)
        k, v = torch.randn_like(q), torch.randn_like(q)
        us = time_gpu(lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v), 10) * 1e6
        fl = 4.0 * L * L * 256 * 18
        out[f"sdpa_{L}"] = {"us": round(us, 1), "bf16_frac": round(fl / us / 1e6 / BF16_PEAK_TFLOPS, 4)}
    print(json.dumps({"yardstick": out}))


def cpu_info():
    """CPU model (from /proc/cpuinfo), BLAS library and its thread count (threadpoolctl)."""
    model = "unknown"
    try:
        model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    blas, threads = "unknown", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')}"
                threads = i.get("num_threads", threads)
                break
    except Exception:
        pass
    return model, blas, threads


def cpu_baseline(sample):
    """The CPU oracle (float64 NumPy; BLAS threads on every core this process may use)
    on the block workloads.  The value is block tokens/s of one whole block of
    `sample` (the guided step's conditional shape, 4608 tokens).  Beside it: the tiny
    block whole, and 16 sampled output rows of the 2048^2 block and of the NF4 6:1
    batch (keys and values for every token of the sampled sequences, queries and MLP
    for the sampled rows only).  Weights are decoded before each timer starts; the
    decoding is timed on its own."""
    import numpy as np
    from oracle import dit as O
    from stream_flow_matching_amd import synth
    from tests._util import np64, oracle_block

    D, F = 4608, 12288

    def run(name, nrows=None):
        w = synth.WORKLOADS[name]
        dims = O.TINY if w.shape.emb_dim == 512 else O.IDEOGRAM4
        p = synth.block_params(w.shape, (0, w.name), w.wfmt)
        x, c = synth.block_inputs(w)
        t0 = time.perf_counter()
        ob = O.predecode(oracle_block(p))
        dec = time.perf_counter() - t0
        xx, cc = np64(x), c.numpy().astype(np.float64)
        rows = None
        if nrows:
            rows = np.linspace(0, w.L - 1, nrows).astype(int)     # rows of the first sequence
        t0 = time.perf_counter()
        O.block_forward(xx[:1] if rows is not None else xx, cc[:1] if rows is not None else cc, ob, w.T, w.gh, w.gw,
                        dims, rows=rows)
        sec = time.perf_counter() - t0
        d, f = w.shape.emb_dim, w.shape.intermediate
        if rows is None:
            flop = block_flops(w.L, w.B, d, f)
            toks = w.B * w.L
        else:
            flop = w.L * 2 * 2 * d * d + nrows * (2 * (2 * d * d + 3 * d * f) + 4 * w.L * d)
            toks = nrows
        r = {"workload": name, "rows": "all" if rows is None else f"{nrows} sampled rows of sequence 0",
             "s": round(sec, 2), "decode_s": round(dec, 2), "gflop_s": round(flop / sec / 1e9, 1)}
        r["tokens_per_s" if rows is None else "rows_per_s"] = round(toks / sec, 2)
        return r

    def fp32_products(name):
        """The matrix products of one whole block in float32 (torch on the CPU, its own
        threads): the QKV, output, gate/up and down projections on decoded weights and the
        attention's two products per head, without the norms, softmax, rotary or
        quantisation; a lower bound on the time of any float32 CPU block."""
        import torch
        w = synth.WORKLOADS[name]
        d, f, L, H = w.shape.emb_dim, w.shape.intermediate, w.L, w.shape.emb_dim // 256
        g = torch.Generator().manual_seed(0)
        mk = lambda *s: torch.randn(*s, generator=g)
        x, wqkv, wo, wgu, wd = mk(L, d), mk(d, 3 * d), mk(d, d), mk(d, 2 * f), mk(f, d)
        q, k, v, s_, hh = mk(H, L, 256), mk(H, 256, L), mk(H, L, 256), mk(L, f), mk(L, d)
        t0 = time.perf_counter()
        torch.mm(x, wqkv)
        for h in range(H):
            torch.mm(torch.mm(q[h], k[h]), v[h])
        torch.mm(hh, wo)
        torch.mm(x, wgu)
        torch.mm(s_, wd)
        sec = time.perf_counter() - t0
        flop = block_flops(L, 1, d, f)
        return {"workload": name, "rows": "all", "s": round(sec, 2), "gflop_s": round(flop / sec / 1e9, 1),
                "tokens_per_s": round(L / sec, 2), "threads": torch.get_num_threads(),
                "what": "float32 matrix products only (torch CPU): a lower bound for a float32 CPU block"}

    main = run(sample)
    runs = [main, run("tiny_block"), run("block_2048", 16), run("block_6to1_nf4", 16)]
    model, blas, threads = cpu_info()
    return {"value": main["tokens_per_s"], "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one whole block of {sample} ({main['s']} s, float64 oracle, weights decoded beforehand "
                      f"in {main['decode_s']} s)",
            "cpu_model": model, "blas": blas, "precision": "float64", "runs": runs,
            "fp32_products": fp32_products(sample)}


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.block_summary:
        block_summary(args.block_summary)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from stream_flow_matching_amd import sfm, synth
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.yardstick:
        yardstick()
        return
    ctx = sfm.Context("ideogram4", 0)
    if args.pmc_probe:
        pmc_probe(sfm, synth, ctx)
        return
    if args.block_probe:
        block_probe(sfm, synth, ctx, args.block_probe)
        return

    w = synth.WORKLOADS["cfg_step_1024"]
    presets = () if args.no_extra else (("V4_TURBO_12", sfm.SFM_PRESET_V4_TURBO_12),
                                         ("V4_QUALITY_48", sfm.SFM_PRESET_V4_QUALITY_48))
    sec, ok, launches, samples, streamed, clock = cfg_step_bench(sfm, synth, ctx, args.steps, args.warmup, presets)
    tokens = w.layers * (w.B * (w.T + w.gh * w.gw) + w.B * w.gh * w.gw)
    flops = w.layers * (block_flops(w.T + w.gh * w.gw, w.B) + block_flops(w.gh * w.gw, w.B))
    step_tflops = flops / sec / 1e12
    roof = roofline(kernel_table(launches, w), w)
    if clock:
        # the same fraction against the matrix peak at the clock measured under this load
        roof["peak_at_clock"] = round(roof["peak"] * clock["mhz_median"] / 2400.0, 1)
        roof["frac_at_clock"] = round(roof["achieved"] / roof["peak_at_clock"], 4)
    hbm = None if args.no_hbm else hbm_kernels(sfm, synth, ctx)
    extra = {}
    if not args.no_extra:
        for name in ("block_1024", "block_2048", "block_6to1_nf4"):
            extra[name] = block_bench(sfm, synth, ctx, name)
        extra["block_1024_mixed"] = block_bench(sfm, synth, ctx, "block_1024", fmt="mixed")
        extra["text_projection_512"] = text_project_bench(sfm, synth, ctx)
        extra["block_1024_varlen_b2"] = block_varlen_bench(sfm, synth, ctx)
        extra["attention_4608"] = attention_bench(sfm, ctx, 4608)
        extra["attention_4096"] = attention_bench(sfm, ctx, 4096)
    cpu = None if args.no_cpu else cpu_baseline(args.cpu_sample)

    line = {
        "metric": "DiT block tokens/s + TFLOP/s (% FP8 MFMA peak) at 1024^2; s per CFG step",
        "value": round(tokens / sec, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 3),
        "s_per_cfg_step": round(sec, 5),
        "step_tflops": round(step_tflops, 2),
        "step_frac_fp8_peak": round(step_tflops / FP8_PEAK_TFLOPS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 matmul (fp32 accumulate), bf16 activations and attention",
        "data": "synthetic",
        "finite": ok,
        "config": {"workload": "cfg_step_1024: " + w.describe, "batch": w.B, "text_tokens": w.T,
                   "image_grid": [w.gh, w.gw], "layers": w.layers, "weight_sets": 2, "guidance": 4.0,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "gpu_clock": clock,
        "hbm_kernels": hbm,
        "cpu_baseline": cpu,
        "blocks": extra,
        "sampler_1024": samples,
        "streamed_weights_1024": streamed,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
