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
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the HBM traffic table and record from the FETCH_SIZE and WRITE_SIZE passes "
                         "over --pmc-probe and exit (no GPU needed)")
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


def cfg_step_bench(sfm, synth, ctx, steps, warmup, presets=()):
    """Times `steps` CFG steps between two synchronisations; the last timed step
    also records HIP events around each of its gate/up projection launches
    (sfm_cfg_step_timed), which gives that kernel's launch durations inside the
    timed region."""
    import torch
    w = synth.WORKLOADS["cfg_step_1024"]
    cond = synth.model_params(w.shape, w.layers, (0, "cond"), device="cuda")
    unc = synth.model_params(w.shape, w.layers, (0, "uncond"), device="cuda")
    text, z, t, dt = synth.step_inputs(w, device="cuda")
    cm, um = sfm.ModelWeights(cond), sfm.ModelWeights(unc)
    ws = sfm.workspace(sfm.sfm_step_workspace_bytes(ctx, w.B, w.T, w.gh, w.gw))
    zo = torch.empty_like(z)
    nev = 2 * w.layers
    evb = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
    eve = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
    for ev in evb + eve:       # creates the HIP events
        ev.record()

    def step():
        sfm.sfm_cfg_step(ctx, cm, um, text, z, zo, t, dt, 4.0, w.B, w.T, w.gh, w.gw, ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps - 1):
        step()
    rec = sfm.sfm_cfg_step_timed(ctx, cm, um, text, z, zo, t, dt, 4.0, w.B, w.T, w.gh, w.gw, ws, evb, eve)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    launches = [evb[i].elapsed_time(eve[i]) * 1e3 for i in range(rec)]   # microseconds
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
    return sec, ok, launches[:w.layers], launches[w.layers:], samples, streamed


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


ROOF_SHAPE = (4608, 4608, 12288)   # M, K, F of the dominant launch (gate/up + SwiGLU, conditional pass)
# its kernel as rocprofv3 names it: tile 256 x 256, SwiGLU epilogue (2), FP8 weights (0)
DOMINANT = "gemm_fp8_kernel<256, 256, 2, 0>"
ROOF_SOURCES = ("stream_flow_matching_amd/csrc/k_gemm_fp8.hip", "stream_flow_matching_amd/csrc/gemm_common.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_fp8_swiglu_4608x24576x4608_traffic.md")
COPY_BYTES = 256 << 20            # plain copy kernel used to calibrate the byte counters


def roof_operands(sfm, synth):
    import torch
    M, K, F = ROOF_SHAPE
    g = torch.Generator(device="cuda").manual_seed(7)
    a = torch.randint(0, 0x7E, (M, K), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
    sa = torch.full((M,), 1e-3, device="cuda")
    wq, wsc = synth.fp8_weight(2 * F, K, ("roof",), device="cuda")
    out = torch.empty(M, F, dtype=torch.bfloat16, device="cuda")
    return a, sa, wq, wsc, out


def sources_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in ROOF_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter runs
    (FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for a plain copy of
    COPY_BYTES), or None when the kernel sources changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = next(json.loads(l.split("traffic-record:", 1)[1]) for l in f if "traffic-record:" in l)
    except (OSError, StopIteration, ValueError):
        return None
    if rec.get("sources_sha256_16") != sources_digest():
        return None
    return rec.get("bytes_per_launch")


def gemm_roofline(cond_us, uncond_us):
    """Dominant kernel: the FP8 gate/up projection with the SwiGLU epilogue
    (gemm_fp8_kernel<256, 256, SWIGLU>), the largest launch of the step.
    Algorithmic work 2*M*N*K per launch at the conditional shape (M 4608,
    N 2 x 12288, K 4608); its average duration over the 34 conditional launches
    of the last timed step, from HIP events recorded on the launch stream."""
    M, K, F = ROOF_SHAPE
    us = sum(cond_us) / len(cond_us)
    flops = 2.0 * M * K * 2 * F
    achieved = flops / (us * 1e-6) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / FP8_PEAK_TFLOPS, 4), "traffic": measured_traffic(),
            "kernel": "gemm_fp8_kernel<256, 256, SWIGLU>, M 4608 N 24576 K 4608 (conditional pass)",
            "avg_launch_us": round(us, 2), "launches": len(cond_us), "flop_per_launch": flops,
            "algorithmic_bytes_per_launch": M * K + 2 * F * K + 2 * F * 4 + M * 4 + M * F * 2,
            "uncond_avg_launch_us": round(sum(uncond_us) / max(len(uncond_us), 1), 2)}


def pmc_probe(sfm, synth, ctx, iters=10):
    """Only the dominant launch and a plain device copy of COPY_BYTES, for the
    FETCH_SIZE / WRITE_SIZE counter passes (run under rocprofv3 --pmc)."""
    import torch
    M, K, F = ROOF_SHAPE
    a, sa, wq, wsc, out = roof_operands(sfm, synth)
    w = sfm.qweight(sfm.SFM_W_FP8_E4M3, wq, wsc)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(iters):
        sfm.sfm_linear(ctx, sfm.SFM_EPI_SWIGLU, a, sa, w, out, M=M, L=M)
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_probe": "done", "copy_bytes": COPY_BYTES, "sources_sha256_16": sources_digest()}))


def pmc_summary(fetch_dir, write_dir):
    """Traffic of the dominant launch from two rocprofv3 --pmc passes over
    --pmc-probe: each counter's mean per dispatch for the GEMM and for the copy of
    COPY_BYTES, the copy fixing the counter's scale (true bytes / counted KiB)."""
    import csv
    import glob
    M, K, F = ROOF_SHAPE
    grid = (M // 256) * (2 * F // 256) * 256

    def means(d, counter):
        f = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
        if not f:
            sys.exit(f"no counter_collection.csv under {d}")
        g, c = [], []
        for r in csv.DictReader(open(f[0])):
            if r["Counter_Name"] != counter:
                continue
            if DOMINANT in r["Kernel_Name"] and int(r["Grid_Size"]) == grid:
                g.append(float(r["Counter_Value"]))
            elif "copyBuffer" in r["Kernel_Name"]:
                c.append(float(r["Counter_Value"]))
        if not g or not c:
            sys.exit(f"{counter}: no GEMM or copy dispatches in {d}")
        return sum(g) / len(g), sum(c) / len(c), len(g)

    fg, fc, n = means(fetch_dir, "FETCH_SIZE")
    wg, wc, _ = means(write_dir, "WRITE_SIZE")
    fs, ws = COPY_BYTES / (fc * 1024), COPY_BYTES / (wc * 1024)
    fb, wb = fg * 1024 * fs, wg * 1024 * ws
    alg = M * K + 2 * F * K + 2 * F * 4 + M * 4 + M * F * 2
    print(f"| counter (KiB per dispatch, mean of {n}) | GEMM | copy of {COPY_BYTES // 1024} KiB | scale |")
    print("|---|---|---|---|")
    print(f"| FETCH_SIZE | {fg:.1f} | {fc:.1f} | {fs:.4f} |")
    print(f"| WRITE_SIZE | {wg:.1f} | {wc:.1f} | {ws:.4f} |")
    print()
    print(f"Scaled: fetch {fb / 1e6:.1f} MB + write {wb / 1e6:.1f} MB = **{(fb + wb) / 1e6:.1f} MB per launch**.")
    print(f"Algorithmic bytes (A codes + weights + scales + bf16 output): {alg / 1e6:.1f} MB.")
    print()
    rec = {"kernel": "gemm_fp8_kernel<256, 256, SWIGLU>", "shape": f"M {M} N {2 * F} K {K}",
           "bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
           "fetch_scale": round(fs, 4), "write_scale": round(ws, 4), "sources_sha256_16": sources_digest()}
    print("traffic-record: " + json.dumps(rec))


def trace_summary(out_dir, layers=34):
    """Markdown tables from rocprofv3's kernel_trace.csv / kernel_stats.csv under
    out_dir: every launch of this library's kernels grouped by (kernel, grid in
    workgroups), and the dominant launch (SwiGLU gate/up at the conditional grid)
    averaged over its last `layers` launches, which are those of the last step
    (the one bench times with events when run as bench.py --steps K)."""
    import csv
    import glob
    from collections import defaultdict

    def short(n):
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

    trace = sorted(glob.glob(os.path.join(out_dir, "**", "*kernel_trace.csv"), recursive=True))
    if not trace:
        sys.exit(f"no kernel_trace.csv under {out_dir}")
    groups = defaultdict(list)
    dominant = []
    rows = sorted(csv.DictReader(open(trace[0])), key=lambda r: int(r["Start_Timestamp"]))
    for r in rows:
        if "sfm::" not in r["Kernel_Name"]:
            continue
        wg = 1
        for ax in "XYZ":
            wg *= int(r[f"Grid_Size_{ax}"]) // max(int(r[f"Workgroup_Size_{ax}"]), 1)
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        name = short(r["Kernel_Name"])
        groups[(name, wg)].append(us)
        M, _, F = ROOF_SHAPE
        if name == DOMINANT and wg == (M // 256) * (2 * F // 256):
            dominant.append(us)
    total = sum(sum(v) for v in groups.values())
    print("| kernel | workgroups | launches | avg us | share of GPU time (%) |")
    print("|---|---|---|---|---|")
    for (name, wg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{name}` | {wg} | {len(v)} | {sum(v) / len(v):.1f} | {100 * sum(v) / total:.1f} |")
    if dominant:
        last = dominant[-layers:]
        print()
        print(f"Dominant launch `{DOMINANT}` at {(ROOF_SHAPE[0] // 256) * (2 * ROOF_SHAPE[2] // 256)} "
              f"workgroups: {len(dominant)} launches, average {sum(dominant) / len(dominant):.2f} us; "
              f"last {len(last)} (the last step): average {sum(last) / len(last):.2f} us.")
    stats = sorted(glob.glob(os.path.join(out_dir, "**", "*kernel_stats.csv"), recursive=True))
    if stats:
        print()
        print("| kernel (rocprofv3 --stats) | calls | avg us | % |")
        print("|---|---|---|---|")
        for r in csv.DictReader(open(stats[0])):
            if "sfm::" in r["Name"]:
                print(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                      f"{float(r['Percentage']):.2f} |")


def cpu_baseline(sample):
    """The CPU oracle (float64 NumPy) on one full-width block of the step's
    conditional shape: 4608 tokens through one block.  Scaled to block tokens/s."""
    import numpy as np
    import torch
    from oracle import dit as O
    from stream_flow_matching_amd import synth
    from tests._util import np64, oracle_block
    w = synth.WORKLOADS[sample]
    p = synth.block_params(w.shape, (0, w.name), w.wfmt)
    x, c = synth.block_inputs(w)
    ob = oracle_block(p)
    xx, cc = np64(x), c.numpy().astype(np.float64)
    t0 = time.perf_counter()
    O.block_forward(xx, cc, ob, w.T, w.gh, w.gw, O.IDEOGRAM4)
    sec = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 0) for i in threadpool_info()), default=cores) or cores
    except Exception:
        pass
    return {"value": round(w.B * w.L / sec, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"one block of {w.describe}, float64 oracle, {sec:.1f} s"}


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
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
    ctx = sfm.Context("ideogram4", 0)
    if args.pmc_probe:
        pmc_probe(sfm, synth, ctx)
        return

    w = synth.WORKLOADS["cfg_step_1024"]
    presets = () if args.no_extra else (("V4_TURBO_12", sfm.SFM_PRESET_V4_TURBO_12),
                                         ("V4_QUALITY_48", sfm.SFM_PRESET_V4_QUALITY_48))
    sec, ok, gu_cond, gu_uncond, samples, streamed = cfg_step_bench(sfm, synth, ctx, args.steps, args.warmup, presets)
    tokens = w.layers * (w.B * (w.T + w.gh * w.gw) + w.B * w.gh * w.gw)
    flops = w.layers * (block_flops(w.T + w.gh * w.gw, w.B) + block_flops(w.gh * w.gw, w.B))
    step_tflops = flops / sec / 1e12
    roof = gemm_roofline(gu_cond, gu_uncond)
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
        "cpu_baseline": cpu,
        "blocks": extra,
        "sampler_1024": samples,
        "streamed_weights_1024": streamed,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
