"""bench.py's host logic on the CPU: the algorithmic work it prices kernels against, the
traffic records' source digests, the per-kernel summaries of rocprofv3 output (small
synthetic CSV files with hand-computed expectations) and the one-GPU guard."""

import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

D, F = 4608, 12288
MiB = 1 << 20


def test_kernel_work_closed_forms():
    M = 4608
    fl, by = bench.kernel_work("gate_up", M)
    assert fl == 2.0 * M * (2 * F) * D
    # E4M3 codes + row scales in, weight codes + column scales, bf16 SwiGLU output (F columns)
    assert by == M * D + 4 * M + 2 * F * D + 4 * 2 * F + 2 * M * F
    fl, by = bench.kernel_work("o", M)
    assert fl == 2.0 * M * D * D
    # the gated residual also reads the bf16 residual
    assert by == M * D + 4 * M + D * D + 4 * D + 2 * M * D + 2 * M * D
    fl, by = bench.kernel_work("attention", 4096)
    assert fl == 4.0 * 4096 * 4096 * D and by == 4 * 4096 * D * 2


def test_block_work_nf4():
    M = 12288
    fl, by = bench.block_work("down", M, "nf4")
    assert fl == 2.0 * M * D * F
    # bf16 activation, packed nibbles, fp32 absmax per 64 weights, bf16 output + residual
    assert by == 2 * M * F + D * F // 2 + 4 * (D * F // 64) + 2 * M * D + 2 * M * D
    assert bench.block_work("qkv", 4608, "fp8") == bench.kernel_work("qkv", 4608)


def test_measured_traffic_follows_the_sources(tmp_path, monkeypatch):
    rec = {"kind": "gate_up", "pass": "cond", "bytes_per_launch": 123,
           "sources_sha256_16": bench.sources_digest("gate_up")}
    f = tmp_path / "counters.md"
    f.write_text("table\ntraffic-record: " + json.dumps(rec) + "\n")
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(f))
    assert bench.measured_traffic("gate_up") == 123
    assert bench.measured_traffic("down") is None
    rec["sources_sha256_16"] = "0" * 16      # taken on other sources: no figure
    f.write_text("traffic-record: " + json.dumps(rec) + "\n")
    assert bench.measured_traffic("gate_up") is None


def _write(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def _name(short):
    return f"void sfm::(anonymous namespace)::{short}(unsigned short const*, int)"


# one block forward's matrix launches in launch order: (kernel, duration in us)
_BLOCK = [("gemm_nf4_kernel<256, 256, 0>", 100.0), ("attn_kernel", 50.0), ("gemm_nf4_kernel<256, 256, 1>", 30.0),
          ("gemm_nf4_kernel<256, 256, 2>", 200.0), ("gemm_nf4_kernel<256, 256, 1>", 80.0)]


def _cells(out, first):
    for line in out.splitlines():
        if line.startswith(f"| {first} |"):
            return [c.strip() for c in line.strip("|").split("|")]
    raise AssertionError(f"no row {first!r} in:\n{out}")


def test_block_summary(tmp_path, capsys):
    """Two forwards (the first, the warm-up, is dropped): durations from the trace, counters
    per dispatch, byte counters scaled by the calibration copy (FETCH_SIZE reads half the
    copy's KiB, so its scale is 2)."""
    trace, t, rows = tmp_path / "trace" / "t_kernel_trace.csv", 0, []
    for rep in range(2):
        for kernel, us in _BLOCK:
            scale = 3.0 if rep == 0 else 1.0          # the warm-up's durations must not count
            rows.append({"Correlation_Id": str(len(rows) + 1), "Kernel_Name": _name(kernel),
                         "Start_Timestamp": str(t), "End_Timestamp": str(t + int(us * scale * 1000))})
            t += 10 ** 6
    _write(str(trace), ["Correlation_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    cnt, rows, did = tmp_path / "pmc" / "p_counter_collection.csv", [], 0
    for rep in range(2):
        for kernel, _ in _BLOCK:
            did += 1
            for name, val in (("FETCH_SIZE", 1000.0 * (rep + 1)), ("WRITE_SIZE", 500.0), ("MfmaUtil", 40.0 + rep)):
                rows.append({"Dispatch_Id": str(did), "Kernel_Name": _name(kernel), "Counter_Name": name,
                             "Counter_Value": str(val)})
    did += 1
    for name, val in (("FETCH_SIZE", bench.COPY_BYTES / 1024 / 2), ("WRITE_SIZE", bench.COPY_BYTES / 1024)):
        rows.append({"Dispatch_Id": str(did), "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": name,
                     "Counter_Value": str(val)})
    _write(str(cnt), ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    bench.block_summary([str(tmp_path / "trace"), str(tmp_path / "pmc")])
    out = capsys.readouterr().out
    M = 4 * (256 + 128 * 22)
    c = _cells(out, "gate_up")
    fl, ab = bench.block_work("gate_up", M, "nf4")
    assert c[1] == "`gemm_nf4_kernel<256, 256, 2>`" and c[2] == "1" and float(c[3]) == 200.0
    assert abs(float(c[4]) - fl / 200.0 / 1e6) < 0.1
    assert float(c[6]) == 41.0                                   # the second forward's MfmaUtil
    assert abs(float(c[8]) - (2000.0 * 2 + 500.0) * 1024 / 1e6) < 0.1   # scaled FETCH + WRITE, MB
    assert abs(float(c[9]) - ab / 1e6) < 0.1
    # the gated residual after attention is O, the one after gate/up is down
    assert float(_cells(out, "o")[3]) == 30.0 and float(_cells(out, "down")[3]) == 80.0
    assert float(_cells(out, "attention")[3]) == 50.0


def test_pmc_summary_traffic_records(tmp_path, capsys):
    """Both passes of one guided step's matrix launches: the records give the conditional and
    the unconditional pass's scaled bytes per launch under the current source digests."""
    kinds = [("gemm_fp8_kernel<256, 256, 4, 0>", "qkv"), ("attn_kernel", "attention"),
             ("gemm_fp8_kernel<256, 256, 1, 0>", "o"), ("gemm_fp8_kernel<256, 256, 2, 0>", "gate_up"),
             ("gemm_fp8_kernel<256, 256, 1, 0>", "down")]
    rows, did = [], 0
    for p in range(2):
        for kernel, _ in kinds:
            did += 1
            for name, val in (("FETCH_SIZE", 100.0 * (p + 1)), ("WRITE_SIZE", 10.0 * (p + 1))):
                rows.append({"Dispatch_Id": str(did), "Kernel_Name": _name(kernel), "Counter_Name": name,
                             "Counter_Value": str(val), "Grid_Size": "256", "Workgroup_Size": "256"})
    did += 1
    for name, val in (("FETCH_SIZE", bench.COPY_BYTES / 1024), ("WRITE_SIZE", bench.COPY_BYTES / 1024)):
        rows.append({"Dispatch_Id": str(did), "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": name,
                     "Counter_Value": str(val), "Grid_Size": "256", "Workgroup_Size": "256"})
    _write(str(tmp_path / "f" / "f_counter_collection.csv"),
           ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Grid_Size", "Workgroup_Size"], rows)
    bench.pmc_summary([str(tmp_path / "f")])
    recs = [json.loads(l.split("traffic-record:", 1)[1]) for l in capsys.readouterr().out.splitlines()
            if l.startswith("traffic-record:")]
    got = {(r["kind"], r["pass"]): r for r in recs}
    assert got[("gate_up", "cond")]["bytes_per_launch"] == (100 + 10) * 1024
    assert got[("down", "uncond")]["bytes_per_launch"] == (200 + 20) * 1024
    assert got[("qkv", "cond")]["sources_sha256_16"] == bench.sources_digest("qkv")
    assert got[("attention", "cond")]["sources_sha256_16"] == bench.sources_digest("attention")


def test_one_gpu_guard():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_clock_summary_keeps_the_late_readings():
    """The clock summary keeps the last fraction of the readings (the metrics table refreshes
    slowly, so the first readings of a load can still hold the idle clock) and reports their
    median, range and socket power; with no readings it reports nothing."""
    cs = bench.ClockSampler.__new__(bench.ClockSampler)
    cs.period = 0.01
    cs.samples = [(150.0, 250.0)] * 6 + [(1800.0, 1380.0), (1850.0, 1390.0), (1840.0, None), (None, 1385.0)]
    got = cs.summary("a test", keep_last=0.4)
    assert got["mhz_median"] == 1840.0 and got["mhz_min"] == 1800.0 and got["mhz_max"] == 1850.0
    assert got["socket_power_w_median"] == 1385.0 and got["samples"] == 3
    assert bench.ClockSampler.summary(cs, "all", keep_last=1.0)["mhz_min"] == 150.0
    cs.samples = []
    assert cs.summary("nothing") is None
