"""Drives the C ABI of the host-instrumented library copy (libsfm_asan.so:
AddressSanitizer + UndefinedBehaviorSanitizer on the host code, device code
unchanged).  Run by tests/test_abi_sanitized.py in a child process that
preloads the sanitizer runtime; any heap overflow, use after free or
undefined behaviour in the host code aborts the child with a report.

  python tests/abi_sanitized_driver.py    # host-only functions and rejected calls

Prints "sanitized driver ok: <n> checks" at the end.
"""

import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from stream_flow_matching_amd import sfm  # noqa: E402

sfm.LIB_PATH = os.path.join(ROOT, "stream_flow_matching_amd", "libsfm_asan.so")
L = sfm.lib()
n_checks = 0


def expect(status, want, what):
    global n_checks
    n_checks += 1
    if status != want:
        msg = L.sfm_last_error().decode()
        raise AssertionError(f"{what}: status {status}, expected {want} ({msg})")
    if want < 0 and not L.sfm_last_error():
        raise AssertionError(f"{what}: no error message")


def host_checks():
    d = L.sfm_dims_ideogram4()
    expect(L.sfm_check_shape(ctypes.byref(d), 1, 512, 64, 64), 0, "spec shape")
    for B, T, gh, gw in [(0, 512, 64, 64), (9, 1, 64, 64), (1, -1, 64, 64), (1, 2049, 64, 64), (1, 0, 15, 64),
                         (1, 0, 129, 64), (1, 0, 16, 97)]:
        expect(L.sfm_check_shape(ctypes.byref(d), B, T, gh, gw), -2, f"shape {B} {T} {gh} {gw}")
    for field, value in [("emb_dim", 4600), ("head_dim", 128), ("rope_dims", 96), ("intermediate", 100),
                         ("adaln_dim", 4), ("latent_ch", 3), ("max_text", 5000)]:
        bad = L.sfm_dims_ideogram4()
        setattr(bad, field, value)
        expect(L.sfm_check_shape(ctypes.byref(bad), 1, 16, 16, 16), -2, f"dims {field}")
    bad = L.sfm_dims_ideogram4()
    bad.eps = 0.0
    expect(L.sfm_check_shape(ctypes.byref(bad), 1, 16, 16, 16), -1, "dims eps")
    expect(L.sfm_check_shape(None, 1, 16, 16, 16), -1, "dims NULL")
    # the positions helper writes exactly 3 L int32 values into an exactly sized host buffer
    for T, gh, gw in [(0, 1, 1), (3, 2, 2), (77, 16, 17), (2048, 128, 128)]:
        pos = np.empty((T + gh * gw, 3), np.int32)
        expect(L.sfm_positions(T, gh, gw, pos.ctypes.data_as(ctypes.c_void_p)), 0, "positions")
        assert pos[T:, 0].tolist() == [T] * (gh * gw)
    expect(L.sfm_positions(1, 1, 1, None), -1, "positions NULL")
    for s in (0, -1, -2, -3, -4, -5, -6, -7, 5):
        assert L.sfm_status_string(s)
    # time grids and presets into exactly sized host arrays
    for n in (1, 12, 48, 200):
        t = np.empty(n + 1, np.float64)
        expect(L.sfm_time_grid(n, 0.0, 1.5, 1024 * 1024, t.ctypes.data_as(ctypes.c_void_p)), 0, "time grid")
        assert t[0] == 1.0 and t[-1] == 0.0
    expect(L.sfm_time_grid(0, 0.0, 1.5, 1024, None), -1, "time grid NULL")
    info = sfm.sfm_preset_info()
    for p in (0, 1, 2):
        expect(L.sfm_preset(p, ctypes.byref(info)), 0, "preset")
        t = np.empty(info.n_steps + 1, np.float64)
        g = np.empty(info.n_steps, np.float32)
        n = L.sfm_preset_schedule(p, 1024, 1024, t.ctypes.data_as(ctypes.c_void_p), g.ctypes.data_as(ctypes.c_void_p),
                                  info.n_steps)
        expect(n, info.n_steps, "preset schedule")
        small = L.sfm_preset_schedule(p, 1024, 1024, t.ctypes.data_as(ctypes.c_void_p),
                                      g.ctypes.data_as(ctypes.c_void_p), info.n_steps - 1)
        expect(small, -1, "preset schedule capacity")
    expect(L.sfm_preset(7, ctypes.byref(info)), -1, "unknown preset")
    # every entry point that takes a context refuses a NULL one before anything else
    for name, (res, args) in sfm.SIGNATURES.items():
        if res is not sfm._I or not args or args[0] is not sfm._P or name in ("sfm_positions",):
            continue
        if name in ("sfm_quant_rows_fp8", "sfm_euler_cfg", "sfm_context_destroy"):
            continue
        vals = [None if (a is sfm._P or hasattr(a, "contents") or a.__name__.startswith("LP_")) else 0
                for a in args]
        expect(getattr(L, name)(*vals), -1, f"{name} with NULL context")
    expect(L.sfm_quant_rows_fp8(None, 1, 64, None, None, None), -1, "quant_rows NULL")
    expect(L.sfm_euler_cfg(None, None, None, None, None, 16, 4.0, 0.1, None), -1, "euler NULL")


if __name__ == "__main__":
    host_checks()
    print(f"sanitized driver ok: {n_checks} checks", flush=True)
