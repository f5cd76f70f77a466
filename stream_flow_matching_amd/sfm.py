"""Python binding of libsfm.so (ctypes): argument marshalling only.

Every function below has the name of the C entry point it calls (include/sfm.h)
and forwards device pointers of caller-owned torch tensors plus the current HIP
stream.  No computation happens here; a missing library raises immediately.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsfm.so")

SFM_W_FP8_E4M3 = 1
SFM_W_NF4_B64 = 2
SFM_W_MXFP4 = 3
SFM_EPI_STORE = 0
SFM_EPI_RESID_GATE = 1
SFM_EPI_SWIGLU = 2

STATUS = {0: "SFM_OK", -1: "SFM_E_INVALID_ARG", -2: "SFM_E_SHAPE", -3: "SFM_E_WORKSPACE",
          -4: "SFM_E_ARCH", -5: "SFM_E_ALIGN", -6: "SFM_E_DEVICE"}


class SfmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class sfm_dims(ctypes.Structure):
    _fields_ = [("emb_dim", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("adaln_dim", ctypes.c_int32), ("latent_ch", ctypes.c_int32),
                ("rope_dims", ctypes.c_int32), ("mrope_section", ctypes.c_int32 * 3), ("max_text", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("eps", ctypes.c_float)]


class sfm_qweight(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class sfm_block_weights(ctypes.Structure):
    _fields_ = [("qkv", sfm_qweight), ("o", sfm_qweight), ("gate_up", sfm_qweight), ("down", sfm_qweight),
                ("q_norm", ctypes.c_void_p), ("k_norm", ctypes.c_void_p), ("mod_w", ctypes.c_void_p),
                ("mod_b", ctypes.c_void_p)]


class sfm_preset_info(ctypes.Structure):
    _fields_ = [("n_steps", ctypes.c_int32), ("n_main", ctypes.c_int32), ("guidance_main", ctypes.c_float),
                ("guidance_polish", ctypes.c_float), ("mu", ctypes.c_double), ("std_dev", ctypes.c_double)]


SFM_PRESET_V4_QUALITY_48 = 0
SFM_PRESET_V4_DEFAULT_20 = 1
SFM_PRESET_V4_TURBO_12 = 2


class sfm_model_weights(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("blocks", ctypes.POINTER(sfm_block_weights)),
                ("x_w", ctypes.c_void_p), ("x_b", ctypes.c_void_p), ("t_w1", ctypes.c_void_p),
                ("t_b1", ctypes.c_void_p), ("t_w2", ctypes.c_void_p), ("t_b2", ctypes.c_void_p),
                ("f_mod_w", ctypes.c_void_p), ("f_mod_b", ctypes.c_void_p), ("f_w", ctypes.c_void_p),
                ("f_b", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t

# name -> (restype, argtypes), mirroring include/sfm.h
SIGNATURES = {
    "sfm_dims_ideogram4": (sfm_dims, []),
    "sfm_dims_tiny": (sfm_dims, []),
    "sfm_context_create": (_I, [ctypes.POINTER(sfm_dims), _I, ctypes.POINTER(_P)]),
    "sfm_context_destroy": (None, [_P]),
    "sfm_check_shape": (_I, [ctypes.POINTER(sfm_dims), _I, _I, _I, _I]),
    "sfm_positions": (_I, [_I, _I, _I, _P]),
    "sfm_modulation": (_I, [_P, _P, _P, _P, _P, _I, _I, _P]),
    "sfm_adaln_norm_fp8": (_I, [_P, _P, _P, _I64, _P, _P, _I, _I, _P]),
    "sfm_adaln_norm_bf16": (_I, [_P, _P, _P, _I64, _P, _I, _I, _P]),
    "sfm_quant_rows_fp8": (_I, [_P, _I, _I, _P, _P, _P]),
    "sfm_linear": (_I, [_P, _I, _P, _P, ctypes.POINTER(sfm_qweight), _P, _P, _P, _I64, _I, _I, _P]),
    "sfm_padded_len": (_I, [_I]),
    "sfm_qk_norm_rope": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "sfm_qkv_rope": (_I, [_P, _P, _P, ctypes.POINTER(sfm_qweight), _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "sfm_attention": (_I, [_P, _P, _P, _P, _P, _I, _I, _P]),
    "sfm_euler_cfg": (_I, [_P, _P, _P, _P, _P, _I64, _F, _F, _P]),
    "sfm_dequant": (_I, [_P, ctypes.POINTER(sfm_qweight), _P, _I, _P]),
    "sfm_block_workspace_bytes": (_SZ, [_P, _I, _I, _I, _I, _I]),
    "sfm_block_forward": (_I, [_P, ctypes.POINTER(sfm_block_weights), _P, _P, _P, _I, _I, _I, _I, _P, _SZ, _P]),
    "sfm_step_workspace_bytes": (_SZ, [_P, _I, _I, _I, _I]),
    "sfm_model_velocity": (_I, [_P, ctypes.POINTER(sfm_model_weights), _P, _P, _F, _P, _I, _I, _I, _I, _P, _SZ,
                                _P]),
    "sfm_cfg_step": (_I, [_P, ctypes.POINTER(sfm_model_weights), ctypes.POINTER(sfm_model_weights), _P, _P, _P, _F,
                          _F, _F, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "sfm_cfg_step_timed": (_I, [_P, ctypes.POINTER(sfm_model_weights), ctypes.POINTER(sfm_model_weights), _P, _P, _P,
                                _F, _F, _F, _I, _I, _I, _I, _P, _P, _P, _SZ, _P, ctypes.POINTER(_P),
                                ctypes.POINTER(_P), _I, ctypes.POINTER(_I)]),
    "sfm_streamed_workspace_bytes": (_SZ, [_P, _I, _I, _I, _I]),
    "sfm_model_velocity_streamed": (_I, [_P, ctypes.POINTER(sfm_model_weights), _P, _P, _F, _P, _I, _I, _I, _I, _P,
                                         _SZ, _P]),
    "sfm_qk_norm_rope_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _I, _I, _P]),
    "sfm_attention_varlen": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P, _P]),
    "sfm_block_forward_varlen": (_I, [_P, ctypes.POINTER(sfm_block_weights), _P, _P, _P, _I, _I, _P, _I, _I, _P,
                                      _SZ, _P]),
    "sfm_model_velocity_varlen": (_I, [_P, ctypes.POINTER(sfm_model_weights), _P, _P, _P, _F, _P, _I, _I, _I, _I,
                                       _P, _SZ, _P]),
    "sfm_cfg_step_varlen": (_I, [_P, ctypes.POINTER(sfm_model_weights), ctypes.POINTER(sfm_model_weights), _P, _P,
                                 _P, _P, _F, _F, _F, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "sfm_sample_varlen": (_I, [_P, ctypes.POINTER(sfm_model_weights), ctypes.POINTER(sfm_model_weights), _P, _P, _P,
                               _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _P]),
    "sfm_text_project_workspace_bytes": (_SZ, [_P, _I, _I]),
    "sfm_text_project": (_I, [_P, _P, _P, ctypes.POINTER(sfm_qweight), _P, _I, _P, _SZ, _P]),
    "sfm_text_project_noalloc": (_I, [_P, _P, _P, ctypes.POINTER(sfm_qweight), _P, _I, _P]),
    "sfm_time_grid": (_I, [_I, ctypes.c_double, ctypes.c_double, _I64, _P]),
    "sfm_preset": (_I, [_I, ctypes.POINTER(sfm_preset_info)]),
    "sfm_preset_schedule": (_I, [_I, _I, _I, _P, _P, _I]),
    "sfm_sample": (_I, [_P, ctypes.POINTER(sfm_model_weights), ctypes.POINTER(sfm_model_weights), _P, _P, _P, _P,
                        _P, _I, _I, _I, _I, _I, _P, _SZ, _P]),
    "sfm_set_sync_check": (_I, [_I]),
    "sfm_status_string": (ctypes.c_char_p, [_I]),
    "sfm_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """Load libsfm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with stream_flow_matching_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise SfmError(status, lib().sfm_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# --------------------------------------------------------------------------- context

class Context:
    """Owns an sfm_context (constant tables on one device)."""

    def __init__(self, dims="ideogram4", device=0):
        L = lib()
        self.dims = L.sfm_dims_ideogram4() if dims == "ideogram4" else (L.sfm_dims_tiny() if dims == "tiny" else dims)
        h = ctypes.c_void_p()
        _check(L.sfm_context_create(ctypes.byref(self.dims), device, ctypes.byref(h)))
        self.handle = h

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.sfm_context_destroy(self.handle)
            self.handle = None


def qweight(fmt, q, scale):
    n = q.shape[0]
    k = q.shape[1] * (2 if fmt in (SFM_W_NF4_B64, SFM_W_MXFP4) else 1)
    return sfm_qweight(fmt, n, k, q.data_ptr(), scale.data_ptr())


class BlockWeights:
    """sfm_block_weights over device tensors (keeps them alive)."""

    def __init__(self, p):
        # "mixed": qkv and o FP8, gate_up and down MXFP4 (the activations path is the FP8 one)
        fmt = SFM_W_FP8_E4M3 if p.fmt in ("fp8", "mixed") else SFM_W_NF4_B64
        ffn = SFM_W_MXFP4 if p.fmt == "mixed" else fmt
        self._keep = p
        self.c = sfm_block_weights(qweight(fmt, *p.qkv), qweight(fmt, *p.o), qweight(ffn, *p.gate_up),
                                   qweight(ffn, *p.down), p.q_norm.data_ptr(), p.k_norm.data_ptr(),
                                   p.mod_w.data_ptr(), p.mod_b.data_ptr())
        self.fmt = fmt


class ModelWeights:
    """sfm_model_weights over device tensors (keeps them alive)."""

    def __init__(self, p):
        self._keep = p
        self.blocks = [BlockWeights(b) for b in p.blocks]
        n = len(self.blocks)
        self._arr = (sfm_block_weights * max(n, 1))(*[b.c for b in self.blocks])
        self.c = sfm_model_weights(n, ctypes.cast(self._arr, ctypes.POINTER(sfm_block_weights)),
                                   p.x_w.data_ptr(), p.x_b.data_ptr(), p.t_w1.data_ptr(), p.t_b1.data_ptr(),
                                   p.t_w2.data_ptr(), p.t_b2.data_ptr(), p.f_mod_w.data_ptr(), p.f_mod_b.data_ptr(),
                                   p.f_w.data_ptr(), p.f_b.data_ptr())


# --------------------------------------------------------------------------- entry points

def sfm_check_shape(dims, B, T, gh, gw):
    return lib().sfm_check_shape(ctypes.byref(dims), B, T, gh, gw)


def sfm_positions(T, gh, gw):
    import numpy as np
    pos = np.zeros((T + gh * gw, 3), np.int32)
    _check(lib().sfm_positions(T, gh, gw, pos.ctypes.data_as(ctypes.c_void_p)))
    return pos


def sfm_padded_len(L):
    return lib().sfm_padded_len(L)


def sfm_modulation(ctx, w, bias, c, mod, stream=None):
    B, n_out = mod.shape
    _check(lib().sfm_modulation(ctx.handle, _ptr(w), _ptr(bias), _ptr(c), _ptr(mod), B, n_out, _stream(stream)))


def sfm_adaln_norm_fp8(ctx, x, scale, mod_batch_stride, hq, hs, B, L, stream=None):
    _check(lib().sfm_adaln_norm_fp8(ctx.handle, _ptr(x), _ptr(scale), mod_batch_stride, _ptr(hq), _ptr(hs), B, L,
                                    _stream(stream)))


def sfm_adaln_norm_bf16(ctx, x, scale, mod_batch_stride, h, B, L, stream=None):
    _check(lib().sfm_adaln_norm_bf16(ctx.handle, _ptr(x), _ptr(scale), mod_batch_stride, _ptr(h), B, L,
                                     _stream(stream)))


def sfm_quant_rows_fp8(a, q, s, stream=None):
    rows, cols = a.shape
    _check(lib().sfm_quant_rows_fp8(_ptr(a), rows, cols, _ptr(q), _ptr(s), _stream(stream)))


def sfm_linear(ctx, epilogue, a, a_scale, w: sfm_qweight, out, resid=None, gate=None, gate_batch_stride=0, M=None,
               L=None, stream=None):
    M = a.shape[0] if M is None else M
    L = M if L is None else L
    _check(lib().sfm_linear(ctx.handle, epilogue, _ptr(a), _ptr(a_scale), ctypes.byref(w), _ptr(out), _ptr(resid),
                            _ptr(gate), gate_batch_stride, M, L, _stream(stream)))


def sfm_qk_norm_rope(ctx, qkv, q_norm, k_norm, q, k, vt, B, T, gh, gw, stream=None):
    _check(lib().sfm_qk_norm_rope(ctx.handle, _ptr(qkv), _ptr(q_norm), _ptr(k_norm), _ptr(q), _ptr(k), _ptr(vt), B,
                                  T, gh, gw, _stream(stream)))


def sfm_qk_norm_rope_varlen(ctx, qkv, q_norm, k_norm, q, k, vt, B, T, text_lens, gh, gw, stream=None):
    keep, p = _lens(text_lens)
    _check(lib().sfm_qk_norm_rope_varlen(ctx.handle, _ptr(qkv), _ptr(q_norm), _ptr(k_norm), _ptr(q), _ptr(k),
                                         _ptr(vt), B, T, p, gh, gw, _stream(stream)))


def sfm_qkv_rope(ctx, a, a_scale, w, q_norm, k_norm, q, k, vt, B, T, gh, gw, text_lens=None, stream=None):
    """w: an sfm_qweight ([3D][D]), as made by qweight(): FP8 (a: E4M3 codes, a_scale: row
    scales) or NF4 (a: bf16, a_scale: None)."""
    keep, p = _lens(text_lens) if text_lens is not None else (None, None)
    _check(lib().sfm_qkv_rope(ctx.handle, _ptr(a), _ptr(a_scale), ctypes.byref(w), _ptr(q_norm), _ptr(k_norm), _ptr(q),
                              _ptr(k), _ptr(vt), B, T, gh, gw, p, _stream(stream)))


def sfm_attention(ctx, q, k, vt, o, B, L, stream=None):
    _check(lib().sfm_attention(ctx.handle, _ptr(q), _ptr(k), _ptr(vt), _ptr(o), B, L, _stream(stream)))


def sfm_euler_cfg(z, v_c, v_u, z_out, v_out=None, guidance=4.0, dt=1.0 / 48, stream=None):
    _check(lib().sfm_euler_cfg(_ptr(z), _ptr(v_c), _ptr(v_u), _ptr(z_out), _ptr(v_out), z.numel(), guidance, dt,
                               _stream(stream)))


def sfm_dequant(ctx, w: sfm_qweight, out, stream=None):
    out_dtype = 1 if out.dtype == torch.bfloat16 else 0
    _check(lib().sfm_dequant(ctx.handle, ctypes.byref(w), _ptr(out), out_dtype, _stream(stream)))


def sfm_block_workspace_bytes(ctx, B, T, gh, gw, wfmt=SFM_W_FP8_E4M3):
    return lib().sfm_block_workspace_bytes(ctx.handle, B, T, gh, gw, wfmt)


def sfm_block_forward(ctx, bw: BlockWeights, x_in, x_out, c, B, T, gh, gw, ws, stream=None):
    _check(lib().sfm_block_forward(ctx.handle, ctypes.byref(bw.c), _ptr(x_in), _ptr(x_out), _ptr(c), B, T, gh, gw,
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def sfm_step_workspace_bytes(ctx, B, T, gh, gw):
    return lib().sfm_step_workspace_bytes(ctx.handle, B, T, gh, gw)


def sfm_model_velocity(ctx, mw: ModelWeights, text, latent, t, v_out, B, T, gh, gw, ws, stream=None):
    _check(lib().sfm_model_velocity(ctx.handle, ctypes.byref(mw.c), _ptr(text) if T > 0 else None, _ptr(latent),
                                    float(t), _ptr(v_out), B, T, gh, gw, _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)))


def sfm_cfg_step(ctx, cond: ModelWeights, uncond: ModelWeights, text, z, z_out, t, dt, guidance, B, T, gh, gw,
                 ws, v_c_out=None, v_u_out=None, stream=None):
    _check(lib().sfm_cfg_step(ctx.handle, ctypes.byref(cond.c), ctypes.byref(uncond.c), _ptr(text) if T > 0 else None,
                              _ptr(z), _ptr(z_out), float(t), float(dt), float(guidance), B, T, gh, gw,
                              _ptr(v_c_out), _ptr(v_u_out), _ptr(ws), ws.numel() * ws.element_size(),
                              _stream(stream)))


def sfm_cfg_step_timed(ctx, cond: ModelWeights, uncond: ModelWeights, text, z, z_out, t, dt, guidance, B, T, gh, gw,
                       ws, ev_begin, ev_end, v_c_out=None, v_u_out=None, stream=None):
    """sfm_cfg_step with torch.cuda.Event pairs recorded around the five matrix
    launches of every block (QKV, attention, output, gate/up, down; the events
    must have been recorded once, so that their HIP handles exist).  Returns the
    number of pairs recorded."""
    n = min(len(ev_begin), len(ev_end))
    arr = ctypes.c_void_p * max(n, 1)
    b = arr(*[ctypes.c_void_p(e.cuda_event) for e in ev_begin[:n]])
    e = arr(*[ctypes.c_void_p(x.cuda_event) for x in ev_end[:n]])
    rec = ctypes.c_int(0)
    _check(lib().sfm_cfg_step_timed(ctx.handle, ctypes.byref(cond.c), ctypes.byref(uncond.c),
                                    _ptr(text) if T > 0 else None, _ptr(z), _ptr(z_out), float(t), float(dt),
                                    float(guidance), B, T, gh, gw, _ptr(v_c_out), _ptr(v_u_out), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream), b, e, n, ctypes.byref(rec)))
    return rec.value


def _lens(text_lens):
    import numpy as np
    a = np.ascontiguousarray(text_lens, np.int32)
    return a, a.ctypes.data_as(_P)


def sfm_model_velocity_streamed(ctx, mw: ModelWeights, text, latent, t, v_out, B, T, gh, gw, ws, stream=None):
    """Velocity with mw's block weights in (pinned) host memory, streamed per layer."""
    _check(lib().sfm_model_velocity_streamed(ctx.handle, ctypes.byref(mw.c), _ptr(text) if T > 0 else None,
                                             _ptr(latent), float(t), _ptr(v_out), B, T, gh, gw, _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream(stream)))


def sfm_attention_varlen(ctx, q, k, vt, o, B, L, T, text_lens, stream=None):
    keep, p = _lens(text_lens)
    _check(lib().sfm_attention_varlen(ctx.handle, _ptr(q), _ptr(k), _ptr(vt), _ptr(o), B, L, T, p, _stream(stream)))


def sfm_block_forward_varlen(ctx, w, x_in, x_out, c, B, T, text_lens, gh, gw, ws, stream=None):
    keep, p = _lens(text_lens)
    _check(lib().sfm_block_forward_varlen(ctx.handle, ctypes.byref(w.c), _ptr(x_in), _ptr(x_out), _ptr(c), B, T, p,
                                          gh, gw, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def sfm_cfg_step_varlen(ctx, cond, uncond, text, text_lens, z, z_out, t, dt, guidance, B, T, gh, gw, ws,
                        v_c_out=None, v_u_out=None, stream=None):
    keep, p = _lens(text_lens)
    _check(lib().sfm_cfg_step_varlen(ctx.handle, ctypes.byref(cond.c), ctypes.byref(uncond.c), _ptr(text), p,
                                     _ptr(z), _ptr(z_out), float(t), float(dt), float(guidance), B, T, gh, gw,
                                     _ptr(v_c_out), _ptr(v_u_out), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))


def sfm_sample_varlen(ctx, cond: ModelWeights, uncond: ModelWeights, text, text_lens, z, z_out, t, guidance, B, T,
                      gh, gw, ws, stream=None):
    """sfm_sample for prompts of different text lengths (text padded to T rows)."""
    import numpy as np
    keep, p = _lens(text_lens)
    t = np.ascontiguousarray(t, np.float64)
    g = np.ascontiguousarray(guidance, np.float32)
    if len(t) != len(g) + 1:
        raise ValueError("t needs one more value than guidance")
    _check(lib().sfm_sample_varlen(ctx.handle, ctypes.byref(cond.c), ctypes.byref(uncond.c), _ptr(text), p, _ptr(z),
                                   _ptr(z_out), t.ctypes.data_as(_P), g.ctypes.data_as(_P), len(g), B, T, gh, gw,
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def sfm_text_project(ctx, raw, norm_w, proj, text_out, ws=None, stream=None):
    """raw fp32 [..., k] -> text_out bf16 [..., emb_dim]; proj a qweight (FP8)."""
    M = raw.numel() // raw.shape[-1]
    if ws is None:
        ws = workspace(lib().sfm_text_project_workspace_bytes(ctx.handle, M, raw.shape[-1]), raw.device)
    _check(lib().sfm_text_project(ctx.handle, _ptr(raw), _ptr(norm_w), ctypes.byref(proj), _ptr(text_out), M,
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def sfm_text_project_noalloc(ctx, raw, norm_w, proj, text_out, stream=None):
    """sfm_text_project on the library's fixed device scratch (no workspace argument)."""
    M = raw.numel() // raw.shape[-1]
    _check(lib().sfm_text_project_noalloc(ctx.handle, _ptr(raw), _ptr(norm_w), ctypes.byref(proj), _ptr(text_out), M,
                                          _stream(stream)))


def sfm_time_grid(n_steps, mu, std_dev, num_pixels):
    """Host time grid (n_steps + 1 float64 values, 1 -> 0) as a numpy array."""
    import numpy as np
    t = np.zeros(max(int(n_steps), 0) + 1, np.float64)
    _check(lib().sfm_time_grid(int(n_steps), float(mu), float(std_dev), int(num_pixels), t.ctypes.data_as(_P)))
    return t


def sfm_preset(preset):
    info = sfm_preset_info()
    _check(lib().sfm_preset(int(preset), ctypes.byref(info)))
    return info


def sfm_preset_schedule(preset, height_px, width_px, capacity=64):
    """(t grid, guidance weights) of a preset at an image size, as numpy arrays."""
    import numpy as np
    t = np.zeros(capacity + 1, np.float64)
    g = np.zeros(capacity, np.float32)
    n = lib().sfm_preset_schedule(int(preset), int(height_px), int(width_px), t.ctypes.data_as(_P),
                                  g.ctypes.data_as(_P), int(capacity))
    _check(min(n, 0))
    return t[:n + 1].copy(), g[:n].copy()


def sfm_sample(ctx, cond: ModelWeights, uncond: ModelWeights, text, z, z_out, t, guidance, B, T, gh, gw, ws,
               stream=None):
    """len(guidance) guided Euler steps over the host grid t (len(guidance) + 1
    decreasing values)."""
    import numpy as np
    t = np.ascontiguousarray(t, np.float64)
    g = np.ascontiguousarray(guidance, np.float32)
    n = len(g)
    if len(t) != n + 1:
        raise ValueError("t needs one more value than guidance")
    _check(lib().sfm_sample(ctx.handle, ctypes.byref(cond.c), ctypes.byref(uncond.c), _ptr(text) if T > 0 else None,
                            _ptr(z), _ptr(z_out), t.ctypes.data_as(_P), g.ctypes.data_as(_P), n, B, T, gh, gw,
                            _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def workspace(nbytes, device="cuda"):
    """A caller-owned workspace tensor of at least nbytes."""
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def sfm_set_sync_check(on):
    """Debug mode: synchronise and check for errors after every launch; returns the previous setting."""
    return lib().sfm_set_sync_check(1 if on else 0)
