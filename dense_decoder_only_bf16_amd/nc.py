"""ctypes binding of libnc.so: the same entry points as include/nc.h, marshalling only.

Every step of the forward pass runs in the library's HIP kernels; this module converts
Python arguments (torch device tensors, ints, shapes) to the C types and raises NcError on a
non-zero status.  There is no fallback: if libnc.so is missing or fails to load, every
call raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnc.so")

NC_OK = 0
NC_ERR_INVALID_ARG = -1
NC_ERR_UNSUPPORTED = -2
NC_ERR_OOM = -3
NC_ERR_CAPACITY = -4
NC_ERR_STATE = -5
NC_ERR_DEVICE = -6
NC_F32 = 0
NC_BF16 = 1

_CODE_NAMES = {NC_ERR_INVALID_ARG: "NC_ERR_INVALID_ARG", NC_ERR_UNSUPPORTED: "NC_ERR_UNSUPPORTED",
               NC_ERR_OOM: "NC_ERR_OOM", NC_ERR_CAPACITY: "NC_ERR_CAPACITY",
               NC_ERR_STATE: "NC_ERR_STATE", NC_ERR_DEVICE: "NC_ERR_DEVICE"}

NC_KC_NONE = 0
NC_KC_DECODE_GEMM = 1
NC_KC_PREFILL_GEMM = 2
NC_KC_PREFILL_ATTN = 3
NC_KC_DECODE_ATTN = 4
NC_STATIC_SCRATCH_BYTES = 64 << 20

EXPORTED = ("nc_model_create", "nc_model_free", "nc_model_set_windows", "nc_model_set_extras",
            "nc_kv_create", "nc_kv_free", "nc_kv_set_lens",
            "nc_kv_get_lens", "nc_kv_export", "nc_kv_copy_rows", "nc_prefill", "nc_decode_step",
            "nc_decode_step_static",
            "nc_decode_greedy", "nc_argmax",
            "nc_sample", "nc_timing_enable", "nc_timing_read", "nc_last_error", "nc_abi_version",
            "nc_diag_mfma_rate", "nc_diag_hbm_read_rate")


class NcError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_CODE_NAMES.get(code, code)}: {msg}")
        self.code = code


class nc_config(ctypes.Structure):
    _fields_ = [("n_layer", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_head", ctypes.c_int32), ("n_kv_head", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("softcap", ctypes.c_float),
                ("norm_eps", ctypes.c_float), ("dtype", ctypes.c_int32)]


class nc_extras(ctypes.Structure):
    _fields_ = [("resid_lambda_host", ctypes.POINTER(ctypes.c_float)),
                ("x0_lambda_host", ctypes.POINTER(ctypes.c_float)),
                ("smear_gate_dev", ctypes.c_void_p), ("smear_channels", ctypes.c_int32),
                ("smear_lambda", ctypes.c_float), ("backout_layer", ctypes.c_int32),
                ("backout_lambda", ctypes.c_float),
                ("ve_dev", ctypes.POINTER(ctypes.c_void_p)),
                ("ve_gate_dev", ctypes.POINTER(ctypes.c_void_p)), ("ve_channels", ctypes.c_int32)]


class nc_timing(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64), ("ms", ctypes.c_double),
                ("bytes", ctypes.c_double), ("flops", ctypes.c_double)]


_lib = None


def lib():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              "`python -m dense_decoder_only_bf16_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32
        L.nc_model_create.argtypes = [ctypes.POINTER(nc_config), ctypes.POINTER(vp), ctypes.POINTER(vp)]
        L.nc_model_free.argtypes = [vp]
        L.nc_model_free.restype = None
        L.nc_model_set_windows.argtypes = [vp, ctypes.POINTER(i32)]
        L.nc_model_set_extras.argtypes = [vp, ctypes.POINTER(nc_extras)]
        L.nc_kv_create.argtypes = [vp, i32, i32, ctypes.POINTER(vp)]
        L.nc_kv_free.argtypes = [vp]
        L.nc_kv_free.restype = None
        L.nc_kv_set_lens.argtypes = [vp, ctypes.POINTER(i32)]
        L.nc_kv_get_lens.argtypes = [vp, ctypes.POINTER(i32)]
        L.nc_kv_export.argtypes = [vp, i32, vp, vp, vp]
        L.nc_kv_copy_rows.argtypes = [vp, ctypes.POINTER(i32), vp, ctypes.POINTER(i32), i32, vp]
        L.nc_prefill.argtypes = [vp, vp, i32, i32, vp, vp, vp]
        L.nc_decode_step.argtypes = [vp, vp, i32, vp, vp, vp]
        L.nc_decode_step_static.argtypes = [vp, vp, i32, vp, vp, vp]
        L.nc_decode_greedy.argtypes = [vp, vp, i32, vp, vp, vp, vp]
        L.nc_argmax.argtypes = [vp, i32, i32, vp, vp]
        L.nc_sample.argtypes = [vp, i32, i32, ctypes.c_float, i32, vp, vp, vp]
        L.nc_timing_enable.argtypes = [i32]
        L.nc_timing_read.argtypes = [ctypes.POINTER(nc_timing)]
        L.nc_last_error.argtypes = []
        L.nc_last_error.restype = ctypes.c_char_p
        L.nc_diag_mfma_rate.argtypes = [i32, ctypes.POINTER(ctypes.c_double)]
        L.nc_diag_hbm_read_rate.argtypes = [ctypes.POINTER(ctypes.c_double)]
        L.nc_abi_version.argtypes = []
        L.nc_abi_version.restype = i32
        for name in ("nc_model_create", "nc_model_set_windows", "nc_model_set_extras", "nc_kv_create", "nc_kv_set_lens", "nc_kv_get_lens",
                     "nc_kv_export", "nc_kv_copy_rows", "nc_prefill", "nc_decode_step", "nc_decode_greedy",
                     "nc_decode_step_static",
                     "nc_argmax",
                     "nc_sample", "nc_timing_enable", "nc_timing_read", "nc_diag_mfma_rate",
                     "nc_diag_hbm_read_rate"):
            getattr(L, name).restype = st
        _lib = L
    return _lib


def _check(code):
    if code != NC_OK:
        raise NcError(code, lib().nc_last_error().decode(errors="replace"))


def _ptr(t):
    """Device address of a torch tensor (or None / int passthrough)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _arg(t, dtype, elems, name):
    """Device address of a tensor argument, after checking what the library cannot: a
    torch tensor must be a contiguous CUDA tensor of `dtype` ("int32" or "float32") with at
    least `elems` elements (NcError NC_ERR_INVALID_ARG otherwise).  None and raw integer
    addresses pass through unchecked."""
    if t is None or isinstance(t, int):
        return t
    want = {"int32": "torch.int32", "float32": "torch.float32"}[dtype]
    if str(t.dtype) != want:
        raise NcError(NC_ERR_INVALID_ARG, f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise NcError(NC_ERR_INVALID_ARG, f"{name} must be a CUDA tensor")
    if not t.is_contiguous():
        raise NcError(NC_ERR_INVALID_ARG, f"{name} must be contiguous")
    if t.numel() < elems:
        raise NcError(NC_ERR_INVALID_ARG, f"{name} holds {t.numel()} elements, {elems} needed")
    return t.data_ptr()


def _vocab(m):
    return _MODEL_VOCAB.get(m.value if isinstance(m, ctypes.c_void_p) else m, 0)


_MODEL_VOCAB = {}  # model handle -> vocab, for the logits size checks


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(shape, max_seq=None):
    """nc_config from an object with the model-shape attributes (see inputs.Shape)."""
    return nc_config(shape.n_layer, shape.d_model, shape.n_head, shape.n_kv_head, shape.head_dim,
                     shape.d_ff, shape.vocab, max_seq or shape.max_seq, shape.rope_base,
                     shape.softcap, shape.norm_eps,
                     NC_BF16 if shape.dtype == "bf16" else NC_F32)


# ------------------------------------------------------------------ entry points ------
def nc_abi_version():
    return lib().nc_abi_version()


def nc_last_error():
    return lib().nc_last_error().decode(errors="replace")


def nc_model_create(cfg, weights):
    """cfg: nc_config; weights: 6L+2 device tensors (or raw addresses) in canonical order."""
    arr = (ctypes.c_void_p * len(weights))(*[_ptr(w) for w in weights])
    out = ctypes.c_void_p()
    _check(lib().nc_model_create(ctypes.byref(cfg), arr, ctypes.byref(out)))
    _MODEL_VOCAB[out.value] = cfg.vocab
    return out


def nc_model_free(m):
    _MODEL_VOCAB.pop(m.value if isinstance(m, ctypes.c_void_p) else m, None)
    lib().nc_model_free(m)


def nc_model_set_windows(m, windows):
    a = np.ascontiguousarray(windows, dtype=np.int32)
    _check(lib().nc_model_set_windows(m, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))


def nc_model_set_extras(m, extras, n_layer, dtype, device="cuda"):
    """extras: None (blocks off) or a dict with any of "resid_lambda", "x0_lambda" (n_layer
    floats), "smear_gate" ([Cs] array) with "smear_lambda", "backout_layer" with
    "backout_lambda", "ve" / "ve_gate" (dicts layer -> [V, n_kv*hd] / [n_kv, Cv] arrays).
    Arrays are uploaded in the model dtype for the call (the library copies them)."""
    if extras is None:
        _check(lib().nc_model_set_extras(m, None))
        return
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    keep = []

    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device=device).to(tdt)
        keep.append(t)
        return t.data_ptr()

    def host(vals):
        a = (ctypes.c_float * n_layer)(*[float(v) for v in vals])
        keep.append(a)
        return ctypes.cast(a, ctypes.POINTER(ctypes.c_float))

    ex = nc_extras()
    if "resid_lambda" in extras:
        ex.resid_lambda_host = host(extras["resid_lambda"])
    if "x0_lambda" in extras:
        ex.x0_lambda_host = host(extras["x0_lambda"])
    if extras.get("smear_gate") is not None:
        g = np.asarray(extras["smear_gate"])
        ex.smear_gate_dev = dev(g)
        ex.smear_channels = g.shape[0]
        ex.smear_lambda = float(extras.get("smear_lambda", 0.0))
    ex.backout_layer = int(extras.get("backout_layer", -1))
    ex.backout_lambda = float(extras.get("backout_lambda", 0.0))
    ve = extras.get("ve") or {}
    if ve:
        tabs = (ctypes.c_void_p * n_layer)(*[dev(ve[l]) if l in ve else None for l in range(n_layer)])
        gates = (ctypes.c_void_p * n_layer)(*[dev(extras["ve_gate"][l]) if l in ve else None
                                              for l in range(n_layer)])
        keep += [tabs, gates]
        ex.ve_dev = ctypes.cast(tabs, ctypes.POINTER(ctypes.c_void_p))
        ex.ve_gate_dev = ctypes.cast(gates, ctypes.POINTER(ctypes.c_void_p))
        ex.ve_channels = np.asarray(extras["ve_gate"][next(iter(ve))]).shape[1]
    _check(lib().nc_model_set_extras(m, ctypes.byref(ex)))
    del keep


def layer_windows(pattern, n_layer, short_window):
    """Per-layer windows for nc_model_set_windows from a pattern such as "SSSL": layer l
    takes pattern[l % len(pattern)], 'S' = short_window, 'L' = -1 (whole context)."""
    table = {"S": int(short_window), "L": -1}
    if not pattern or any(ch not in table for ch in pattern):
        raise ValueError(f"window pattern {pattern!r} must be a non-empty string of S and L")
    return [table[pattern[i % len(pattern)]] for i in range(n_layer)]


def nc_kv_create(m, batch, max_seq):
    out = ctypes.c_void_p()
    _check(lib().nc_kv_create(m, batch, max_seq, ctypes.byref(out)))
    return out


def nc_kv_free(kv):
    lib().nc_kv_free(kv)


def nc_kv_set_lens(kv, lens):
    a = np.ascontiguousarray(lens, dtype=np.int32)
    _check(lib().nc_kv_set_lens(kv, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))


def nc_kv_get_lens(kv, batch):
    a = np.zeros(batch, dtype=np.int32)
    _check(lib().nc_kv_get_lens(kv, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return a


def nc_kv_export(kv, layer, k_out, v_out, stream=None):
    _check(lib().nc_kv_export(kv, layer, _ptr(k_out), _ptr(v_out), _stream(stream)))


def nc_kv_copy_rows(dst, dst_rows, src, src_rows, stream=None):
    d = np.ascontiguousarray(dst_rows, dtype=np.int32)
    s = np.ascontiguousarray(src_rows, dtype=np.int32)
    if d.shape != s.shape or d.ndim != 1:
        raise ValueError("dst_rows and src_rows must be 1-D of the same length")
    p = ctypes.POINTER(ctypes.c_int32)
    _check(lib().nc_kv_copy_rows(dst, d.ctypes.data_as(p), src, s.ctypes.data_as(p), d.shape[0],
                                 _stream(stream)))


def nc_prefill(m, tokens, B, T, kv, logits, stream=None):
    """tokens int32 [B, T]; logits float32 [B, T, V] or None."""
    n = max(B, 0) * max(T, 0)
    _check(lib().nc_prefill(m, _arg(tokens, "int32", n, "tokens"), B, T, kv,
                            _arg(logits, "float32", n * _vocab(m), "logits"), _stream(stream)))


def nc_decode_step(m, tokens, B, kv, logits, stream=None):
    """tokens int32 [B]; logits float32 [B, V]."""
    _check(lib().nc_decode_step(m, _arg(tokens, "int32", max(B, 0), "tokens"), B, kv,
                                _arg(logits, "float32", max(B, 0) * _vocab(m), "logits"),
                                _stream(stream)))


def nc_decode_step_static(m, tokens, B, kv, logits, stream=None):
    """tokens int32 [B]; logits float32 [B, V]; the workspace in the library's static array."""
    _check(lib().nc_decode_step_static(m, _arg(tokens, "int32", max(B, 0), "tokens"), B, kv,
                                       _arg(logits, "float32", max(B, 0) * _vocab(m), "logits"),
                                       _stream(stream)))


def nc_decode_greedy(m, tokens, B, kv, logits, next_tokens, stream=None):
    """tokens int32 [B]; logits float32 [B, V]; next_tokens int32 [B] (may be tokens)."""
    _check(lib().nc_decode_greedy(m, _arg(tokens, "int32", max(B, 0), "tokens"), B, kv,
                                  _arg(logits, "float32", max(B, 0) * _vocab(m), "logits"),
                                  _arg(next_tokens, "int32", max(B, 0), "next_tokens"),
                                  _stream(stream)))


def nc_argmax(logits, B, V, out, stream=None):
    """logits float32 [B, V]; out int32 [B]."""
    n = max(B, 0)
    _check(lib().nc_argmax(_arg(logits, "float32", n * max(V, 0), "logits"), B, V,
                           _arg(out, "int32", n, "out"), _stream(stream)))


def nc_sample(logits, B, V, temperature, top_k, u, out, stream=None):
    """logits float32 [B, V]; u float32 [B] (or None for greedy); out int32 [B]."""
    n = max(B, 0)
    _check(lib().nc_sample(_arg(logits, "float32", n * max(V, 0), "logits"), B, V,
                           float(temperature), int(top_k), _arg(u, "float32", n, "u"),
                           _arg(out, "int32", n, "out"), _stream(stream)))


def nc_timing_enable(kernel_class):
    _check(lib().nc_timing_enable(kernel_class))


def nc_timing_read():
    """(launches, ms, bytes, flops) accumulated since nc_timing_enable."""
    t = nc_timing()
    _check(lib().nc_timing_read(ctypes.byref(t)))
    return t.launches, t.ms, t.bytes, t.flops


def nc_diag_mfma_rate(random_operands=True):
    v = ctypes.c_double()
    _check(lib().nc_diag_mfma_rate(1 if random_operands else 0, ctypes.byref(v)))
    return v.value


def nc_diag_hbm_read_rate():
    v = ctypes.c_double()
    _check(lib().nc_diag_hbm_read_rate(ctypes.byref(v)))
    return v.value


# ------------------------------------------------------------------ convenience -------
def upload_weights(weights_list, dtype, device="cuda"):
    """float32 numpy arrays (exact values of the storage dtype) -> device tensors."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return [torch.from_numpy(np.ascontiguousarray(w)).to(device=device).to(tdt) for w in weights_list]


class Model:
    """Owning wrapper: model handle + its KV caches."""

    def __init__(self, shape, weights_list, max_seq=None, device="cuda", windows=None, extras=None):
        self.shape = shape
        self.cfg = make_config(shape, max_seq)
        dev = upload_weights(weights_list, shape.dtype, device)
        self.handle = nc_model_create(self.cfg, dev)
        del dev
        if windows is not None:
            nc_model_set_windows(self.handle, windows)
        if extras is not None:
            nc_model_set_extras(self.handle, extras, shape.n_layer, shape.dtype, device)

    def new_kv(self, batch, max_seq):
        return KV(self, batch, max_seq)

    def close(self):
        if self.handle is not None:
            nc_model_free(self.handle)
            self.handle = None


class KV:
    def __init__(self, model, batch, max_seq):
        self.model, self.batch, self.max_seq = model, batch, max_seq
        self.handle = nc_kv_create(model.handle, batch, max_seq)

    def _shape(self, t, shape, name):
        if t is not None and tuple(t.shape) != tuple(shape):
            raise NcError(NC_ERR_INVALID_ARG, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")

    def prefill(self, tokens, logits, stream=None):
        """tokens int32 [B, T]; logits float32 [B, T, V] or None (cache only)."""
        B, T = tokens.shape
        self._shape(logits, (B, T, self.model.shape.vocab), "logits")
        nc_prefill(self.model.handle, tokens, B, T, self.handle, logits, stream)

    def decode(self, tokens, logits, stream=None):
        """tokens int32 [B]; logits float32 [B, V]."""
        self._shape(tokens, (self.batch,), "tokens")
        self._shape(logits, (self.batch, self.model.shape.vocab), "logits")
        nc_decode_step(self.model.handle, tokens, self.batch, self.handle, logits, stream)

    def decode_static(self, tokens, logits, stream=None):
        """decode with the workspace in the library's static array (allocates nothing)."""
        self._shape(tokens, (self.batch,), "tokens")
        self._shape(logits, (self.batch, self.model.shape.vocab), "logits")
        nc_decode_step_static(self.model.handle, tokens, self.batch, self.handle, logits, stream)

    def decode_greedy(self, tokens, logits, next_tokens, stream=None):
        """decode + argmax of the logits into next_tokens (may be tokens), one graph."""
        self._shape(tokens, (self.batch,), "tokens")
        self._shape(logits, (self.batch, self.model.shape.vocab), "logits")
        self._shape(next_tokens, (self.batch,), "next_tokens")
        nc_decode_greedy(self.model.handle, tokens, self.batch, self.handle, logits, next_tokens, stream)

    def set_lens(self, lens):
        nc_kv_set_lens(self.handle, lens)

    def lens(self):
        return nc_kv_get_lens(self.handle, self.batch)

    def export(self, layer, k_out, v_out, stream=None):
        nc_kv_export(self.handle, layer, k_out, v_out, stream)

    def copy_rows_from(self, src, src_rows, dst_rows, stream=None):
        """Rows dst_rows of this cache take rows src_rows of cache `src` (same model)."""
        nc_kv_copy_rows(self.handle, dst_rows, src.handle, src_rows, stream)

    def close(self):
        if self.handle is not None:
            nc_kv_free(self.handle)
            self.handle = None
