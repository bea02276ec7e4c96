"""ctypes binding of libpi_ae.so (argument marshalling only).

Every step of the denoise loop runs in the library's HIP kernels; this module
only turns Python objects (NumPy host arrays for the weights, torch device
tensors for the call buffers) into the C-ABI's plain pointers and sizes.  If
the library is missing the import fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; PI_AE_LIB names another build of the same library (the
# host-sanitized one the CPU tests load)
LIB_PATH = os.environ.get("PI_AE_LIB") or os.path.join(HERE, "libpi_ae.so")

PI_AE_OK, PI_AE_EINVAL, PI_AE_EUNSUPPORTED, PI_AE_ENOMEM, PI_AE_EHIP, PI_AE_ESTATE = range(6)

# symbols declared in include/pi_ae.h
EXPORTS = ("pi_ae_prepare_weights", "pi_ae_sample", "pi_ae_sample_noalloc", "pi_ae_destroy", "pi_ae_status_string",
           "pi_ae_last_error", "pi_ae_debug_table", "pi_ae_debug_host_table", "pi_ae_debug_probe",
           "pi_ae_debug_time_phase", "pi_ae_vlm_prepare", "pi_ae_vlm_prefill", "pi_ae_vlm_destroy",
           "pi_ae_vlm_debug_time_phase", "pi_ae_pipeline_create", "pi_ae_pipeline_run", "pi_ae_pipeline_destroy",
           "pi_ae_vision_prepare", "pi_ae_vision_encode", "pi_ae_vision_destroy", "pi_ae_vision_debug_time_phase",
           "pi_ae_inference_create", "pi_ae_inference_run", "pi_ae_inference_destroy",
           "pi_ae_debug_stream_read", "pi_ae_debug_graph_floor", "pi_ae_debug_grid_sync",
           "pi_ae_debug_check_guards", "pi_ae_debug_live_device_bytes")


class PiAeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pi_ae status {status}: {message}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("width", ctypes.c_int32), ("mlp_dim", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("action_dim", ctypes.c_int32), ("chunk_len", ctypes.c_int32), ("num_steps", ctypes.c_int32),
                ("t0", ctypes.c_float), ("dt", ctypes.c_float), ("max_batch", ctypes.c_int32),
                ("max_prefix_len", ctypes.c_int32), ("rope_base", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("final_norm", ctypes.c_int32), ("variant", ctypes.c_int32)]


class Linear(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("b", ctypes.c_void_p)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, Linear) for n in ("attn_mod", "q", "k", "v", "o", "ffn_mod", "gate", "up", "down")] + \
               [("attn_norm", ctypes.c_void_p), ("ffn_norm", ctypes.c_void_p)]


class Weights(ctypes.Structure):
    _fields_ = [("action_in", Linear), ("time_in", Linear), ("time_out", Linear), ("final_mod", Linear),
                ("action_out", Linear), ("layers", ctypes.POINTER(LayerWeights)),
                ("action_time_in", Linear), ("action_time_out", Linear), ("final_norm", ctypes.c_void_p)]


class PrefixKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pad_mask", ctypes.c_void_p),
                ("prefix_len", ctypes.c_int32)]


class VlmConfig(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("width", ctypes.c_int32), ("mlp_dim", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_batch", ctypes.c_int32), ("max_prefix_len", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("rms_eps", ctypes.c_float)]


VLM_LAYER_FIELDS = ("attn_norm", "q", "k", "v", "o", "ffn_norm", "gate", "up", "down")


class VlmLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in VLM_LAYER_FIELDS]


class VisionConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("num_layers", "width", "mlp_dim", "num_heads", "head_dim", "patch",
                                              "image", "out_width", "max_views")] + [("ln_eps", ctypes.c_float)]


VISION_LAYER_FIELDS = ("ln1_w", "ln1_b", "q_w", "q_b", "k_w", "k_b", "v_w", "v_b", "o_w", "o_b",
                       "ln2_w", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")


class VisionLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in VISION_LAYER_FIELDS]


class VisionWeights(ctypes.Structure):
    _fields_ = [("patch_w", ctypes.c_void_p), ("patch_b", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("layers", ctypes.POINTER(VisionLayerWeights)), ("post_ln_w", ctypes.c_void_p),
                ("post_ln_b", ctypes.c_void_p), ("proj_w", ctypes.c_void_p), ("proj_b", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libpi_ae.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m flow_matching_action_amd.build`")
    lib = ctypes.CDLL(path)
    lib.pi_ae_prepare_weights.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), ctypes.POINTER(ctypes.c_void_p)]
    lib.pi_ae_prepare_weights.restype = ctypes.c_int
    lib.pi_ae_sample.argtypes = [ctypes.c_void_p, ctypes.POINTER(PrefixKV), ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_int32, ctypes.c_void_p]
    lib.pi_ae_sample.restype = ctypes.c_int
    lib.pi_ae_sample_noalloc.argtypes = [ctypes.c_void_p, ctypes.POINTER(PrefixKV), ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    lib.pi_ae_sample_noalloc.restype = ctypes.c_int
    lib.pi_ae_destroy.argtypes = [ctypes.c_void_p]
    lib.pi_ae_destroy.restype = None
    lib.pi_ae_status_string.argtypes = [ctypes.c_int]
    lib.pi_ae_status_string.restype = ctypes.c_char_p
    lib.pi_ae_last_error.argtypes = []
    lib.pi_ae_last_error.restype = ctypes.c_char_p
    lib.pi_ae_debug_table.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t]
    lib.pi_ae_debug_table.restype = ctypes.c_int
    lib.pi_ae_debug_host_table.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_size_t]
    lib.pi_ae_debug_host_table.restype = ctypes.c_int
    lib.pi_ae_debug_probe.argtypes = [ctypes.c_void_p, ctypes.POINTER(PrefixKV), ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_size_t]
    lib.pi_ae_debug_probe.restype = ctypes.c_int
    lib.pi_ae_debug_time_phase.argtypes = [ctypes.c_void_p, ctypes.POINTER(PrefixKV), ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.POINTER(ctypes.c_float)]
    lib.pi_ae_debug_time_phase.restype = ctypes.c_int
    lib.pi_ae_vlm_prepare.argtypes = [ctypes.POINTER(VlmConfig), ctypes.POINTER(VlmLayerWeights),
                                      ctypes.POINTER(ctypes.c_void_p)]
    lib.pi_ae_vlm_prepare.restype = ctypes.c_int
    lib.pi_ae_vlm_prefill.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.POINTER(PrefixKV), ctypes.c_void_p]
    lib.pi_ae_vlm_prefill.restype = ctypes.c_int
    lib.pi_ae_vlm_destroy.argtypes = [ctypes.c_void_p]
    lib.pi_ae_vlm_destroy.restype = None
    lib.pi_ae_vlm_debug_time_phase.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                               ctypes.POINTER(ctypes.c_float)]
    lib.pi_ae_vlm_debug_time_phase.restype = ctypes.c_int
    lib.pi_ae_pipeline_create.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
    lib.pi_ae_pipeline_create.restype = ctypes.c_int
    lib.pi_ae_pipeline_run.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.pi_ae_pipeline_run.restype = ctypes.c_int
    lib.pi_ae_pipeline_destroy.argtypes = [ctypes.c_void_p]
    lib.pi_ae_pipeline_destroy.restype = None
    lib.pi_ae_vision_prepare.argtypes = [ctypes.POINTER(VisionConfig), ctypes.POINTER(VisionWeights),
                                         ctypes.POINTER(ctypes.c_void_p)]
    lib.pi_ae_vision_prepare.restype = ctypes.c_int
    lib.pi_ae_vision_encode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.pi_ae_vision_encode.restype = ctypes.c_int
    lib.pi_ae_vision_destroy.argtypes = [ctypes.c_void_p]
    lib.pi_ae_vision_destroy.restype = None
    lib.pi_ae_vision_debug_time_phase.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                                  ctypes.POINTER(ctypes.c_float)]
    lib.pi_ae_vision_debug_time_phase.restype = ctypes.c_int
    lib.pi_ae_inference_create.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.POINTER(ctypes.c_void_p)]
    lib.pi_ae_inference_create.restype = ctypes.c_int
    lib.pi_ae_inference_run.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.pi_ae_inference_run.restype = ctypes.c_int
    lib.pi_ae_inference_destroy.argtypes = [ctypes.c_void_p]
    lib.pi_ae_inference_destroy.restype = None
    lib.pi_ae_debug_stream_read.argtypes = [ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.POINTER(ctypes.c_float)]
    lib.pi_ae_debug_stream_read.restype = ctypes.c_int
    lib.pi_ae_debug_graph_floor.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.POINTER(ctypes.c_float)]
    lib.pi_ae_debug_graph_floor.restype = ctypes.c_int
    lib.pi_ae_debug_grid_sync.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.POINTER(ctypes.c_float)]
    lib.pi_ae_debug_grid_sync.restype = ctypes.c_int
    lib.pi_ae_debug_check_guards.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.POINTER(ctypes.c_int32)]
    lib.pi_ae_debug_check_guards.restype = ctypes.c_int
    lib.pi_ae_debug_live_device_bytes.argtypes = []
    lib.pi_ae_debug_live_device_bytes.restype = ctypes.c_int64
    _lib = lib
    return lib


def _check(status: int):
    if status != PI_AE_OK:
        lib = load_library()
        raise PiAeError(status, lib.pi_ae_last_error().decode())


def make_config(cfg, max_batch: int, max_prefix_len: int) -> Config:
    """pi_ae_config from an :class:`inputs.ExpertConfig`-like object."""
    return Config(cfg.num_layers, cfg.width, cfg.mlp_dim, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim,
                  cfg.action_dim, cfg.chunk_len, cfg.num_steps, cfg.t0, cfg.dt, max_batch, max_prefix_len,
                  cfg.rope_base, cfg.rms_eps, 1 if cfg.final_norm else 0, int(getattr(cfg, "variant", 0)))


def _ptr(a):
    """Host pointer of a NumPy array, device pointer of a torch tensor, NULL for None."""
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("host arrays must be C-contiguous")
        return a.ctypes.data
    if hasattr(a, "data_ptr"):
        if not a.is_contiguous():
            raise ValueError("device tensors must be contiguous")
        return a.data_ptr()
    return int(a)


_DTYPES = {"bf16": ("torch.int16", "torch.uint16", "torch.bfloat16"), "f32": ("torch.float32",),
           "u8": ("torch.uint8", "torch.int8", "torch.bool")}


def _dev(t, name: str, kind: str, numel: int):
    """Device pointer of a call buffer, after the checks the C ABI cannot make:
    a contiguous torch tensor on the GPU, of the element type the call reads
    (bf16 bits as int16 / bfloat16, fp32, or a byte mask), holding at least
    ``numel`` elements.  None passes as NULL (the ABI rejects it where a buffer
    is required)."""
    if t is None:
        return None
    if not hasattr(t, "data_ptr") or not hasattr(t, "is_cuda"):
        raise TypeError(f"{name} must be a torch tensor on the GPU")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if str(t.dtype) not in _DTYPES[kind]:
        raise TypeError(f"{name} has dtype {t.dtype}; expected one of {_DTYPES[kind]}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements; the call reads {numel}")
    return t.data_ptr()


def _stream_handle(stream):
    if stream is None:
        return None
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


class _MarshalledWeights:
    """pi_ae_weights pointing into host arrays that this object keeps alive."""

    def __init__(self, cfg, weights: dict):
        self.keep = {n: np.ascontiguousarray(a, dtype=np.uint16) for n, a in weights.items()}

        def lin(name, bias=True):
            return Linear(_ptr(self.keep.get(name + ".w")), _ptr(self.keep.get(name + ".b")) if bias else None)

        self.layers = (LayerWeights * max(cfg.num_layers, 1))()
        for l in range(cfg.num_layers):
            p = f"layers.{l}."
            self.layers[l] = LayerWeights(lin(p + "attn_mod"), lin(p + "q", False), lin(p + "k", False),
                                          lin(p + "v", False), lin(p + "o", False), lin(p + "ffn_mod"),
                                          lin(p + "gate", False), lin(p + "up", False), lin(p + "down", False),
                                          _ptr(self.keep.get(p + "attn_norm.w")), _ptr(self.keep.get(p + "ffn_norm.w")))
        self.w = Weights(lin("action_in"), lin("time_in"), lin("time_out"), lin("final_mod"), lin("action_out"),
                         ctypes.cast(self.layers, ctypes.POINTER(LayerWeights)),
                         lin("action_time_in"), lin("action_time_out"), _ptr(self.keep.get("final_norm.w")))


def host_table(cfg, weights: dict, which: int, n: int, max_batch: int = 1, max_prefix_len: int = 0) -> np.ndarray:
    """pi_ae_debug_host_table: the preparation's fp64 tables, computed on the host only."""
    lib = load_library()
    c = make_config(cfg, max_batch, max_prefix_len)
    mw = _MarshalledWeights(cfg, weights)
    out = np.empty(n, np.float32)
    _check(lib.pi_ae_debug_host_table(ctypes.byref(c), ctypes.byref(mw.w), int(which), out.ctypes.data, out.size))
    return out


class Context:
    """A prepared expert (owns the library context)."""

    def __init__(self, cfg, weights: dict, max_batch: int, max_prefix_len: int):
        lib = load_library()
        self.cfg = cfg
        self._c = make_config(cfg, max_batch, max_prefix_len)
        mw = _MarshalledWeights(cfg, weights)
        handle = ctypes.c_void_p()
        _check(lib.pi_ae_prepare_weights(ctypes.byref(self._c), ctypes.byref(mw.w), ctypes.byref(handle)))
        self._h = handle
        self._lib = lib

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            self._lib.pi_ae_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _kv(self, k, v, pad_mask, batch, prefix_len):
        b, p = max(int(batch), 0), max(int(prefix_len), 0)
        n = self.cfg.num_layers * b * p * self.cfg.head_dim
        return PrefixKV(_dev(k, "k", "bf16", n), _dev(v, "v", "bf16", n), _dev(pad_mask, "pad_mask", "u8", b * p),
                        int(prefix_len))

    def _xbuf(self, t, name, batch):
        return _dev(t, name, "f32", max(int(batch), 0) * self.cfg.chunk_len * self.cfg.action_dim)

    def sample(self, k, v, pad_mask, noise, actions, batch: int, prefix_len: int, stream=None):
        """Enqueue pi_ae_sample on `stream` (torch tensors on the device)."""
        kv = self._kv(k, v, pad_mask, batch, prefix_len)
        _check(self._lib.pi_ae_sample(self._h, ctypes.byref(kv), self._xbuf(noise, "noise", batch),
                                      self._xbuf(actions, "actions", batch), int(batch), _stream_handle(stream)))

    def sample_noalloc(self, k, v, pad_mask, noise, actions, batch: int, prefix_len: int, stream=None):
        """Enqueue pi_ae_sample_noalloc (the library's fixed working memory, no graph)."""
        kv = self._kv(k, v, pad_mask, batch, prefix_len)
        _check(self._lib.pi_ae_sample_noalloc(self._h, ctypes.byref(kv), self._xbuf(noise, "noise", batch),
                                              self._xbuf(actions, "actions", batch), int(batch),
                                              _stream_handle(stream)))

    def time_phase(self, k, v, pad_mask, noise, actions, batch, prefix_len, phase, chunks, stream=None) -> float:
        """Mean duration (us) of one phase's kernel inside the loop: `chunks` whole
        passes on `stream`, a HIP event pair bound to each launch of that kernel."""
        kv = self._kv(k, v, pad_mask, batch, prefix_len)
        us = ctypes.c_float()
        _check(self._lib.pi_ae_debug_time_phase(self._h, ctypes.byref(kv), self._xbuf(noise, "noise", batch),
                                                self._xbuf(actions, "actions", batch), int(batch), int(phase),
                                                int(chunks), _stream_handle(stream), ctypes.byref(us)))
        return float(us.value)

    def table(self, which: int, n: int) -> np.ndarray:
        out = np.empty(n, np.float32)
        _check(self._lib.pi_ae_debug_table(self._h, int(which), out.ctypes.data, out.size))
        return out

    def probe(self, k, v, pad_mask, noise, batch, prefix_len, step, layer, phase, which):
        T = self.cfg.chunk_len
        M = batch * T
        shapes = {0: ((M, 1024), np.float32), 1: ((M, 8, 256), np.uint16), 2: ((M, 256), np.uint16),
                  3: ((M, 256), np.uint16), 4: ((M, 2048), np.uint16), 5: ((M, 4096), np.uint16),
                  6: ((M, 32), np.float32), 7: ((M, 2048), np.uint16), 8: ((M, 8, 4), np.float32)}
        shape, dt = shapes[which]
        out = np.empty(shape, dt)
        kv = self._kv(k, v, pad_mask, batch, prefix_len)
        _check(self._lib.pi_ae_debug_probe(self._h, ctypes.byref(kv), self._xbuf(noise, "noise", batch), int(batch),
                                           int(step), int(layer),
                                           int(phase), int(which), out.ctypes.data, out.nbytes))
        return out


def make_vlm_config(cfg, max_batch: int, max_prefix_len: int) -> VlmConfig:
    """pi_ae_vlm_config from an :class:`inputs.PrefillConfig`-like object."""
    return VlmConfig(cfg.num_layers, cfg.width, cfg.mlp_dim, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim,
                     max_batch, max_prefix_len, cfg.rope_base, cfg.rms_eps)


class _MarshalledVlmWeights:
    """pi_ae_vlm_layer_weights[] pointing into host arrays kept alive by this object."""

    def __init__(self, cfg, weights: dict):
        self.keep = {n: np.ascontiguousarray(a, dtype=np.uint16) for n, a in weights.items()}
        self.layers = (VlmLayerWeights * max(cfg.num_layers, 1))()
        for l in range(cfg.num_layers):
            self.layers[l] = VlmLayerWeights(*[_ptr(self.keep.get(f"layers.{l}.{n}.w")) for n in VLM_LAYER_FIELDS])


class Prefill:
    """A prepared VLM prefill (owns the library context and its prefix cache)."""

    def __init__(self, cfg, weights: dict, max_batch: int, max_prefix_len: int):
        lib = load_library()
        self.cfg = cfg
        self._c = make_vlm_config(cfg, max_batch, max_prefix_len)
        mw = _MarshalledVlmWeights(cfg, weights)
        handle = ctypes.c_void_p()
        _check(lib.pi_ae_vlm_prepare(ctypes.byref(self._c), mw.layers, ctypes.byref(handle)))
        self._h = handle
        self._lib = lib

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            self._lib.pi_ae_vlm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def run(self, emb, pad_mask, batch: int, prefix_len: int, stream=None) -> PrefixKV:
        """Enqueue pi_ae_vlm_prefill; returns the pi_ae_prefix_kv of the cache it fills."""
        kv = PrefixKV()
        _check(self._lib.pi_ae_vlm_prefill(self._h, *self._in(emb, pad_mask, batch, prefix_len), int(batch),
                                           int(prefix_len), ctypes.byref(kv), _stream_handle(stream)))
        return kv

    def _in(self, emb, pad_mask, batch, prefix_len):
        n = max(int(batch), 0) * max(int(prefix_len), 0)
        return _dev(emb, "prefix_emb", "bf16", n * self.cfg.width), _dev(pad_mask, "pad_mask", "u8", n)

    def time_phase(self, emb, pad_mask, batch, prefix_len, phase, reps, stream=None) -> float:
        us = ctypes.c_float()
        _check(self._lib.pi_ae_vlm_debug_time_phase(self._h, *self._in(emb, pad_mask, batch, prefix_len), int(batch),
                                                    int(prefix_len), int(phase), int(reps), _stream_handle(stream),
                                                    ctypes.byref(us)))
        return float(us.value)


def sample_from_cache(ctx: "Context", kv: PrefixKV, noise, actions, batch: int, stream=None):
    """pi_ae_sample on the prefix cache a Prefill has just filled."""
    _check(ctx._lib.pi_ae_sample(ctx._h, ctypes.byref(kv), ctx._xbuf(noise, "noise", batch),
                                 ctx._xbuf(actions, "actions", batch), int(batch), _stream_handle(stream)))


class Pipeline:
    """pi_ae_pipeline: a Prefill and an expert Context run as one graph per call."""

    def __init__(self, prefill: Prefill, ctx: "Context"):
        self._lib = load_library()
        self.prefill, self.ctx = prefill, ctx  # keeps both alive
        handle = ctypes.c_void_p()
        _check(self._lib.pi_ae_pipeline_create(prefill._h, ctx._h, ctypes.byref(handle)))
        self._h = handle

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            self._lib.pi_ae_pipeline_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def run(self, emb, pad_mask, noise, actions, batch: int, prefix_len: int, stream=None):
        e, m = self.prefill._in(emb, pad_mask, batch, prefix_len)
        _check(self._lib.pi_ae_pipeline_run(self._h, e, m, self.ctx._xbuf(noise, "noise", batch),
                                            self.ctx._xbuf(actions, "actions", batch), int(batch), int(prefix_len),
                                            _stream_handle(stream)))


def make_vision_config(cfg, max_views: int) -> VisionConfig:
    """pi_ae_vision_config from an :class:`inputs.VisionConfig`-like object."""
    return VisionConfig(cfg.num_layers, cfg.width, cfg.mlp_dim, cfg.num_heads, cfg.head_dim, cfg.patch, cfg.image,
                        cfg.out_width, max_views, cfg.ln_eps)


class _MarshalledVisionWeights:
    """pi_ae_vision_weights pointing into host arrays kept alive by this object."""

    def __init__(self, cfg, weights: dict):
        self.keep = {n: np.ascontiguousarray(a, dtype=np.uint16) for n, a in weights.items()}
        g = lambda n: _ptr(self.keep.get(n))
        self.layers = (VisionLayerWeights * max(cfg.num_layers, 1))()
        for l in range(cfg.num_layers):
            self.layers[l] = VisionLayerWeights(
                *[g(f"layers.{l}.{f.rsplit('_', 1)[0]}.{f.rsplit('_', 1)[1]}") for f in VISION_LAYER_FIELDS])
        self.w = VisionWeights(g("patch.w"), g("patch.b"), g("pos"), ctypes.cast(self.layers, ctypes.POINTER(VisionLayerWeights)),
                               g("post_ln.w"), g("post_ln.b"), g("proj.w"), g("proj.b"))


class Vision:
    """A prepared vision encoder (owns the library context)."""

    def __init__(self, cfg, weights: dict, max_views: int):
        lib = load_library()
        self.cfg = cfg
        self._c = make_vision_config(cfg, max_views)
        mw = _MarshalledVisionWeights(cfg, weights)
        handle = ctypes.c_void_p()
        _check(lib.pi_ae_vision_prepare(ctypes.byref(self._c), ctypes.byref(mw.w), ctypes.byref(handle)))
        self._h = handle
        self._lib = lib

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            self._lib.pi_ae_vision_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def encode(self, images, views: int, tokens, stream=None):
        """Enqueue pi_ae_vision_encode: images [views][224][224][3] bf16 -> tokens [views*256][2048] bf16."""
        im, tk = self._io(images, views, tokens)
        _check(self._lib.pi_ae_vision_encode(self._h, im, int(views), tk, _stream_handle(stream)))

    def _io(self, images, views, tokens):
        v = max(int(views), 0)
        c = self.cfg
        return (_dev(images, "images", "bf16", v * c.image * c.image * 3),
                _dev(tokens, "tokens", "bf16", v * (c.image // c.patch) ** 2 * c.out_width))

    def time_phase(self, images, views, tokens, phase, reps, stream=None) -> float:
        us = ctypes.c_float()
        im, tk = self._io(images, views, tokens)
        _check(self._lib.pi_ae_vision_debug_time_phase(self._h, im, int(views), tk, int(phase),
                                                       int(reps), _stream_handle(stream), ctypes.byref(us)))
        return float(us.value)


def check_guards(obj, corrupt: int = -1) -> int:
    """pi_ae_debug_check_guards on a Context / Prefill / Vision: -1 if every
    guard is intact, else raises PiAeError (ESTATE) naming the first changed one."""
    lib = load_library()
    kind = {"Context": 0, "Prefill": 1, "Vision": 2}[type(obj).__name__]
    bad = ctypes.c_int32(-1)
    _check(lib.pi_ae_debug_check_guards(obj._h, kind, int(corrupt), ctypes.byref(bad)))
    return bad.value


def live_device_bytes() -> int:
    """pi_ae_debug_live_device_bytes: device bytes held by the process's prepared objects."""
    return int(load_library().pi_ae_debug_live_device_bytes())


def stream_read_gbps(nbytes: int = 2 << 30, reps: int = 5, stream=None) -> float:
    """pi_ae_debug_stream_read: the best plain streaming-read rate in GB/s."""
    lib = load_library()
    out = ctypes.c_float()
    _check(lib.pi_ae_debug_stream_read(int(nbytes), int(reps), _stream_handle(stream), ctypes.byref(out)))
    return float(out.value)


def graph_floor_us(kernels: int = 200, grid: int = 256, stream=None) -> float:
    """pi_ae_debug_graph_floor: time per kernel of a replayed graph of empty dependent kernels."""
    lib = load_library()
    out = ctypes.c_float()
    _check(lib.pi_ae_debug_graph_floor(int(kernels), int(grid), _stream_handle(stream), ctypes.byref(out)))
    return float(out.value)


def grid_sync_us(rounds: int = 2000, mode: int = 0, stream=None) -> float:
    """pi_ae_debug_grid_sync: time per grid-wide barrier round inside one persistent kernel."""
    lib = load_library()
    out = ctypes.c_float()
    _check(lib.pi_ae_debug_grid_sync(int(rounds), int(mode), _stream_handle(stream), ctypes.byref(out)))
    return float(out.value)


class Inference:
    """pi_ae_inference: vision encoder, VLM prefill and denoise loop of one episode as one graph."""

    def __init__(self, vision: Vision, prefill: Prefill, ctx: "Context"):
        self._lib = load_library()
        self.vision, self.prefill, self.ctx = vision, prefill, ctx  # keeps the three alive
        handle = ctypes.c_void_p()
        _check(self._lib.pi_ae_inference_create(vision._h, prefill._h, ctx._h, ctypes.byref(handle)))
        self._h = handle

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            self._lib.pi_ae_inference_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def run(self, images, views: int, prompt_emb, prompt_len: int, pad_mask, noise, actions, stream=None):
        im, _ = self.vision._io(images, views, None)
        c = self.vision.cfg
        n = max(int(views), 0) * (c.image // c.patch) ** 2 + max(int(prompt_len), 0)
        pe = _dev(prompt_emb, "prompt_emb", "bf16", max(int(prompt_len), 0) * self.prefill.cfg.width)
        _check(self._lib.pi_ae_inference_run(self._h, im, int(views), pe, int(prompt_len),
                                             _dev(pad_mask, "pad_mask", "u8", n), self.ctx._xbuf(noise, "noise", 1),
                                             self.ctx._xbuf(actions, "actions", 1), _stream_handle(stream)))
