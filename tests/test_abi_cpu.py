"""C-ABI checks that need no GPU: the library loads and exports every symbol
the header declares, arguments are validated (with the documented status codes)
before any device work, and the host half of the weight preparation (fp64
tabulation and shift folding) equals the oracle's folded tables."""
import ctypes
import os
import re

import numpy as np
import pytest

from flow_matching_action_amd import inputs
from flow_matching_action_amd import pi_ae
from oracle import pi_ae_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pi_ae.h")

def _has_hipcc():
    import shutil
    return bool(shutil.which("hipcc")) or os.path.exists("/opt/rocm/bin/hipcc")


# Where the toolchain is present the library must have been built (a missing
# build is a failure, not a skip); only a machine without hipcc skips.
needs_lib = pytest.mark.skipif(not os.path.exists(pi_ae.LIB_PATH) and not _has_hipcc(),
                               reason="no ROCm toolchain to build libpi_ae.so")



def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pi_ae_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert header_functions() == sorted(pi_ae.EXPORTS)


@needs_lib
def test_library_exports_every_header_symbol():
    lib = ctypes.CDLL(pi_ae.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {pi_ae.LIB_PATH}").read()
    exported = set(re.findall(r"\bT (pi_ae_\w+)", out))
    assert exported == set(header_functions())


@needs_lib
def test_status_strings_and_null_arguments():
    lib = pi_ae.load_library()
    assert lib.pi_ae_status_string(0) == b"ok"
    assert lib.pi_ae_status_string(pi_ae.PI_AE_EUNSUPPORTED) == b"unsupported shape"
    assert lib.pi_ae_status_string(99) == b"unknown status"
    assert lib.pi_ae_prepare_weights(None, None, None) == pi_ae.PI_AE_EINVAL
    assert b"non-NULL" in lib.pi_ae_last_error()
    kv = pi_ae.PrefixKV(None, None, None, 0)
    assert lib.pi_ae_sample(None, ctypes.byref(kv), None, None, 1, None) == pi_ae.PI_AE_EINVAL
    assert lib.pi_ae_destroy(None) is None


def _tiny_weights(cfg):
    return {n: np.zeros(s, np.uint16) for n, s in inputs.weight_shapes(cfg)}


@needs_lib
@pytest.mark.parametrize("field,value,status", [
    ("width", 512, pi_ae.PI_AE_EUNSUPPORTED),
    ("num_kv_heads", 2, pi_ae.PI_AE_EUNSUPPORTED),
    ("head_dim", 128, pi_ae.PI_AE_EUNSUPPORTED),
    ("num_layers", 0, pi_ae.PI_AE_EINVAL),
    ("num_steps", 0, pi_ae.PI_AE_EINVAL),
    ("chunk_len", 0, pi_ae.PI_AE_EINVAL),
    ("chunk_len", 257, pi_ae.PI_AE_EINVAL),
    ("max_batch", 0, pi_ae.PI_AE_EINVAL),
    ("max_batch", 1025, pi_ae.PI_AE_EINVAL),
    ("max_prefix_len", -1, pi_ae.PI_AE_EINVAL),
    ("max_prefix_len", 8193, pi_ae.PI_AE_EINVAL),
    ("rope_base", 0.0, pi_ae.PI_AE_EINVAL),
    ("final_norm", 2, pi_ae.PI_AE_EINVAL),
])
def test_config_validation(field, value, status):
    """Invalid configs are rejected before any allocation (no GPU needed)."""
    cfg = inputs.WORKLOADS["c1"].cfg
    c = pi_ae.make_config(cfg, 1, 16)
    setattr(c, field, value)
    mw = pi_ae._MarshalledWeights(cfg, _tiny_weights(cfg))
    lib = pi_ae.load_library()
    h = ctypes.c_void_p()
    assert lib.pi_ae_prepare_weights(ctypes.byref(c), ctypes.byref(mw.w), ctypes.byref(h)) == status
    assert h.value is None
    assert lib.pi_ae_last_error() != b""


@needs_lib
def test_rows_per_gemm_limit():
    """max_batch x chunk_len (the rows of every GEMM) is limited to 65536."""
    cfg = inputs.WORKLOADS["c1"].cfg
    mw = pi_ae._MarshalledWeights(cfg, _tiny_weights(cfg))
    lib = pi_ae.load_library()
    for batch, T, status in [(1024, 65, pi_ae.PI_AE_EINVAL), (257, 256, pi_ae.PI_AE_EINVAL)]:
        c = pi_ae.make_config(cfg.replace(chunk_len=T), batch, 16)
        h = ctypes.c_void_p()
        assert lib.pi_ae_prepare_weights(ctypes.byref(c), ctypes.byref(mw.w), ctypes.byref(h)) == status
        assert h.value is None and b"65536" in lib.pi_ae_last_error()


@needs_lib
def test_missing_weight_pointer():
    cfg = inputs.WORKLOADS["c1"].cfg
    w = _tiny_weights(cfg)
    del w["layers.1.up.w"]
    with pytest.raises(pi_ae.PiAeError) as e:
        pi_ae.host_table(cfg, w, 8, cfg.num_steps)
    assert e.value.status == pi_ae.PI_AE_EINVAL and "layer 1" in str(e.value)
    w = _tiny_weights(cfg)
    del w["final_mod.b"]
    with pytest.raises(pi_ae.PiAeError):
        pi_ae.host_table(cfg, w, 8, cfg.num_steps)
    # without the final norm its modulation is not needed
    pi_ae.host_table(cfg.replace(final_norm=False), w, 8, cfg.num_steps)


@needs_lib
def test_host_tables_match_oracle():
    """The library's fp64 preparation equals the oracle's folded tables
    (tabulated time MLP, modulation split, shift folded into c = shift @ W^T)."""
    cfg = inputs.WORKLOADS["c1"].cfg.replace(num_steps=3, dt=-1.0 / 3)
    wb = inputs.make_weights(cfg, seed=3, std=0.05, cache=False)
    W = O.Weights(wb, cfg)
    tabs = O.folded_tables(W)
    S, L, D = cfg.num_steps, cfg.num_layers, cfg.width

    def get(which, n):
        return pi_ae.host_table(cfg, wb, which, n).astype(np.float64)

    def close(got, want, rtol=2e-6):
        want = np.asarray(want, np.float64).ravel()
        err = np.max(np.abs(got - want))
        assert err <= rtol * max(1.0, np.max(np.abs(want))), err

    close(get(8, S), tabs["t"])
    close(get(9, S * D), np.concatenate(tabs["cond"]))
    close(get(0, S * L * D), [tabs["attn"][k][l]["scale1"] for k in range(S) for l in range(L)])
    close(get(1, S * L * D), [tabs["attn"][k][l]["gate"] for k in range(S) for l in range(L)])
    close(get(2, S * L * D), [tabs["ffn"][k][l]["scale1"] for k in range(S) for l in range(L)])
    close(get(3, S * L * D), [tabs["ffn"][k][l]["gate"] for k in range(S) for l in range(L)])
    close(get(4, S * D), [tabs["final"][k]["scale1"] for k in range(S)])
    close(get(5, S * 32), [tabs["final"][k]["c_out"] for k in range(S)])
    close(get(6, S * L * 2560), [tabs["attn"][k][l]["c_qkv"] for k in range(S) for l in range(L)])
    close(get(7, S * L * 8192), [tabs["ffn"][k][l]["c_gu"] for k in range(S) for l in range(L)])
    # without the final norm, c_out is the bare output bias
    cfg2 = cfg.replace(final_norm=False)
    close(pi_ae.host_table(cfg2, wb, 5, S * 32).astype(np.float64),
          np.tile(O.bf16_to_float(wb["action_out.b"]), S))


@needs_lib
def test_host_tables_match_oracle_pi0():
    """pi0 variant: the library's fp64 preparation equals the oracle's folded
    tables (norm scales as (1 + scale), unit gates, zero shift biases, the
    action-time encoder's per-step bias before its SiLU)."""
    cfg = inputs.WORKLOADS["c1pi0"].cfg.replace(num_steps=3, dt=-1.0 / 3)
    wb = inputs.make_weights(cfg, seed=4, std=0.05, cache=False)
    W = O.Weights(wb, cfg)
    tabs = O.folded_tables(W)
    S, L, D = cfg.num_steps, cfg.num_layers, cfg.width

    def close(which, n, want, rtol=2e-6):
        got = pi_ae.host_table(cfg, wb, which, n).astype(np.float64)
        want = np.asarray(want, np.float64).ravel()
        err = np.max(np.abs(got - want))
        assert err <= rtol * max(1.0, np.max(np.abs(want))), (which, err)

    close(8, S, tabs["t"])
    close(9, S * D, np.concatenate(tabs["cond"]))
    close(0, S * L * D, [tabs["attn"][k][l]["scale1"] for k in range(S) for l in range(L)])
    close(1, S * L * D, [tabs["attn"][k][l]["gate"] for k in range(S) for l in range(L)])
    close(2, S * L * D, [tabs["ffn"][k][l]["scale1"] for k in range(S) for l in range(L)])
    close(3, S * L * D, [tabs["ffn"][k][l]["gate"] for k in range(S) for l in range(L)])
    close(4, S * D, [tabs["final"][k]["scale1"] for k in range(S)])
    close(5, S * 32, [tabs["final"][k]["c_out"] for k in range(S)])
    close(6, S * L * 2560, np.zeros(S * L * 2560))
    close(7, S * L * 8192, np.zeros(S * L * 8192))


@needs_lib
def test_pi0_weight_validation():
    cfg = inputs.WORKLOADS["c1pi0"].cfg
    w = _tiny_weights(cfg)
    del w["layers.1.ffn_norm.w"]
    with pytest.raises(pi_ae.PiAeError) as e:
        pi_ae.host_table(cfg, w, 8, cfg.num_steps)
    assert e.value.status == pi_ae.PI_AE_EINVAL and "layer 1" in str(e.value)
    w = _tiny_weights(cfg)
    del w["action_time_in.b"]
    with pytest.raises(pi_ae.PiAeError):
        pi_ae.host_table(cfg, w, 8, cfg.num_steps)
    c = pi_ae.make_config(cfg, 1, 16)
    c.variant = 2
    mw = pi_ae._MarshalledWeights(cfg, _tiny_weights(cfg))
    h = ctypes.c_void_p()
    assert pi_ae.load_library().pi_ae_prepare_weights(ctypes.byref(c), ctypes.byref(mw.w), ctypes.byref(h)) == \
        pi_ae.PI_AE_EINVAL


# ------------------------------------------------------------------ VLM prefill
def _vlm_null_layers(L):
    return (pi_ae.VlmLayerWeights * L)()


@needs_lib
@pytest.mark.parametrize("field,value,status", [
    ("width", 1024, pi_ae.PI_AE_EUNSUPPORTED),
    ("mlp_dim", 8192, pi_ae.PI_AE_EUNSUPPORTED),
    ("num_kv_heads", 8, pi_ae.PI_AE_EUNSUPPORTED),
    ("head_dim", 128, pi_ae.PI_AE_EUNSUPPORTED),
    ("num_layers", 0, pi_ae.PI_AE_EINVAL),
    ("num_layers", 65, pi_ae.PI_AE_EINVAL),
    ("max_batch", 0, pi_ae.PI_AE_EINVAL),
    ("max_prefix_len", 0, pi_ae.PI_AE_EINVAL),
    ("max_prefix_len", 4097, pi_ae.PI_AE_EINVAL),
    ("rms_eps", 0.0, pi_ae.PI_AE_EINVAL),
])
def test_vlm_config_validation(field, value, status):
    """pi_ae_vlm_prepare rejects unsupported shapes and bad limits before any
    device work (no GPU needed)."""
    cfg = inputs.PrefillConfig(num_layers=2)
    c = pi_ae.make_vlm_config(cfg, 1, 256)
    setattr(c, field, value)
    lib = pi_ae.load_library()
    h = ctypes.c_void_p()
    layers = _vlm_null_layers(max(c.num_layers, 1))
    assert lib.pi_ae_vlm_prepare(ctypes.byref(c), layers, ctypes.byref(h)) == status
    assert h.value is None
    assert lib.pi_ae_last_error() != b""


@needs_lib
def test_vlm_weight_pointers_and_null_arguments():
    lib = pi_ae.load_library()
    cfg = inputs.PrefillConfig(num_layers=2)
    c = pi_ae.make_vlm_config(cfg, 1, 256)
    h = ctypes.c_void_p()
    assert lib.pi_ae_vlm_prepare(None, None, None) == pi_ae.PI_AE_EINVAL
    # every pointer NULL: layer 0 is named
    assert lib.pi_ae_vlm_prepare(ctypes.byref(c), _vlm_null_layers(2), ctypes.byref(h)) == pi_ae.PI_AE_EINVAL
    assert b"layer 0" in lib.pi_ae_last_error()
    # the last layer needs only its norm and Q/K/V; the others everything
    keep = {n: np.zeros(s, np.uint16) for n, s in inputs.prefill_weight_shapes(cfg)}
    for n in ("o", "ffn_norm", "gate", "up", "down"):
        del keep[f"layers.0.{n}.w"]
    mw = pi_ae._MarshalledVlmWeights(cfg, keep)
    assert lib.pi_ae_vlm_prepare(ctypes.byref(c), mw.layers, ctypes.byref(h)) == pi_ae.PI_AE_EINVAL
    assert b"layer 0" in lib.pi_ae_last_error()
    kv = pi_ae.PrefixKV()
    assert lib.pi_ae_vlm_prefill(None, None, None, 1, 1, ctypes.byref(kv), None) == pi_ae.PI_AE_EINVAL
    us = ctypes.c_float()
    assert lib.pi_ae_vlm_debug_time_phase(None, None, None, 1, 1, 1, 1, None, ctypes.byref(us)) == pi_ae.PI_AE_EINVAL
    assert lib.pi_ae_vlm_destroy(None) is None



# ------------------------------------------------------------------ vision encoder
@needs_lib
@pytest.mark.parametrize("field,value,status", [
    ("width", 1024, pi_ae.PI_AE_EUNSUPPORTED),
    ("head_dim", 64, pi_ae.PI_AE_EUNSUPPORTED),
    ("patch", 16, pi_ae.PI_AE_EUNSUPPORTED),
    ("num_layers", 0, pi_ae.PI_AE_EINVAL),
    ("max_views", 0, pi_ae.PI_AE_EINVAL),
    ("max_views", 65, pi_ae.PI_AE_EINVAL),
    ("ln_eps", 0.0, pi_ae.PI_AE_EINVAL),
])
def test_vision_config_validation(field, value, status):
    """pi_ae_vision_prepare rejects unsupported shapes and bad limits before
    any device work (no GPU needed)."""
    cfg = inputs.VisionConfig(num_layers=2)
    c = pi_ae.make_vision_config(cfg, 1)
    setattr(c, field, value)
    lib = pi_ae.load_library()
    w = pi_ae.VisionWeights()
    h = ctypes.c_void_p()
    assert lib.pi_ae_vision_prepare(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)) == status
    assert h.value is None
    assert lib.pi_ae_last_error() != b""


@needs_lib
def test_vision_weight_pointers_and_null_arguments():
    lib = pi_ae.load_library()
    cfg = inputs.VisionConfig(num_layers=2)
    c = pi_ae.make_vision_config(cfg, 1)
    h = ctypes.c_void_p()
    assert lib.pi_ae_vision_prepare(None, None, None) == pi_ae.PI_AE_EINVAL
    w = {n: np.zeros(s, np.uint16) for n, s in inputs.vision_weight_shapes(cfg)}
    del w["layers.1.fc2.b"]
    mw = pi_ae._MarshalledVisionWeights(cfg, w)
    assert lib.pi_ae_vision_prepare(ctypes.byref(c), ctypes.byref(mw.w), ctypes.byref(h)) == pi_ae.PI_AE_EINVAL
    assert b"layer 1" in lib.pi_ae_last_error()
    assert lib.pi_ae_vision_encode(None, None, 1, None, None) == pi_ae.PI_AE_EINVAL
    us = ctypes.c_float()
    assert lib.pi_ae_vision_debug_time_phase(None, None, 1, None, 0, 1, None, ctypes.byref(us)) == pi_ae.PI_AE_EINVAL
    assert lib.pi_ae_vision_destroy(None) is None
