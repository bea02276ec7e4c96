"""Seeded synthetic workloads for the action-expert denoise loop.

This module holds random draws and the bf16 storage format only: none of the
method's arithmetic lives here, so the HIP path and the CPU oracle can both take
their inputs from it without sharing any computation.

Workload shapes follow the pages (Realtime-VLA blog, "pi0.5 inference flow":
256 tokens per camera view, a 32-dim action chunk, an 18-layer expert of width
1024 / MLP 4096 / 8 query heads x 256 / one KV head; "Running VLAs at Real-time
Speed" notes, Table 1: empty prompt, chunk length 63, 1/2/3 views).  No dataset
or trained checkpoint is used: every tensor below is a seeded Gaussian draw.

Draw recipe (stated here so that any reader can regenerate it):
  * weights: one ``numpy.random.Generator(PCG64(seed))`` stream, seed 0;
    every tensor (biases included) is ``standard_normal(shape, float32) * 0.02``
    rounded to bf16 (round-to-nearest-even).  Order: action_in, time_in,
    time_out, final_mod, action_out (weight then bias each), then for each layer
    attn_mod (w, b), q, k, v, o, ffn_mod (w, b), gate, up, down.
  * the pi0 variant (``variant = 1``: action-time encoder, RMSNorm scales
    instead of AdaRMS; "Running VLAs at Real-time Speed" notes, section How):
    order action_in, action_time_in, action_time_out, final_norm, action_out,
    then per layer attn_norm, q, k, v, o, ffn_norm, gate, up, down; the norm
    scales are 1 + standard_normal * 0.02 (the others as above).
  * prefix K/V cache: seed 1, drawn per layer as K[l] then V[l], each of shape
    [batch][prefix_len][head_dim], N(0, 1) rounded to bf16.
  * noise: seed 2, [batch][chunk][action_dim] N(0, 1) in fp32 (not rounded).
  * pad mask: the first ``n_valid`` prefix positions are valid (1), the rest 0.
  * the VLM prefix prefill (Realtime-VLA blog, "pi0.5 inference flow", Encoder
    phase; section 4 encoder kernel list: width 2048, fused QKV 2560, MLP
    16384, 18 layers): weights seed 3, per layer attn_norm, q, k, v, o,
    ffn_norm, gate, up, down as above (norm scales 1 + N(0, 0.02)); the prefix
    sequence (image and prompt embeddings after their sqrt(2048) scaling)
    seed 4, [batch][prefix_len][2048] N(0, 1) rounded to bf16.
  * the vision encoder (Realtime-VLA blog, "pi0.5 inference flow" and
    "LeRobot implementation": SigLIP, 27 layers, 224x224 -> 256 tokens, width
    1152, projector 1152 -> 2048): weights seed 5 in the order of
    vision_weight_shapes, N(0, 0.02) (LayerNorm scales 1 + N(0, 0.02), their
    biases N(0, 0.02)); images seed 6, [views][224][224][3] uniform in
    [-1, 1) rounded to bf16.
"""
from __future__ import annotations

import dataclasses
import functools
from dataclasses import dataclass

import numpy as np

__all__ = [
    "ExpertConfig", "Workload", "WORKLOADS", "workload",
    "f32_to_bf16_bits", "bf16_bits_to_f32",
    "make_weights", "make_prefix_kv", "make_pad_mask", "make_noise",
    "weight_shapes",
    "PrefillConfig", "PrefillWorkload", "PREFILL_WORKLOADS", "prefill_weight_shapes",
    "make_prefill_weights", "make_prefix_embeddings",
    "VisionConfig", "vision_weight_shapes", "make_vision_weights", "make_images",
]


@dataclass(frozen=True)
class ExpertConfig:
    """Shape and schedule of the action expert (Gemma-300M-shaped, AdaRMS)."""
    num_layers: int = 18
    width: int = 1024
    mlp_dim: int = 4096
    num_heads: int = 8
    num_kv_heads: int = 1
    head_dim: int = 256
    action_dim: int = 32
    chunk_len: int = 63
    num_steps: int = 10
    t0: float = 1.0
    dt: float = -0.1
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    final_norm: bool = True
    variant: int = 0          # 0: pi0.5 (AdaRMS); 1: pi0 (action-time encoder, RMSNorm scales)

    def replace(self, **kw) -> "ExpertConfig":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class Workload:
    """One benchmark / parity workload: the expert plus the call's sizes."""
    name: str
    cfg: ExpertConfig
    batch: int
    prefix_len: int
    n_valid: int
    description: str = ""

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_FULL = ExpertConfig()

WORKLOADS = {
    "c1": Workload("c1", _FULL.replace(num_layers=2, num_steps=1), 1, 256, 256,
                   "reduced expert: 2 layers, 1 Euler step, 1 view (256 prefix keys)"),
    "c2": Workload("c2", _FULL, 1, 256, 256,
                   "18 layers x 10 steps, batch 1, 1 view (256 prefix keys)"),
    "c3": Workload("c3", _FULL, 1, 512, 512,
                   "18 layers x 10 steps, batch 1, 2 views (512 prefix keys)"),
    "c4": Workload("c4", _FULL, 1, 816, 800,
                   "18 layers x 10 steps, batch 1, 3 views + 48 prompt tokens, last 16 padded"),
    "c5": Workload("c5", _FULL.replace(chunk_len=50), 32, 712, 712,
                   "18 layers x 10 steps, 32 episodes x 50 tokens, 2 views + 200 prompt tokens each"),
    # the pi0 variant of the expert (action-time encoder, RMSNorm scales)
    "c1pi0": Workload("c1pi0", _FULL.replace(num_layers=2, num_steps=1, variant=1), 1, 256, 256,
                      "pi0 variant: reduced expert, 2 layers, 1 Euler step, 1 view (256 prefix keys)"),
    "c2pi0": Workload("c2pi0", _FULL.replace(variant=1), 1, 256, 256,
                      "pi0 variant: 18 layers x 10 steps, batch 1, 1 view (256 prefix keys)"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


# ---------------------------------------------------------------- bf16 format
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exactly equal fp32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- weights
def weight_shapes(cfg: ExpertConfig):
    """(name, shape) in draw order; nn.Linear layout [out][in]."""
    D, F, H, d, A = cfg.width, cfg.mlp_dim, cfg.num_heads, cfg.head_dim, cfg.action_dim
    kv = cfg.num_kv_heads * d
    if cfg.variant == 1:
        out = [("action_in.w", (D, A)), ("action_in.b", (D,)),
               ("action_time_in.w", (D, 2 * D)), ("action_time_in.b", (D,)),
               ("action_time_out.w", (D, D)), ("action_time_out.b", (D,))]
        if cfg.final_norm:
            out += [("final_norm.w", (D,))]
        out += [("action_out.w", (A, D)), ("action_out.b", (A,))]
        for l in range(cfg.num_layers):
            p = f"layers.{l}."
            out += [
                (p + "attn_norm.w", (D,)),
                (p + "q.w", (H * d, D)), (p + "k.w", (kv, D)), (p + "v.w", (kv, D)),
                (p + "o.w", (D, H * d)),
                (p + "ffn_norm.w", (D,)),
                (p + "gate.w", (F, D)), (p + "up.w", (F, D)), (p + "down.w", (D, F)),
            ]
        return out
    out = [
        ("action_in.w", (D, A)), ("action_in.b", (D,)),
        ("time_in.w", (D, D)), ("time_in.b", (D,)),
        ("time_out.w", (D, D)), ("time_out.b", (D,)),
        ("final_mod.w", (3 * D, D)), ("final_mod.b", (3 * D,)),
        ("action_out.w", (A, D)), ("action_out.b", (A,)),
    ]
    for l in range(cfg.num_layers):
        p = f"layers.{l}."
        out += [
            (p + "attn_mod.w", (3 * D, D)), (p + "attn_mod.b", (3 * D,)),
            (p + "q.w", (H * d, D)), (p + "k.w", (kv, D)), (p + "v.w", (kv, D)),
            (p + "o.w", (D, H * d)),
            (p + "ffn_mod.w", (3 * D, D)), (p + "ffn_mod.b", (3 * D,)),
            (p + "gate.w", (F, D)), (p + "up.w", (F, D)), (p + "down.w", (D, F)),
        ]
    return out


def _weights_uncached(cfg: ExpertConfig, seed: int, std: float) -> dict:
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, shape in weight_shapes(cfg):
        x = rng.standard_normal(shape, dtype=np.float32)
        x *= np.float32(std)
        if name.endswith("norm.w"):  # a norm's scale: around 1
            x += np.float32(1.0)
        out[name] = f32_to_bf16_bits(x)
    return out


@functools.lru_cache(maxsize=2)
def _weights_cached(cfg: ExpertConfig, seed: int, std: float):
    w = _weights_uncached(cfg, seed, std)
    for v in w.values():
        v.setflags(write=False)
    return w


def make_weights(cfg: ExpertConfig, seed: int = 0, std: float = 0.02, cache: bool = True) -> dict:
    """Unfolded expert weights as bf16 bit patterns, keyed by tensor name.

    Arrays from the cache are read-only; pass ``cache=False`` to get a fresh,
    writable set (tests that edit weights do that).
    """
    if cache:
        return dict(_weights_cached(cfg, seed, std))
    return _weights_uncached(cfg, seed, std)


# ---------------------------------------------------------------- call inputs
def make_prefix_kv(cfg: ExpertConfig, batch: int, prefix_len: int, seed: int = 1):
    """Prefix K and V, each bf16 bits [L][batch][P][head_dim] (RoPE already applied by the producer)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    L, d = cfg.num_layers, cfg.num_kv_heads * cfg.head_dim
    k = np.empty((L, batch, prefix_len, d), np.uint16)
    v = np.empty((L, batch, prefix_len, d), np.uint16)
    for l in range(L):
        k[l] = f32_to_bf16_bits(rng.standard_normal((batch, prefix_len, d), dtype=np.float32))
        v[l] = f32_to_bf16_bits(rng.standard_normal((batch, prefix_len, d), dtype=np.float32))
    return k, v


def make_pad_mask(batch: int, prefix_len: int, n_valid) -> np.ndarray:
    """u8 [batch][P]; the first n_valid[b] positions valid (n_valid: int or per-episode list)."""
    nv = np.broadcast_to(np.asarray(n_valid, dtype=np.int64), (batch,))
    m = np.zeros((batch, prefix_len), np.uint8)
    for b in range(batch):
        m[b, : int(nv[b])] = 1
    return m


def make_noise(cfg: ExpertConfig, batch: int, seed: int = 2) -> np.ndarray:
    """fp32 [batch][chunk][action_dim] ~ N(0, 1): the initial state x at t = t0."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((batch, cfg.chunk_len, cfg.action_dim), dtype=np.float32)


def make_workload_inputs(w: Workload, weight_seed: int = 0, kv_seed: int = 1, noise_seed: int = 2):
    """Everything one call needs: (weights, k, v, pad_mask, noise)."""
    weights = make_weights(w.cfg, weight_seed)
    k, v = make_prefix_kv(w.cfg, w.batch, w.prefix_len, kv_seed)
    mask = make_pad_mask(w.batch, w.prefix_len, w.n_valid)
    noise = make_noise(w.cfg, w.batch, noise_seed)
    return weights, k, v, mask, noise


# ---------------------------------------------------------------- VLM prefix prefill
@dataclass(frozen=True)
class PrefillConfig:
    """Shape of the Gemma-2B-shaped VLM whose layers fill the prefix KV cache."""
    num_layers: int = 18
    width: int = 2048
    mlp_dim: int = 16384
    num_heads: int = 8
    num_kv_heads: int = 1
    head_dim: int = 256
    rope_base: float = 10000.0
    rms_eps: float = 1e-6

    def replace(self, **kw) -> "PrefillConfig":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    cfg: PrefillConfig
    batch: int
    prefix_len: int
    n_valid: int
    description: str = ""


_VLM = PrefillConfig()

PREFILL_WORKLOADS = {
    "p1": PrefillWorkload("p1", _VLM, 1, 256, 256, "VLM prefill, 18 layers, 1 view (256 tokens), empty prompt"),
    "p2": PrefillWorkload("p2", _VLM, 1, 512, 512, "VLM prefill, 18 layers, 2 views (512 tokens), empty prompt"),
    "p3": PrefillWorkload("p3", _VLM, 1, 816, 800,
                          "VLM prefill, 18 layers, 3 views + 48 prompt tokens, last 16 padded"),
}


def prefill_weight_shapes(cfg: PrefillConfig):
    """(name, shape) in draw order; nn.Linear layout [out][in]."""
    D, F, H, d = cfg.width, cfg.mlp_dim, cfg.num_heads, cfg.head_dim
    kv = cfg.num_kv_heads * d
    out = []
    for l in range(cfg.num_layers):
        p = f"layers.{l}."
        out += [
            (p + "attn_norm.w", (D,)),
            (p + "q.w", (H * d, D)), (p + "k.w", (kv, D)), (p + "v.w", (kv, D)),
            (p + "o.w", (D, H * d)),
            (p + "ffn_norm.w", (D,)),
            (p + "gate.w", (F, D)), (p + "up.w", (F, D)), (p + "down.w", (D, F)),
        ]
    return out


def make_prefill_weights(cfg: PrefillConfig, seed: int = 3, std: float = 0.02) -> dict:
    """VLM weights as bf16 bit patterns keyed ``layers.{l}.<name>`` (a fresh dict)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, shape in prefill_weight_shapes(cfg):
        x = rng.standard_normal(shape, dtype=np.float32)
        x *= np.float32(std)
        if name.endswith("norm.w"):
            x += np.float32(1.0)
        out[name] = f32_to_bf16_bits(x)
    return out


def make_prefix_embeddings(cfg: PrefillConfig, batch: int, prefix_len: int, seed: int = 4) -> np.ndarray:
    """The prefix sequence, bf16 bits [batch][prefix_len][width] ~ N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return f32_to_bf16_bits(rng.standard_normal((batch, prefix_len, cfg.width), dtype=np.float32))


# ---------------------------------------------------------------- vision encoder
@dataclass(frozen=True)
class VisionConfig:
    """Shape of the SigLIP-shaped vision encoder (one view: 256 patch tokens)."""
    num_layers: int = 27
    width: int = 1152
    mlp_dim: int = 4304
    num_heads: int = 16
    head_dim: int = 72
    patch: int = 14
    image: int = 224
    channels: int = 3
    out_width: int = 2048
    ln_eps: float = 1e-6

    def replace(self, **kw) -> "VisionConfig":
        return dataclasses.replace(self, **kw)


def vision_weight_shapes(cfg: VisionConfig):
    """(name, shape) in draw order; nn.Linear layout [out][in], convolution [out][c][y][x]."""
    D, F, P, C = cfg.width, cfg.mlp_dim, cfg.patch, cfg.channels
    n = (cfg.image // P) ** 2
    out = [("patch.w", (D, C, P, P)), ("patch.b", (D,)), ("pos", (n, D))]
    for l in range(cfg.num_layers):
        p = f"layers.{l}."
        out += [(p + "ln1.w", (D,)), (p + "ln1.b", (D,)),
                (p + "q.w", (D, D)), (p + "q.b", (D,)), (p + "k.w", (D, D)), (p + "k.b", (D,)),
                (p + "v.w", (D, D)), (p + "v.b", (D,)), (p + "o.w", (D, D)), (p + "o.b", (D,)),
                (p + "ln2.w", (D,)), (p + "ln2.b", (D,)),
                (p + "fc1.w", (F, D)), (p + "fc1.b", (F,)), (p + "fc2.w", (D, F)), (p + "fc2.b", (D,))]
    out += [("post_ln.w", (D,)), ("post_ln.b", (D,)), ("proj.w", (cfg.out_width, D)), ("proj.b", (cfg.out_width,))]
    return out


def make_vision_weights(cfg: VisionConfig, seed: int = 5, std: float = 0.02) -> dict:
    """Vision-encoder weights as bf16 bit patterns (a fresh dict)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, shape in vision_weight_shapes(cfg):
        x = rng.standard_normal(shape, dtype=np.float32)
        x *= np.float32(std)
        if name.endswith("ln1.w") or name.endswith("ln2.w") or name == "post_ln.w":
            x += np.float32(1.0)
        out[name] = f32_to_bf16_bits(x)
    return out


def make_images(cfg: VisionConfig, views: int, seed: int = 6) -> np.ndarray:
    """bf16 bits [views][image][image][channels], uniform in [-1, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.random((views, cfg.image, cfg.image, cfg.channels), dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    return f32_to_bf16_bits(x)
