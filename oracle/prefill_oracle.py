"""CPU oracle for the VLM prefix prefill that produces the expert's KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: tests, the smoke check and the benchmark's CPU baseline use it to
check the HIP path.  It shares no code with the HIP path or its weight
preparation (only the generic helpers of the expert oracle next to it).

What it computes, in fp64 by default, is the encoder (prefix) phase as the
pages describe it:

  Realtime-VLA technical blog (blog.w4k4.me), section "pi0.5 inference flow",
  Encoder (prefix) phase, run once per inference: the image tokens (256 per
  view) and the prompt tokens, each already scaled by sqrt(2048), are joined
  into the prefix sequence, which passes through the 18 layers of the Gemma-2B
  VLM; every layer's key and value are kept as the KV cache that the action
  expert reads.  The same blog, section 4 (kernel fusion), lists the encoder
  layer as RMSNorm + fused QKV projection (2048 -> 2560) + RoPE, O projection
  (2048 -> 2048) + residual, RMSNorm + gated up projection (2048 -> 16384,
  gate and up), down projection (16384 -> 2048) + residual; its section 4.1
  runs only 17 layers in full, because the 18th hands over nothing but its
  keys and values.

Readings taken where the pages are silent (also listed in the repository's
design notes):
  * the input is the prefix sequence after the sqrt(2048) scaling (the vision
    encoder and the token embedding are not part of this step);
  * the norms are RMS norms with a learnable scale gamma that multiplies the
    normalised activation (eps 1e-6), like the pi0 expert's; no biases;
  * 8 query heads x 256 and one KV head of 256 (2560 = (8 + 2) x 256, and the
    expert attends to these keys with its own 256-wide heads);
  * attention is bidirectional over the prefix: every token attends to every
    valid (pad mask 1) token of its episode, masked keys excluded exactly;
  * a token sits at the RoPE position given by the number of valid tokens
    before it in its episode (rotate-half pairs, base 10000, as for the
    expert's keys): the valid tokens take positions 0 .. n_valid - 1 in order
    whatever pads lie between them, which is where the expert's suffix, at
    n_valid + j, continues them; the cache holds the rotated keys, which is
    what the expert expects of its prefix cache;
  * the MLP is GELU(tanh)(x W_g^T) * (x W_u^T), then W_d;
  * an episode without any valid token has no softmax support: its attention
    output is taken as 0.

Parity of a trained model's behaviour is unpinned: there are no trained
weights on the pages.
"""
from __future__ import annotations

import math

import numpy as np

from .pi_ae_oracle import attention, bf16_to_float, gelu_tanh, rms_normalize, rope


def prefill_layer(get, l: int, h, key_valid, positions, cfg, kv_only: bool = False):
    """One VLM layer on one episode; returns (h after the layer, K, V).

    (Blog section 4 kernel list, Encoder layers: RMSNorm + QKV + RoPE, O +
    residual, RMSNorm + gated up, down + residual.)  ``get(name)`` returns the
    layer's fp weight; h: [P][D]; key_valid: bool [P].  With ``kv_only`` the
    layer stops after its keys and values (blog section 4.1: the last layer's
    attention and MLP are skipped) and h is returned unchanged.
    """
    P = h.shape[0]
    H, d, eps = cfg.num_heads, cfg.head_dim, cfg.rms_eps
    u = rms_normalize(h, eps) * get("attn_norm.w")
    k = rope(u @ get("k.w").T, positions, cfg.rope_base)
    v = u @ get("v.w").T
    if kv_only:
        return h, k, v
    q = (u @ get("q.w").T).reshape(P, H, d)
    q = rope(q.transpose(1, 0, 2), positions, cfg.rope_base).transpose(1, 0, 2)
    if key_valid.any():
        o = attention(q, k, v, key_valid, 1.0 / math.sqrt(d)).reshape(P, H * d)
    else:  # no valid key in the episode: the softmax has no support; taken as 0
        o = np.zeros((P, H * d), h.dtype)
    h = h + o @ get("o.w").T
    u2 = rms_normalize(h, eps) * get("ffn_norm.w")
    m = gelu_tanh(u2 @ get("gate.w").T) * (u2 @ get("up.w").T)
    return h + m @ get("down.w").T, k, v


def token_positions(key_valid):
    """RoPE position of every prefix token: the number of valid tokens before it.

    (The expert's suffix token j sits at n_valid + j, right after the valid
    prefix tokens; this places those at 0 .. n_valid - 1 in order, so that pads
    anywhere in the prefix leave no gap in the positions.  With trailing pads it
    is simply the token's index.)
    """
    v = np.asarray(key_valid, bool)
    return np.concatenate([[0], np.cumsum(v)[:-1]]) if v.size else np.zeros(0, np.int64)


def prefill(weight_bits: dict, cfg, emb_bits, pad_mask, dtype=np.float64, full_last_layer: bool = False,
            layers=None):
    """The prefix KV cache of every layer.

    weight_bits: bf16 bits keyed ``layers.{l}.<name>`` (nn.Linear layout
    [out][in]); emb_bits: bf16 [B][P][D], the scaled prefix sequence; pad_mask:
    [B][P] (nonzero = valid) or None.  Returns (K, V), each ``dtype``
    [L][B][P][head_dim] with RoPE applied to K.  ``full_last_layer`` runs the
    last layer in full too (its keys and values cannot depend on it: a check
    of the 17-layer shortcut).  ``layers`` limits the run to the first n
    layers' caches.
    """
    L = cfg.num_layers if layers is None else layers
    emb = bf16_to_float(emb_bits, dtype)
    B, P, _ = emb.shape
    valid = np.ones((B, P), bool) if pad_mask is None else np.asarray(pad_mask) != 0
    d = cfg.num_kv_heads * cfg.head_dim
    K = np.empty((L, B, P, d), dtype)
    V = np.empty((L, B, P, d), dtype)
    cache = {}

    def getter(l):
        def get(name):
            key = f"layers.{l}.{name}"
            if key not in cache:
                cache.clear()  # one layer's weights at a time (the full VLM is ~4 GB of bf16)
                for n in ("attn_norm.w", "q.w", "k.w", "v.w", "o.w", "ffn_norm.w", "gate.w", "up.w", "down.w"):
                    cache[f"layers.{l}.{n}"] = bf16_to_float(weight_bits[f"layers.{l}.{n}"], dtype)
            return cache[key]
        return get

    hs = [emb[b] for b in range(B)]
    for l in range(L):
        get = getter(l)
        last = (l == cfg.num_layers - 1) and not full_last_layer
        for b in range(B):
            hs[b], K[l, b], V[l, b] = prefill_layer(get, l, hs[b], valid[b], token_positions(valid[b]), cfg,
                                                    kv_only=last)
    return K, V
