"""CPU oracle for the SigLIP-shaped vision encoder that turns each camera view
into the image tokens of the VLM prefix.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: tests, the smoke check and the benchmark's CPU baseline use it to
check the HIP path.  It shares no code with the HIP path or its weight
preparation (only the generic helpers of the expert oracle next to it).

What it computes, in fp64 by default:

  Realtime-VLA technical blog (blog.w4k4.me), section "pi0.5 inference flow":
  the vision encoder is SigLIP (400M), which turns a 224x224 view into 256
  tokens; the Encoder (prefix) phase scales them by sqrt(2048) before they join
  the prompt tokens.  Section "LeRobot implementation" (class tree): the
  vision tower has 27 layers and is followed by the multi-modal projector, a
  Linear 1152 -> 2048.  Section 4 (partial split-K): the vision encoder's
  attention projections are 1152 x 1152 GEMMs.

Readings taken where the pages are silent (also listed in the repository's
design notes):
  * the SigLIP-So400m/14 layer: 14x14 patches (224 / 14 = 16, 16 x 16 = 256
    tokens) embedded by a strided convolution with bias, plus a learned
    position embedding per patch; pre-norm layers with LayerNorm (scale and
    bias, eps 1e-6), 16 attention heads of 72 (1152 / 16), biases on every
    linear, a 4304-wide MLP with GELU (tanh approximation); a final
    LayerNorm before the projector;
  * attention is bidirectional over the 256 patches of a view (no mask);
  * patches are taken row by row, each flattened in (channel, y, x) order,
    the order of a convolution weight [out][channel][y][x];
  * the projector's output is multiplied by sqrt(2048) (the blog's scaling of
    the image embedding), giving the bf16 prefix tokens the VLM reads;
  * images arrive as [views][224][224][3] (rows, columns, RGB), already
    resized and normalised (resizing is outside this step).

Parity of a trained model's behaviour is unpinned: there are no trained
weights on the pages.
"""
from __future__ import annotations

import math

import numpy as np

from .pi_ae_oracle import attention, bf16_to_float, gelu_tanh


def patchify(img, patch: int):
    """[H][W][C] -> [(H/p)(W/p)][C p p]: patches row by row, each in (c, y, x) order."""
    H, W, C = img.shape
    gy, gx = H // patch, W // patch
    x = img.reshape(gy, patch, gx, patch, C).transpose(0, 2, 4, 1, 3)  # [gy][gx][c][y][x]
    return x.reshape(gy * gx, C * patch * patch)


def layer_norm(h, w, b, eps):
    """(h - mean) / sqrt(var + eps) * w + b over the last axis."""
    mu = h.mean(axis=-1, keepdims=True)
    var = ((h - mu) ** 2).mean(axis=-1, keepdims=True)
    return (h - mu) / np.sqrt(var + eps) * w + b


def vision_layer(get, h, cfg):
    """One pre-norm encoder layer on one view's tokens h [n][width]."""
    n = h.shape[0]
    H, d, eps = cfg.num_heads, cfg.head_dim, cfg.ln_eps
    u = layer_norm(h, get("ln1.w"), get("ln1.b"), eps)
    q = (u @ get("q.w").T + get("q.b")).reshape(n, H, d)
    k = (u @ get("k.w").T + get("k.b")).reshape(n, H, d)
    v = (u @ get("v.w").T + get("v.b")).reshape(n, H, d)
    valid = np.ones(n, bool)
    o = np.concatenate([attention(q[:, hh:hh + 1, :], k[:, hh, :], v[:, hh, :], valid, 1.0 / math.sqrt(d))
                        for hh in range(H)], axis=1).reshape(n, H * d)
    h = h + o @ get("o.w").T + get("o.b")
    u2 = layer_norm(h, get("ln2.w"), get("ln2.b"), eps)
    return h + gelu_tanh(u2 @ get("fc1.w").T + get("fc1.b")) @ get("fc2.w").T + get("fc2.b")


def vision_encode(weight_bits: dict, cfg, image_bits, dtype=np.float64, layers=None):
    """Image tokens of every view: bf16 images [V][224][224][3] -> [V][256][out_width].

    weight_bits: bf16 bits keyed as in the input module's vision_weight_shapes
    (convolution weight [width][3][patch][patch]); ``layers`` limits the run to
    the first n encoder layers (the post-norm and the projector still apply).
    """
    L = cfg.num_layers if layers is None else layers
    f = lambda name: bf16_to_float(weight_bits[name], dtype)
    imgs = bf16_to_float(image_bits, dtype)
    V = imgs.shape[0]
    wpatch = f("patch.w").reshape(cfg.width, -1)
    out = np.empty((V, (cfg.image // cfg.patch) ** 2, cfg.out_width), dtype)
    layer_w = [dict() for _ in range(L)]
    for v in range(V):
        h = patchify(imgs[v], cfg.patch) @ wpatch.T + f("patch.b") + f("pos")
        for l in range(L):
            if not layer_w[l]:
                for key in weight_bits:
                    if key.startswith(f"layers.{l}."):
                        layer_w[l][key[len(f"layers.{l}."):]] = f(key)
            h = vision_layer(layer_w[l].__getitem__, h, cfg)
        h = layer_norm(h, f("post_ln.w"), f("post_ln.b"), cfg.ln_eps)
        out[v] = (h @ f("proj.w").T + f("proj.b")) * math.sqrt(cfg.out_width)
    return out
