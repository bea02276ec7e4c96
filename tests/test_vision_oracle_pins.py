"""Pins of the vision-encoder oracle to facts that do not come from it.

The vision oracle (oracle/vision_oracle.py) is checked against: the figures
the pages give (27 layers, 256 tokens from 224x224, width 1152, the 1152 ->
2048 projector, the sqrt(2048) scale), a library convolution for the patch
embedding, the textbook properties of LayerNorm, brute force with scalar loops
on a tiny encoder, and invariances the mathematics fixes (relabelling the
attention heads, episodes of views being independent).
"""
import json
import math
import os

import numpy as np
import torch

from flow_matching_action_amd import inputs
from oracle import pi_ae_oracle as O
from oracle import vision_oracle as VO

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")

TINY = inputs.VisionConfig(num_layers=2, width=8, mlp_dim=12, num_heads=2, head_dim=4, patch=2, image=6,
                           out_width=5)


def test_vision_shapes_match_pages():
    with open(GOLDEN) as f:
        g = json.load(f)["vision"]
    cfg = inputs.VisionConfig()
    shapes = dict(inputs.vision_weight_shapes(cfg))
    assert cfg.num_layers == g["layers"] == sum(1 for n in shapes if n.endswith(".q.w"))
    assert (cfg.image // cfg.patch) ** 2 == g["tokens_per_view"] and cfg.image == g["image_side"]
    assert shapes["layers.0.q.w"] == (g["width"], g["width"])   # the 1152 x 1152 attention GEMMs
    assert list(shapes["proj.w"][::-1]) == g["projector"]
    assert g["output_scale"] == f"sqrt({cfg.out_width})"
    assert cfg.num_heads * cfg.head_dim == cfg.width


def test_patch_embedding_is_the_strided_convolution():
    cfg = TINY
    rng = np.random.default_rng(0)
    img = rng.standard_normal((cfg.image, cfg.image, cfg.channels))
    w = rng.standard_normal((cfg.width, cfg.channels, cfg.patch, cfg.patch))
    b = rng.standard_normal(cfg.width)
    ours = VO.patchify(img, cfg.patch) @ w.reshape(cfg.width, -1).T + b
    ref = torch.nn.functional.conv2d(torch.from_numpy(img.transpose(2, 0, 1))[None], torch.from_numpy(w),
                                     torch.from_numpy(b), stride=cfg.patch)[0]        # [width][gy][gx]
    ref = ref.numpy().reshape(cfg.width, -1).T                                       # patches row by row
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-12)


def test_layer_norm_textbook():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((5, 16)) * 3 + 7
    y = VO.layer_norm(h, np.ones(16), np.zeros(16), 0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose((y ** 2).mean(axis=1), 1, atol=1e-12)
    # a constant row normalises to the bias
    bias = rng.standard_normal(16)
    np.testing.assert_allclose(VO.layer_norm(np.full((1, 16), 4.0), rng.standard_normal(16), bias, 1e-6)[0], bias,
                               atol=1e-12)
    torch_ln = torch.nn.functional.layer_norm(torch.from_numpy(h), (16,), eps=1e-6).numpy()
    np.testing.assert_allclose(VO.layer_norm(h, np.ones(16), np.zeros(16), 1e-6), torch_ln, rtol=1e-10, atol=1e-12)


def _brute(wb, cfg, img_bits):
    f = lambda n: O.bf16_to_float(wb[n]).tolist()
    D, H, d, P = cfg.width, cfg.num_heads, cfg.head_dim, cfg.patch
    g = cfg.image // P
    out = []
    for img in O.bf16_to_float(img_bits):
        W, bw, pos = f("patch.w"), f("patch.b"), f("pos")
        h = []
        for py in range(g):
            for px in range(g):
                row = []
                for o in range(D):
                    acc = bw[o] + pos[py * g + px][o]
                    for c in range(cfg.channels):
                        for y in range(P):
                            for x in range(P):
                                acc += W[o][c][y][x] * img[py * P + y][px * P + x][c]
                    row.append(acc)
                h.append(row)
        n = len(h)

        def ln(rows, w, b):
            res = []
            for r in rows:
                mu = sum(r) / D
                var = sum((x - mu) ** 2 for x in r) / D
                res.append([(r[i] - mu) / math.sqrt(var + cfg.ln_eps) * w[i] + b[i] for i in range(D)])
            return res

        def lin(rows, w, b):
            return [[b[o] + sum(r[i] * w[o][i] for i in range(len(r))) for o in range(len(w))] for r in rows]

        for l in range(cfg.num_layers):
            p = lambda s_: f(f"layers.{l}.{s_}")
            u = ln(h, p("ln1.w"), p("ln1.b"))
            q, k, v = lin(u, p("q.w"), p("q.b")), lin(u, p("k.w"), p("k.b")), lin(u, p("v.w"), p("v.b"))
            o = [[0.0] * D for _ in range(n)]
            for hh in range(H):
                for i in range(n):
                    s = [sum(q[i][hh * d + e] * k[j][hh * d + e] for e in range(d)) / math.sqrt(d) for j in range(n)]
                    mx = max(s)
                    z = sum(math.exp(x - mx) for x in s)
                    for e in range(d):
                        o[i][hh * d + e] = sum(math.exp(s[j] - mx) / z * v[j][hh * d + e] for j in range(n))
            ao = lin(o, p("o.w"), p("o.b"))
            h = [[h[i][c] + ao[i][c] for c in range(D)] for i in range(n)]
            u2 = ln(h, p("ln2.w"), p("ln2.b"))
            m = [[0.5 * x * (1 + math.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3))) for x in r]
                 for r in lin(u2, p("fc1.w"), p("fc1.b"))]
            mo = lin(m, p("fc2.w"), p("fc2.b"))
            h = [[h[i][c] + mo[i][c] for c in range(D)] for i in range(n)]
        h = ln(h, f("post_ln.w"), f("post_ln.b"))
        out.append([[x * math.sqrt(cfg.out_width) for x in r] for r in lin(h, f("proj.w"), f("proj.b"))])
    return np.array(out)


def test_vision_encoder_matches_brute_force():
    wb = inputs.make_vision_weights(TINY, seed=7, std=0.3)
    imgs = inputs.make_images(TINY, 2, seed=8)
    np.testing.assert_allclose(VO.vision_encode(wb, TINY, imgs), _brute(wb, TINY, imgs), rtol=1e-10, atol=1e-10)


def test_relabelling_heads_changes_nothing():
    """Swapping the two heads (their q, k, v rows and the matching o columns)
    leaves the output unchanged: the heads are computed independently."""
    wb = inputs.make_vision_weights(TINY, seed=9, std=0.3)
    imgs = inputs.make_images(TINY, 1, seed=10)
    ref = VO.vision_encode(wb, TINY, imgs)
    d = TINY.head_dim
    perm = np.concatenate([np.arange(d, 2 * d), np.arange(0, d)])
    w2 = dict(wb)
    for l in range(TINY.num_layers):
        for n in ("q", "k", "v"):
            w2[f"layers.{l}.{n}.w"] = wb[f"layers.{l}.{n}.w"][perm]
            w2[f"layers.{l}.{n}.b"] = wb[f"layers.{l}.{n}.b"][perm]
        w2[f"layers.{l}.o.w"] = wb[f"layers.{l}.o.w"][:, perm]
    np.testing.assert_allclose(VO.vision_encode(w2, TINY, imgs), ref, rtol=1e-12, atol=1e-12)


def test_views_are_independent():
    wb = inputs.make_vision_weights(TINY, seed=11, std=0.3)
    imgs = inputs.make_images(TINY, 3, seed=12)
    out = VO.vision_encode(wb, TINY, imgs)
    for v in range(3):
        np.testing.assert_allclose(VO.vision_encode(wb, TINY, imgs[v:v + 1])[0], out[v], rtol=1e-12, atol=1e-12)
