"""CPU oracle for the pi0.5-style action-expert flow-matching denoise loop.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: it exists so that tests, the smoke check and the benchmark's CPU
baseline can check the HIP path against a plain, slow, obviously correct
reference.  It shares no code with the HIP path or its weight preparation; it
reads only its inputs (bf16 bit patterns, fp32 noise, u8 masks) and NumPy.

What it computes is the UNFOLDED model as the pages describe it, in fp64 by
default (``dtype=np.float32`` is available for CPU timing):

  Realtime-VLA technical blog (blog.w4k4.me), section "pi0.5 inference flow",
  Decoder (suffix) phase, repeated for every denoise step:
    1. the noisy chunk goes through action_in_proj (Linear 32->1024); the
       timestep goes through a sinusoidal embedding and a two-layer time MLP
       whose output is the AdaRMS condition;
    2. every expert layer: AdaRMS norm (a dense 1024->3072 maps the condition
       to scale, shift and gate; x_norm * (1 + scale) + shift), Q/K/V
       projections + RoPE, attention over the prefix KV cache together with
       the suffix's own keys, O projection, gated residual (res + out * gate),
       then AdaRMS norm, GELU-gated MLP and a second gated residual;
    3. action_out_proj (Linear 1024->32) gives the velocity v_t;
    4. Euler step x <- x + dt * v_t with dt = -1/num_steps.
  The same page, section "LeRobot implementation", gives the per-layer shapes
  (q 1024->2048 as 8 heads x 256, k and v 1024->256 for one KV head, o
  2048->1024, bias-free gate/up 1024->4096 and down 4096->1024) and the
  "eager attention" form Q K^T * scaling -> softmax -> V after repeat_kv.

Readings taken where the pages are silent or ambiguous (each also listed in the
design notes of the repository):
  * sinusoidal embedding: [sin(2 pi t / tau_i) | cos(2 pi t / tau_i)],
    i < width/2, periods tau_i geometric from 4e-3 to 4.0 (not on the pages);
  * time MLP order: the explicit precompute formula of the blog's section
    "precompute (__init__)", SiLU(Linear(SiLU(Linear(emb)))), is followed;
  * RMS epsilon 1e-6; AdaRMS has no separate gamma, its affine is (1+scale, shift);
  * a final AdaRMS norm with its own modulation dense precedes action_out_proj
    (flag ``final_norm``; the pages go straight from the layers to the output);
  * attention scaling 1/sqrt(head_dim); masked prefix keys are excluded exactly
    (the pages fill them with -2.38e38 before the softmax, which gives exp = 0);
  * GELU is the tanh approximation; biases only on action_in, the time MLP,
    the modulation denses and action_out;
  * RoPE pairs (i, i + head_dim/2) ("rotate half"), inverse frequencies
    base^(-2i/head_dim) from the blog's precompute section; the prefix keys
    arrive already rotated; suffix token j sits at position n_valid + j, where
    n_valid is the number of valid prefix keys of its episode;
  * the modulation output is split in contiguous thirds (scale, shift, gate);
    the gate is used as is (no activation);
  * timestep k is t_k = fp32(t0 + k * dt), evaluated in fp64.

The pi0 variant (``cfg.variant == 1``) follows the "Running VLAs at Real-time
Speed" notes (knowledgebase summary, section How) and the Realtime-VLA blog's
section 3.2: the expert layers use plain RMS norms with a learnable scale
gamma (x_norm * gamma, which the pages fold into the next linear) and plain
residuals; the step input is the action-time encoder, whose two linear layers
the pages fold, tabulating the per-timestep part into the bias before the SiLU.
Readings: the encoder is Linear(2048 -> 1024) on the concatenation
[action_in_proj(x) | emb(t)], then SiLU, then Linear(1024 -> 1024); a final RMS
norm with its own scale precedes action_out_proj (flag ``final_norm``).

Every function states the passage it follows.  Parity of the trained model's
behaviour is unpinned: there are no trained weights on the pages.
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------- helpers


def bf16_to_float(bits, dtype=np.float64) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact values in ``dtype``."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(dtype)


def silu(x):
    """SiLU(x) = x * sigmoid(x) (time MLP of the blog's "pi0.5 inference flow")."""
    return x / (1.0 + np.exp(-x))


def gelu_tanh(x):
    """GELU, tanh approximation (the MLP activation, "LeRobot implementation" layer list)."""
    c = math.sqrt(2.0 / math.pi)
    return 0.5 * x * (1.0 + np.tanh(c * (x + 0.044715 * x ** 3)))


def timesteps(num_steps: int, t0: float, dt: float) -> np.ndarray:
    """t_k for k = 0..S-1.

    The blog's section 3.2 ("Action Time Encoder folding") says only
    t in {1.0, 0.9, ..., 0.1} occur; with dt = -1/num_steps ("pi0.5 inference
    flow", Euler step) that is t_k = t0 + k dt.  Each t_k is evaluated in fp64
    from the fp32 config values and stored as fp32.
    """
    t0 = float(np.float32(t0))
    dt = float(np.float32(dt))
    return np.array([float(np.float32(t0 + k * dt)) for k in range(num_steps)], dtype=np.float64)


def sinusoidal_embedding(t: float, dim: int, min_period: float = 4e-3, max_period: float = 4.0,
                         dtype=np.float64) -> np.ndarray:
    """Sinusoidal timestep embedding ("pi0.5 inference flow", step 1: t -> 1024 dims).

    The pages do not define it; the reading taken is dim/2 sine and dim/2 cosine
    channels whose periods grow geometrically from ``min_period`` to
    ``max_period``: channel i (i < dim/2) has period
    tau_i = min_period * (max_period / min_period) ** (i / (dim/2 - 1)).
    """
    half = dim // 2
    frac = np.arange(half, dtype=np.float64) / (half - 1)
    period = min_period * (max_period / min_period) ** frac
    ang = 2.0 * math.pi * float(t) / period
    return np.concatenate([np.sin(ang), np.cos(ang)]).astype(dtype)


def rms_normalize(h, eps):
    """h / sqrt(mean(h^2) + eps) over the last axis (the RMS part of AdaRMS)."""
    r = np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return h / r


def adarms(h, scale, shift, eps):
    """AdaRMS: x_norm * (1 + scale) + shift ("pi0.5 inference flow", layer step)."""
    return rms_normalize(h, eps) * (1.0 + scale) + shift


def rope(x, positions, base):
    """Rotary position embedding on the last axis ("LeRobot implementation",
    apply_rotary_pos_emb; inverse frequencies from the blog's precompute section).

    x: [..., n, d]; positions: [n].  Channel pair (i, i + d/2) is rotated by
    angle positions * base^(-2i/d).
    """
    d = x.shape[-1]
    half = d // 2
    inv_freq = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang).astype(x.dtype)
    sin = np.sin(ang).astype(x.dtype)
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def attention(q, k, v, key_valid, scale):
    """Softmax attention of H query heads sharing one KV head.

    ("LeRobot implementation": repeat_kv expands the single KV head to the 8
    query heads, then Q K^T * scaling -> softmax -> V; the prefix pad mask
    removes invalid keys: the Realtime-VLA prefix/suffix softmax kernel fills
    them with -2.38e38, i.e. weight exactly 0 after exp.)

    q: [n_q, H, d]; k, v: [n_k, d]; key_valid: bool [n_k].  Returns [n_q, H, d].
    """
    kk = k[key_valid]
    vv = v[key_valid]
    s = np.einsum("qhd,kd->qhk", q, kk) * scale
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.einsum("qhk,kd->qhd", p, vv)


# --------------------------------------------------------------------------- model


class Weights:
    """Unfolded weights upcast from bf16 bits, nn.Linear layout [out][in]."""

    def __init__(self, bits: dict, cfg, dtype=np.float64):
        self.cfg = cfg
        self.dtype = dtype
        self.w = {name: bf16_to_float(arr, dtype) for name, arr in bits.items()}

    def __getitem__(self, name):
        return self.w[name]

    def layer(self, l, name):
        return self.w[f"layers.{l}.{name}"]


def time_condition(W: Weights, t: float) -> np.ndarray:
    """adarms_cond for timestep t: SiLU(Linear(SiLU(Linear(emb(t))))).

    (Blog section "precompute (__init__)": the time embedding is the formula
    SiLU(Linear(SiLU(Linear(t)))) evaluated once per timestep.)
    """
    D = W.cfg.width
    emb = sinusoidal_embedding(t, D, dtype=W.dtype)
    a = silu(W["time_in.w"] @ emb + W["time_in.b"])
    return silu(W["time_out.w"] @ a + W["time_out.b"])


def modulation(w, b, cond):
    """dense(cond) split into (scale, shift, gate), contiguous thirds
    ("pi0.5 inference flow": a dense 1024->3072 produces scale, shift and gate)."""
    m = w @ cond + b
    D = m.shape[0] // 3
    return m[:D], m[D:2 * D], m[2 * D:]


def expert_layer(W: Weights, l: int, h, cond, prefix_k, prefix_v, key_valid, positions):
    """One expert decoder layer on one episode ("LeRobot implementation",
    PiGemmaDecoderLayer.forward).  h: [T][D]; prefix_k/v: [P][d]."""
    cfg = W.cfg
    T = h.shape[0]
    H, d = cfg.num_heads, cfg.head_dim
    eps = cfg.rms_eps
    # attention block
    s, sh, g = modulation(W.layer(l, "attn_mod.w"), W.layer(l, "attn_mod.b"), cond)
    u = adarms(h, s, sh, eps)
    q = (u @ W.layer(l, "q.w").T).reshape(T, H, d)
    ks = u @ W.layer(l, "k.w").T
    vs = u @ W.layer(l, "v.w").T
    q = rope(q.transpose(1, 0, 2), positions, cfg.rope_base).transpose(1, 0, 2)
    ks = rope(ks, positions, cfg.rope_base)
    keys = np.concatenate([prefix_k, ks], axis=0)
    vals = np.concatenate([prefix_v, vs], axis=0)
    valid = np.concatenate([key_valid, np.ones(T, dtype=bool)])
    o = attention(q, keys, vals, valid, 1.0 / math.sqrt(d)).reshape(T, H * d)
    h = h + (o @ W.layer(l, "o.w").T) * g            # gated residual
    # MLP block
    s2, sh2, g2 = modulation(W.layer(l, "ffn_mod.w"), W.layer(l, "ffn_mod.b"), cond)
    u2 = adarms(h, s2, sh2, eps)
    m = gelu_tanh(u2 @ W.layer(l, "gate.w").T) * (u2 @ W.layer(l, "up.w").T)
    h = h + (m @ W.layer(l, "down.w").T) * g2        # gated residual
    return h


def encoder_pi0(W: Weights, x, t) -> np.ndarray:
    """pi0 step input: Linear(SiLU(Linear([action_in_proj(x) | emb(t)]))).

    ("Running VLAs at Real-time Speed" notes, section How: the action-time
    encoder has two linear layers with a SiLU between them; its input joins the
    projected action chunk with the timestep embedding.)  x: [T][A] -> [T][D].
    """
    D = W.cfg.width
    a = x @ W["action_in.w"].T + W["action_in.b"]
    emb = sinusoidal_embedding(t, D, dtype=W.dtype)
    cat = np.concatenate([a, np.broadcast_to(emb, a.shape)], axis=1)
    z = silu(cat @ W["action_time_in.w"].T + W["action_time_in.b"])
    return z @ W["action_time_out.w"].T + W["action_time_out.b"]


def expert_layer_pi0(W: Weights, l: int, h, prefix_k, prefix_v, key_valid, positions):
    """One pi0 expert layer: RMS norm with scale gamma, attention, residual,
    RMS norm with scale gamma, GELU-gated MLP, residual (Realtime-VLA blog,
    section 3.2: the norm's learnable scale multiplies the normalised
    activation)."""
    cfg = W.cfg
    T = h.shape[0]
    H, d = cfg.num_heads, cfg.head_dim
    eps = cfg.rms_eps
    u = rms_normalize(h, eps) * W.layer(l, "attn_norm.w")
    q = (u @ W.layer(l, "q.w").T).reshape(T, H, d)
    ks = u @ W.layer(l, "k.w").T
    vs = u @ W.layer(l, "v.w").T
    q = rope(q.transpose(1, 0, 2), positions, cfg.rope_base).transpose(1, 0, 2)
    ks = rope(ks, positions, cfg.rope_base)
    keys = np.concatenate([prefix_k, ks], axis=0)
    vals = np.concatenate([prefix_v, vs], axis=0)
    valid = np.concatenate([key_valid, np.ones(T, dtype=bool)])
    o = attention(q, keys, vals, valid, 1.0 / math.sqrt(d)).reshape(T, H * d)
    h = h + o @ W.layer(l, "o.w").T
    u2 = rms_normalize(h, eps) * W.layer(l, "ffn_norm.w")
    m = gelu_tanh(u2 @ W.layer(l, "gate.w").T) * (u2 @ W.layer(l, "up.w").T)
    return h + m @ W.layer(l, "down.w").T


def velocity(W: Weights, x, t, prefix_k, prefix_v, key_valid):
    """v_t for one episode: x [T][A] -> [T][A] ("pi0.5 inference flow", steps 1-3).

    prefix_k/v: [L][P][d] (values); key_valid: bool [P].
    """
    cfg = W.cfg
    n_valid = int(np.count_nonzero(key_valid))
    positions = n_valid + np.arange(x.shape[0])
    if cfg.variant == 1:
        h = encoder_pi0(W, x, t)
        for l in range(cfg.num_layers):
            h = expert_layer_pi0(W, l, h, prefix_k[l], prefix_v[l], key_valid, positions)
        if cfg.final_norm:
            h = rms_normalize(h, cfg.rms_eps) * W["final_norm.w"]
        return h @ W["action_out.w"].T + W["action_out.b"]
    cond = time_condition(W, t)
    h = x @ W["action_in.w"].T + W["action_in.b"]
    for l in range(cfg.num_layers):
        h = expert_layer(W, l, h, cond, prefix_k[l], prefix_v[l], key_valid, positions)
    if cfg.final_norm:
        sf, shf, _ = modulation(W["final_mod.w"], W["final_mod.b"], cond)
        h = adarms(h, sf, shf, cfg.rms_eps)
    return h @ W["action_out.w"].T + W["action_out.b"]


def sample(weight_bits: dict, cfg, prefix_k_bits, prefix_v_bits, pad_mask, noise,
           dtype=np.float64, weights: Weights | None = None, return_velocities=False):
    """The denoise loop: x <- x + dt * v_t for t = t_0 .. t_{S-1}.

    ("pi0.5 inference flow", step 4: Euler integration with dt = -1/num_steps.)
    prefix_k/v_bits: bf16 [L][B][P][d]; pad_mask: [B][P] (nonzero = valid);
    noise: fp32 [B][T][A].  Returns x after S steps as ``dtype`` [B][T][A]
    (and the per-step velocities when asked).
    """
    W = weights if weights is not None else Weights(weight_bits, cfg, dtype)
    dt = float(np.float32(cfg.dt))
    ts = timesteps(cfg.num_steps, cfg.t0, cfg.dt)
    B = noise.shape[0]
    pk = bf16_to_float(prefix_k_bits, dtype)
    pv = bf16_to_float(prefix_v_bits, dtype)
    if pad_mask is None:
        valid = np.ones(pk.shape[1:3], dtype=bool)
    else:
        valid = np.asarray(pad_mask) != 0
    out = np.empty(noise.shape, dtype=dtype)
    vels = []
    for b in range(B):
        x = noise[b].astype(dtype)
        vb = []
        for t in ts:
            v = velocity(W, x, t, pk[:, b], pv[:, b], valid[b])
            vb.append(v)
            x = x + dt * v
        out[b] = x
        vels.append(vb)
    if return_velocities:
        return out, vels
    return out


# --------------------------------------------------------------------------- folded graph


def folded_tables(W: Weights):
    """The one-time tables of the folded graph, in fp64.

    (Blog section "precompute (__init__)": the time embedding for the 10
    timesteps and the per-(step, layer) style projections time_emb @ mod_w +
    mod_b are computed once; action_out_proj's weight and bias are multiplied by
    dt so the loop only adds.  Section 3.2: the norm affine is absorbed into the
    following linear, and Q, K, V become one (hidden, (heads + 2) * head_dim)
    matrix.)  For AdaRMS the affine is per (step, layer): the shift folds into a
    bias c = shift @ W^T of the following linear, the scale stays an elementwise
    factor on the normalised activation.
    """
    cfg = W.cfg
    ts = timesteps(cfg.num_steps, cfg.t0, cfg.dt)
    L = cfg.num_layers
    tabs = {"t": ts, "cond": [], "attn": [], "ffn": [], "final": []}
    if cfg.variant == 1:
        return _folded_tables_pi0(W, ts, tabs)
    for t in ts:
        cond = time_condition(W, t)
        tabs["cond"].append(cond)
        attn_k, ffn_k = [], []
        for l in range(L):
            wqkv = np.concatenate([W.layer(l, "q.w"), W.layer(l, "k.w"), W.layer(l, "v.w")], axis=0)
            s, sh, g = modulation(W.layer(l, "attn_mod.w"), W.layer(l, "attn_mod.b"), cond)
            attn_k.append({"scale1": 1.0 + s, "shift": sh, "gate": g, "c_qkv": wqkv @ sh})
            wgu = np.concatenate([W.layer(l, "gate.w"), W.layer(l, "up.w")], axis=0)
            s2, sh2, g2 = modulation(W.layer(l, "ffn_mod.w"), W.layer(l, "ffn_mod.b"), cond)
            ffn_k.append({"scale1": 1.0 + s2, "shift": sh2, "gate": g2, "c_gu": wgu @ sh2})
        tabs["attn"].append(attn_k)
        tabs["ffn"].append(ffn_k)
        if cfg.final_norm:
            sf, shf, _ = modulation(W["final_mod.w"], W["final_mod.b"], cond)
            c_out = W["action_out.w"] @ shf + W["action_out.b"]
            tabs["final"].append({"scale1": 1.0 + sf, "shift": shf, "c_out": c_out})
        else:
            tabs["final"].append({"scale1": None, "shift": None, "c_out": W["action_out.b"].copy()})
    return tabs


def _folded_tables_pi0(W: Weights, ts, tabs):
    """pi0: the encoder's two linear layers folded ("Running VLAs at Real-time
    Speed" notes, section How: the per-timestep part becomes a tabulated bias
    before the SiLU): W_fold = W_ti[:, :D] @ W_in and, per step k, c_k =
    W_ti[:, :D] @ b_in + W_ti[:, D:] @ emb(t_k) + b_ti; the layers' norm scales
    become the (1 + scale) factors (shift 0, gate 1)."""
    cfg = W.cfg
    D, L = cfg.width, cfg.num_layers
    wti = W["action_time_in.w"]
    tabs["w_fold"] = wti[:, :D] @ W["action_in.w"]
    for t in ts:
        emb = sinusoidal_embedding(t, D, dtype=np.float64)
        tabs["cond"].append(wti[:, :D] @ W["action_in.b"] + wti[:, D:] @ emb + W["action_time_in.b"])
        attn_k, ffn_k = [], []
        for l in range(L):
            zq = np.zeros(cfg.num_heads * cfg.head_dim + 2 * cfg.head_dim)
            attn_k.append({"scale1": W.layer(l, "attn_norm.w").copy(), "shift": np.zeros(D),
                           "gate": np.ones(D), "c_qkv": zq})
            ffn_k.append({"scale1": W.layer(l, "ffn_norm.w").copy(), "shift": np.zeros(D),
                          "gate": np.ones(D), "c_gu": np.zeros(2 * cfg.mlp_dim)})
        tabs["attn"].append(attn_k)
        tabs["ffn"].append(ffn_k)
        if cfg.final_norm:
            tabs["final"].append({"scale1": W["final_norm.w"].copy(), "shift": np.zeros(D),
                                  "c_out": W["action_out.b"].copy()})
        else:
            tabs["final"].append({"scale1": None, "shift": None, "c_out": W["action_out.b"].copy()})
    return tabs


def sample_folded(weight_bits: dict, cfg, prefix_k_bits, prefix_v_bits, pad_mask, noise,
                  weights: Weights | None = None, tables=None):
    """The same loop evaluated through the folded graph, in fp64.

    Used only to pin the fold identities: it must equal ``sample`` to rounding.
    Shift-as-bias (c = shift @ W^T), fused QKV with RoPE applied to the fused
    output, fused gate/up, and the dt-scaled action_out_proj (x <- x + out).
    """
    W = weights if weights is not None else Weights(weight_bits, cfg, np.float64)
    tabs = tables if tables is not None else folded_tables(W)
    D, H, d, F = cfg.width, cfg.num_heads, cfg.head_dim, cfg.mlp_dim
    L, eps = cfg.num_layers, cfg.rms_eps
    dt = float(np.float32(cfg.dt))
    pk = bf16_to_float(prefix_k_bits, np.float64)
    pv = bf16_to_float(prefix_v_bits, np.float64)
    valid_all = np.ones(pk.shape[1:3], bool) if pad_mask is None else np.asarray(pad_mask) != 0
    w_out_dt = dt * W["action_out.w"]
    B, T, _ = noise.shape
    out = np.empty(noise.shape)
    for b in range(B):
        x = noise[b].astype(np.float64)
        valid = valid_all[b]
        n_valid = int(np.count_nonzero(valid))
        pos = n_valid + np.arange(T)
        for k in range(cfg.num_steps):
            if cfg.variant == 1:
                z = silu(x @ tabs["w_fold"].T + tabs["cond"][k])
                h = z @ W["action_time_out.w"].T + W["action_time_out.b"]
            else:
                h = x @ W["action_in.w"].T + W["action_in.b"]
            for l in range(L):
                ta = tabs["attn"][k][l]
                wqkv = np.concatenate([W.layer(l, "q.w"), W.layer(l, "k.w"), W.layer(l, "v.w")], axis=0)
                qkv = (rms_normalize(h, eps) * ta["scale1"]) @ wqkv.T + ta["c_qkv"]
                q = qkv[:, :H * d].reshape(T, H, d)
                ks = qkv[:, H * d:H * d + d]
                vs = qkv[:, H * d + d:]
                q = rope(q.transpose(1, 0, 2), pos, cfg.rope_base).transpose(1, 0, 2)
                ks = rope(ks, pos, cfg.rope_base)
                keys = np.concatenate([pk[l, b], ks])
                vals = np.concatenate([pv[l, b], vs])
                kv_valid = np.concatenate([valid, np.ones(T, bool)])
                o = attention(q, keys, vals, kv_valid, 1.0 / math.sqrt(d)).reshape(T, H * d)
                h = h + (o @ W.layer(l, "o.w").T) * ta["gate"]
                tf = tabs["ffn"][k][l]
                wgu = np.concatenate([W.layer(l, "gate.w"), W.layer(l, "up.w")], axis=0)
                gu = (rms_normalize(h, eps) * tf["scale1"]) @ wgu.T + tf["c_gu"]
                m = gelu_tanh(gu[:, :F]) * gu[:, F:]
                h = h + (m @ W.layer(l, "down.w").T) * tf["gate"]
            tfin = tabs["final"][k]
            if cfg.final_norm:
                uf = rms_normalize(h, eps) * tfin["scale1"]
            else:
                uf = h
            x = x + (uf @ w_out_dt.T + dt * tfin["c_out"])
        out[b] = x
    return out
