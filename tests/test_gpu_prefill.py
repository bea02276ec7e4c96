"""Parity of the VLM prefix prefill (HIP path, through the C-ABI) with the
CPU oracle (oracle/prefill_oracle.py), and of the whole pipeline: prefill,
then the denoise loop on the cache the prefill leaves.

Bars.  The cache of layer l is compared with the fp64 oracle on the same
seeded inputs.  Its values have an rms near 0.9; the HIP path rounds every
GEMM operand (the normalised activations, the attention output, the MLP
product) and the cache itself to bf16, which costs about 2.3e-3 relative
rms at layer 0, and a residual network of random layers carries each
layer's rounding forward undamped, so independent per-layer errors add up
as the square root of the depth.  The bar is therefore
rel-L2(l) <= 3.5e-3 * sqrt(l + 1) (1.5x the layer-0 rounding, growing as the
accumulated rounding does; 1.5e-2 at the 18th layer) and max-abs(l) <= 8 *
rel-L2 bar (about 9 standard deviations of the error at rms 0.9).  The
whole pipeline's final actions keep the loop's own bar (relative L2 <=
1e-2, max-abs <= 5e-2).  Pad-token rows are compared like the others: both
sides compute them by the same definition.
"""
import ctypes

import numpy as np
import pytest
import torch

from flow_matching_action_amd import inputs
from flow_matching_action_amd import pi_ae
from oracle import pi_ae_oracle as O
from oracle import prefill_oracle as PO

pytestmark = pytest.mark.gpu

TOL_REL_L2 = 1e-2      # final actions of the pipeline
TOL_MAX_ABS = 5e-2


def cache_tol(l):
    """(rel-L2, max-abs) bar for layer l's K and V."""
    rel = 3.5e-3 * (l + 1) ** 0.5
    return rel, 8 * rel


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    pi_ae.load_library()
    yield
    torch.cuda.synchronize()


def to_dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rel_l2(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-30))


_hip = None


def _memcpy_d2d(dst, src, nbytes):
    """hipMemcpy device to device (the cache is the library's own memory)."""
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    assert _hip.hipMemcpy(dst, src, nbytes, 3) == 0  # hipMemcpyDeviceToDevice


def cache_to_host(kv, L, B, P):
    """The cache a prefill filled (device pointers in kv) as bf16 bits [L][B][P][256]."""
    n = L * B * P * 256
    out = []
    for ptr in (kv.k, kv.v):
        t = torch.empty(n, dtype=torch.int16, device="cuda")
        torch.cuda.synchronize()
        _memcpy_d2d(t.data_ptr(), ptr, n * 2)
        out.append(t.cpu().numpy().view(np.uint16).reshape(L, B, P, 256))
    return out


def run_prefill(cfg, w, emb, mask, max_batch=None, max_prefix=None, pf=None):
    B, P = emb.shape[0], emb.shape[1]
    own = pf is None
    if own:
        pf = pi_ae.Prefill(cfg, w, max_batch or B, max_prefix or P)
    demb, dmask = to_dev(emb), to_dev(mask)
    kv = pf.run(demb, dmask, B, P)
    torch.cuda.synchronize()
    k, v = cache_to_host(kv, cfg.num_layers, B, P)
    if own:
        pf.close()
    return k, v


def check_cache(k_bits, v_bits, K, V, tag):
    for l in range(K.shape[0]):
        kg, vg = O.bf16_to_float(k_bits[l]), O.bf16_to_float(v_bits[l])
        ek, ev = rel_l2(kg, K[l]), rel_l2(vg, V[l])
        mk, mv = float(np.max(np.abs(kg - K[l]))), float(np.max(np.abs(vg - V[l])))
        tr, ta = cache_tol(l)
        if l in (0, K.shape[0] - 1) or max(ek, ev) > tr or max(mk, mv) > ta:
            log(f"[{tag}] layer {l}: K rel_l2={ek:.3e} max_abs={mk:.3e}  V rel_l2={ev:.3e} max_abs={mv:.3e}"
                f"  (bar {tr:.2e} / {ta:.2e})")
        assert np.all(np.isfinite(kg)) and np.all(np.isfinite(vg))
        assert ek <= tr and ev <= tr and mk <= ta and mv <= ta, (l, ek, ev, mk, mv)


def test_prefill_reduced_ragged_two_episodes():
    """3 layers at full width; 300 tokens (a ragged last key block and row
    tile); episode 1 has 290 valid tokens."""
    cfg = inputs.PrefillConfig(num_layers=3)
    w = inputs.make_prefill_weights(cfg)
    emb = inputs.make_prefix_embeddings(cfg, 2, 300)
    mask = inputs.make_pad_mask(2, 300, [300, 290])
    log("step: prefill 3 layers, B=2, P=300, n_valid=[300, 290]")
    k, v = run_prefill(cfg, w, emb, mask)
    K, V = PO.prefill(w, cfg, emb, mask)
    check_cache(k, v, K, V, "p-reduced")


def test_prefill_edge_sizes():
    """Tiny prefixes (one partial key block, padding past the sequence), an
    episode with no valid token, and a second call on the same context with
    other sizes (graphs per shape, buffers reused)."""
    cfg = inputs.PrefillConfig(num_layers=2)
    w = inputs.make_prefill_weights(cfg)
    pf = pi_ae.Prefill(cfg, w, 3, 64)
    try:
        for B, P, nv in ((2, 40, [37, 0]), (3, 5, [5, 1, 3]), (1, 64, [64])):
            log(f"step: prefill edge B={B} P={P} n_valid={nv}")
            emb = inputs.make_prefix_embeddings(cfg, B, P, seed=9 + P)
            mask = inputs.make_pad_mask(B, P, nv)
            k, v = run_prefill(cfg, w, emb, mask, pf=pf)
            K, V = PO.prefill(w, cfg, emb, mask)
            check_cache(k, v, K, V, f"p-edge B={B} P={P}")
    finally:
        pf.close()


def test_prefill_many_episodes_rows_attention():
    """From 8 episodes on the prefill's attention runs the rows kernel (each
    episode's K/V on one XCD): 9 episodes of 40 tokens, ragged masks, one
    episode without a valid token, 2 layers."""
    cfg = inputs.PrefillConfig(num_layers=2)
    w = inputs.make_prefill_weights(cfg)
    nv = [40, 33, 1, 0, 17, 40, 39, 2, 25]
    B, P = len(nv), 40
    emb = inputs.make_prefix_embeddings(cfg, B, P, seed=21)
    mask = inputs.make_pad_mask(B, P, nv)
    log(f"step: prefill 2 layers, B={B} P={P} n_valid={nv}")
    k, v = run_prefill(cfg, w, emb, mask)
    K, V = PO.prefill(w, cfg, emb, mask)
    check_cache(k, v, K, V, "p-9ep")


def test_prefill_maximum_prefix_length():
    """The context's largest prefix (4096 tokens: 128 key blocks per query,
    2048 query blocks), 2 layers, a ragged tail of pad tokens."""
    cfg = inputs.PrefillConfig(num_layers=2)
    w = inputs.make_prefill_weights(cfg)
    P = 4096
    emb = inputs.make_prefix_embeddings(cfg, 1, P, seed=31)
    mask = inputs.make_pad_mask(1, P, P - 37)
    log(f"step: prefill 2 layers, P={P} (max), {P - 37} valid")
    k, v = run_prefill(cfg, w, emb, mask, max_prefix=4096)
    K, V = PO.prefill(w, cfg, emb, mask)
    check_cache(k, v, K, V, "p-max")


def test_prefill_three_views_with_padded_prompt():
    """The 3-view shape (816 tokens, last 16 padded), 2 layers."""
    cfg = inputs.PrefillConfig(num_layers=2)
    wl = inputs.PREFILL_WORKLOADS["p3"]
    w = inputs.make_prefill_weights(cfg)
    emb = inputs.make_prefix_embeddings(cfg, 1, wl.prefix_len)
    mask = inputs.make_pad_mask(1, wl.prefix_len, wl.n_valid)
    log("step: prefill 2 layers, P=816 (800 valid)")
    k, v = run_prefill(cfg, w, emb, mask)
    K, V = PO.prefill(w, cfg, emb, mask)
    check_cache(k, v, K, V, "p3-2layers")


@pytest.fixture(scope="module")
def full_p1():
    wl = inputs.PREFILL_WORKLOADS["p1"]
    cfg = wl.cfg
    log("step: full VLM weights (18 layers), p1 inputs and oracle")
    w = inputs.make_prefill_weights(cfg)
    emb = inputs.make_prefix_embeddings(cfg, 1, wl.prefix_len)
    mask = inputs.make_pad_mask(1, wl.prefix_len, wl.n_valid)
    K, V = PO.prefill(w, cfg, emb, mask)
    return cfg, w, emb, mask, K, V


def test_prefill_full_one_view(full_p1):
    cfg, w, emb, mask, K, V = full_p1
    log("step: prefill 18 layers, P=256")
    k, v = run_prefill(cfg, w, emb, mask)
    check_cache(k, v, K, V, "p1")


def test_prefill_then_denoise_loop(full_p1):
    """The whole pipeline: the expert samples from the cache the prefill left,
    against the oracle expert on the oracle prefill's cache (rounded to the
    cache's bf16 format)."""
    cfg, w, emb, mask, K, V = full_p1
    ecfg = inputs.ExpertConfig()
    ew = inputs.make_weights(ecfg)
    noise = inputs.make_noise(ecfg, 1)
    B, P = 1, emb.shape[1]
    log("step: prefill 18 layers then the 10-step loop (c2 shape)")
    pf = pi_ae.Prefill(cfg, w, B, P)
    ctx = pi_ae.Context(ecfg, ew, B, P)
    try:
        demb, dmask, dnoise = to_dev(emb), to_dev(mask), to_dev(noise)
        actions = torch.empty_like(dnoise)
        kv = pf.run(demb, dmask, B, P)
        pi_ae.sample_from_cache(ctx, kv, dnoise, actions, B)
        torch.cuda.synchronize()
        x = actions.cpu().numpy()
    finally:
        ctx.close()
        pf.close()
    kb = inputs.f32_to_bf16_bits(K.astype(np.float32))
    vb = inputs.f32_to_bf16_bits(V.astype(np.float32))
    ref = O.sample(ew, ecfg, kb, vb, mask, noise)
    e = rel_l2(x, ref)
    mx = float(np.max(np.abs(x - ref)))
    d = rel_l2(x - noise, ref - noise)
    log(f"[prefill+loop] rel_l2={e:.3e} max_abs={mx:.3e} delta_rel_l2={d:.3e}")
    assert np.all(np.isfinite(x))
    assert e <= TOL_REL_L2 and mx <= TOL_MAX_ABS and d <= 2e-2, (e, mx, d)


def test_pipeline_graph_equals_separate_calls():
    """pi_ae_pipeline_run (prefill and loop in one graph) gives bitwise the
    actions of pi_ae_vlm_prefill followed by pi_ae_sample, and both match the
    oracle pipeline; two sizes on one pipeline."""
    L = 2
    cfg = inputs.PrefillConfig(num_layers=L)
    ecfg = inputs.ExpertConfig(num_layers=L)
    w = inputs.make_prefill_weights(cfg)
    ew = inputs.make_weights(ecfg)
    pf = pi_ae.Prefill(cfg, w, 2, 300)
    ctx = pi_ae.Context(ecfg, ew, 2, 300)
    pipe = pi_ae.Pipeline(pf, ctx)
    try:
        for B, P, nv in ((1, 256, [256]), (2, 300, [300, 290])):
            log(f"step: pipeline B={B} P={P}")
            emb = inputs.make_prefix_embeddings(cfg, B, P)
            mask = inputs.make_pad_mask(B, P, nv)
            noise = inputs.make_noise(ecfg, B)
            demb, dmask, dnoise = to_dev(emb), to_dev(mask), to_dev(noise)
            a_pipe = torch.empty_like(dnoise)
            pipe.run(demb, dmask, dnoise, a_pipe, B, P)
            torch.cuda.synchronize()
            a_sep = torch.empty_like(dnoise)
            kv = pf.run(demb, dmask, B, P)
            pi_ae.sample_from_cache(ctx, kv, dnoise, a_sep, B)
            torch.cuda.synchronize()
            x = a_pipe.cpu().numpy()
            assert np.array_equal(x, a_sep.cpu().numpy())
            K, V = PO.prefill(w, cfg, emb, mask)
            ref = O.sample(ew, ecfg, inputs.f32_to_bf16_bits(K.astype(np.float32)),
                           inputs.f32_to_bf16_bits(V.astype(np.float32)), mask, noise)
            e, mx = rel_l2(x, ref), float(np.max(np.abs(x - ref)))
            log(f"[pipeline B={B} P={P}] rel_l2={e:.3e} max_abs={mx:.3e}")
            assert e <= TOL_REL_L2 and mx <= TOL_MAX_ABS
    finally:
        pipe.close()
        ctx.close()
        pf.close()


def test_holed_and_left_padded_prompts_then_loop():
    """Pads inside the prefix (a hole) and in front of it (left padding): every
    token sits at the count of valid tokens before it, the expert's suffix
    right after the valid ones.  The cache against the oracle prefill, then the
    loop on it against the oracle chain, then the same through the pipeline
    graph (bitwise equal to the separate calls)."""
    L = 2
    cfg = inputs.PrefillConfig(num_layers=L)
    ecfg = inputs.ExpertConfig(num_layers=L, num_steps=2, dt=-0.5)
    w = inputs.make_prefill_weights(cfg)
    ew = inputs.make_weights(ecfg)
    B, P = 2, 120
    mask = np.ones((B, P), np.uint8)
    mask[0, 40:60] = 0      # a hole in the middle
    mask[0, 110:] = 0       # and trailing pads
    mask[1, :30] = 0        # left padding
    emb = inputs.make_prefix_embeddings(cfg, B, P, seed=77)
    noise = inputs.make_noise(ecfg, B, seed=78)
    pf = pi_ae.Prefill(cfg, w, B, P)
    ctx = pi_ae.Context(ecfg, ew, B, P)
    pipe = pi_ae.Pipeline(pf, ctx)
    try:
        log("step: prefill with holed / left-padded masks")
        demb, dmask, dnoise = to_dev(emb), to_dev(mask), to_dev(noise)
        kv = pf.run(demb, dmask, B, P)
        torch.cuda.synchronize()
        k, v = cache_to_host(kv, L, B, P)
        K, V = PO.prefill(w, cfg, emb, mask)
        check_cache(k, v, K, V, "p-holed")
        a_sep = torch.empty_like(dnoise)
        pi_ae.sample_from_cache(ctx, kv, dnoise, a_sep, B)
        torch.cuda.synchronize()
        a_pipe = torch.empty_like(dnoise)
        pipe.run(demb, dmask, dnoise, a_pipe, B, P)
        torch.cuda.synchronize()
        x = a_sep.cpu().numpy()
        assert np.array_equal(x, a_pipe.cpu().numpy())
    finally:
        pipe.close()
        ctx.close()
        pf.close()
    ref = O.sample(ew, ecfg, inputs.f32_to_bf16_bits(K.astype(np.float32)),
                   inputs.f32_to_bf16_bits(V.astype(np.float32)), mask, noise)
    for b in range(B):
        e, mx = rel_l2(x[b], ref[b]), float(np.max(np.abs(x[b] - ref[b])))
        log(f"[prefill+loop holed b={b}] rel_l2={e:.3e} max_abs={mx:.3e}")
        assert e <= TOL_REL_L2 and mx <= TOL_MAX_ABS
