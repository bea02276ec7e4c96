"""Parity of the HIP path (through the C-ABI) with the CPU oracle.

Bar (per the target of this path): on the final actions, relative L2 error
<= 1e-2 and max-abs error <= 5e-2 against the fp64 oracle, on the same
seeded inputs; the relative L2 error of the integrated displacement
(x_final - x_0) is checked too (<= 2e-2), because x_final is dominated by
the noise that both sides share.  Intermediates of one step are compared
phase by phase: each is stored in bf16 (a relative rounding of at most 2^-9
per element) from bf16 operands, so the relative L2 error is about 1.6e-3
(two such roundings in quadrature) and the largest element error a few times
that in units of the tensor's RMS; the bars are relative L2 <= 5e-3 and,
element by element, |error| <= 2.5e-2 x RMS(reference) + 2^-6 x |reference|
(an absolute part for elements near zero, whose error is the propagated
rounding of their inputs, and four bf16 units relative for the large ones),
which an error confined to one head, row tile or column tile would exceed.  Invariances that hold exactly for this
implementation (no atomics, row-independent GEMM tiles) are checked bitwise.
"""
import time

import numpy as np
import pytest
import torch

from flow_matching_action_amd import inputs
from flow_matching_action_amd import pi_ae
from oracle import pi_ae_oracle as O

pytestmark = pytest.mark.gpu

TOL_REL_L2 = 1e-2
TOL_MAX_ABS = 5e-2
TOL_DELTA_REL_L2 = 2e-2


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


class Run:
    """Device copies of one workload's call inputs."""

    def __init__(self, k, v, mask, noise):
        self.k, self.v, self.mask, self.noise = k, v, mask, noise
        self.dk, self.dv = to_dev(k), to_dev(v)
        self.dmask = to_dev(mask)
        self.dnoise = to_dev(noise)
        self.B, self.P = noise.shape[0], (k.shape[2] if k is not None else 0)

    def sample(self, ctx, stream=None, actions=None):
        out = actions if actions is not None else torch.empty_like(self.dnoise)
        ctx.sample(self.dk, self.dv, self.dmask, self.dnoise, out, self.B, self.P, stream)
        torch.cuda.synchronize()
        return out.cpu().numpy()


TOL_PROBE_REL_L2 = 5e-3
TOL_PROBE_ABS_RMS = 2.5e-2
TOL_PROBE_REL = 2.0 ** -6


def check_probe(name, got, ref):
    """One phase's intermediate against the oracle's: relative L2, and every
    element within 2.5e-2 RMS + 2^-6 of its own magnitude (the worst ratio of
    error to that bound is logged)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    e = rel_l2(got, ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    worst = float(np.max(err / (TOL_PROBE_ABS_RMS * rms + TOL_PROBE_REL * np.abs(ref))))
    log(f"  {name}: rel_l2={e:.3e} max_abs/rms={float(np.max(err)) / max(rms, 1e-30):.3e} "
        f"worst element / bound={worst:.3f}")
    assert np.all(np.isfinite(got)), name
    assert e <= TOL_PROBE_REL_L2 and worst <= 1.0, (name, e, worst)


def check_actions(x_gpu, x_ref, noise, tag):
    e = rel_l2(x_gpu, x_ref)
    mx = float(np.max(np.abs(x_gpu - x_ref)))
    d = rel_l2(x_gpu - noise, x_ref - noise)
    log(f"[{tag}] rel_l2={e:.3e} max_abs={mx:.3e} delta_rel_l2={d:.3e}")
    assert np.all(np.isfinite(x_gpu))
    assert e <= TOL_REL_L2 and mx <= TOL_MAX_ABS and d <= TOL_DELTA_REL_L2, (e, mx, d)


# ------------------------------------------------------------------ per-phase (c1)
def oracle_step0_intermediates(wb, cfg, k, v, mask, noise):
    """Layer-0 intermediates of step 0 for episode 0, from the oracle's pieces."""
    W = O.Weights(wb, cfg)
    t = O.timesteps(cfg.num_steps, cfg.t0, cfg.dt)[0]
    cond = O.time_condition(W, t)
    x = noise[0].astype(np.float64)
    h0 = x @ W["action_in.w"].T + W["action_in.b"]
    pk, pv = O.bf16_to_float(k[0, 0]), O.bf16_to_float(v[0, 0])
    valid = mask[0] != 0
    T, H, d = cfg.chunk_len, cfg.num_heads, cfg.head_dim
    pos = valid.sum() + np.arange(T)
    s, sh, g = O.modulation(W.layer(0, "attn_mod.w"), W.layer(0, "attn_mod.b"), cond)
    u = O.adarms(h0, s, sh, cfg.rms_eps)
    q = O.rope((u @ W.layer(0, "q.w").T).reshape(T, H, d).transpose(1, 0, 2), pos, cfg.rope_base).transpose(1, 0, 2)
    ks = O.rope(u @ W.layer(0, "k.w").T, pos, cfg.rope_base)
    vs = u @ W.layer(0, "v.w").T
    keys, vals = np.concatenate([pk, ks]), np.concatenate([pv, vs])
    o = O.attention(q, keys, vals, np.concatenate([valid, np.ones(T, bool)]), d ** -0.5).reshape(T, H * d)
    h1 = h0 + (o @ W.layer(0, "o.w").T) * g
    s2, sh2, g2 = O.modulation(W.layer(0, "ffn_mod.w"), W.layer(0, "ffn_mod.b"), cond)
    u2 = O.adarms(h1, s2, sh2, cfg.rms_eps)
    m = O.gelu_tanh(u2 @ W.layer(0, "gate.w").T) * (u2 @ W.layer(0, "up.w").T)
    h2 = h1 + (m @ W.layer(0, "down.w").T) * g2
    return dict(h0=h0, q=q, ks=ks, vs=vs, o=o, h1=h1, m=m, h2=h2)


# c1, and c1 with the 816-key prefix of c4 (16 padded): the latter is long
# enough for the attention to split each query's keys over two workgroups
C1_VARIANTS = {"c1": inputs.WORKLOADS["c1"],
               "c1-long": inputs.WORKLOADS["c1"].replace(name="c1-long", prefix_len=816, n_valid=800)}


@pytest.fixture(scope="module", params=list(C1_VARIANTS))
def c1_setup(request):
    w = C1_VARIANTS[request.param]
    wb, k, v, mask, noise = inputs.make_workload_inputs(w)
    ctx = pi_ae.Context(w.cfg, wb, w.batch, w.prefix_len)
    return w, wb, Run(k, v, mask, noise), ctx


def test_prepared_tables_match_host(c1_setup):
    w, wb, run, ctx = c1_setup
    S, L = w.cfg.num_steps, w.cfg.num_layers
    for which, n in [(0, S * L * 1024), (6, S * L * 2560), (7, S * L * 8192), (5, S * 32)]:
        np.testing.assert_array_equal(ctx.table(which, n), pi_ae.host_table(w.cfg, wb, which, n))


def test_c1_phase_by_phase(c1_setup):
    w, wb, run, ctx = c1_setup
    ref = oracle_step0_intermediates(wb, w.cfg, run.k, run.v, run.mask, run.noise)
    bf = lambda a: O.bf16_to_float(a)

    def probe(phase, which):
        log(f"probe phase={phase} which={which}")
        return ctx.probe(run.dk, run.dv, run.dmask, run.dnoise, 1, run.P, 0, 0, phase, which)

    h0 = probe(0, 0)
    assert rel_l2(h0, ref["h0"]) < 1e-5
    q = bf(probe(1, 1))
    ks = bf(probe(1, 2))
    vs = bf(probe(1, 3))
    for name, got in [("q", q), ("ks", ks), ("vs", vs)]:
        check_probe(name, got, ref[name])
    # per head as well: an error confined to one head must not hide in the whole
    for hd in range(8):
        check_probe(f"q head {hd}", q[:, hd], ref["q"][:, hd])
    M, nkb = w.cfg.chunk_len, (run.P + w.cfg.chunk_len + 31) // 32
    if M < 129 and nkb >= 16:
        # the keys of every query are split into two ranges: merge the two
        # normalised partial outputs by their (max, sum) as documented for
        # the probe, then compare with the oracle's attention output
        o0, o1, st = bf(probe(2, 4)), bf(probe(2, 7)), probe(2, 8).astype(np.float64)
        m0, l0, m1, l1 = st[..., 0], st[..., 1], st[..., 2], st[..., 3]
        assert np.all(l0 > 0) and np.all(l1 > 0), "both key ranges hold valid keys"
        mx = np.maximum(m0, m1)
        a0 = np.where(m0 == -np.inf, 0.0, np.exp2(m0 - mx)) * l0
        a1 = np.where(m1 == -np.inf, 0.0, np.exp2(m1 - mx)) * l1
        w0, w1 = (a0 / (a0 + a1))[..., None], (a1 / (a0 + a1))[..., None]
        o = (o0.reshape(M, 8, 256) * w0 + o1.reshape(M, 8, 256) * w1).reshape(M, 2048)
        tag = "o (two key ranges merged)"
    else:
        o, tag = bf(probe(2, 4)), "o"
    check_probe(tag, o, ref["o"])
    for hd in range(8):
        check_probe(f"o head {hd}", o[:, hd * 256:(hd + 1) * 256], ref["o"][:, hd * 256:(hd + 1) * 256])
    h1 = probe(3, 0)
    check_probe("h1-h0", h1 - h0, ref["h1"] - ref["h0"])
    m = bf(probe(4, 5))
    check_probe("m", m, ref["m"])
    h2 = probe(5, 0)
    check_probe("h2-h1", h2 - h1, ref["h2"] - ref["h1"])


def test_c1_end_to_end(c1_setup):
    w, wb, run, ctx = c1_setup
    x_ref = O.sample(wb, w.cfg, run.k, run.v, run.mask, run.noise)
    check_actions(run.sample(ctx), x_ref, run.noise, "c1")


# ------------------------------------------------------------------ full configs
@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c2pi0"])
def test_batch1_configs(name):
    w = inputs.WORKLOADS[name]
    wb, k, v, mask, noise = inputs.make_workload_inputs(w)
    log(f"[{name}] preparing")
    ctx = pi_ae.Context(w.cfg, wb, w.batch, w.prefix_len)
    run = Run(k, v, mask, noise)
    x = run.sample(ctx)
    t0 = time.time()
    x_ref = O.sample(wb, w.cfg, k, v, mask, noise)
    log(f"[{name}] oracle {time.time() - t0:.1f}s")
    check_actions(x, x_ref, noise, name)
    ctx.close()


@pytest.fixture(scope="module")
def c5_run():
    """The 32 episodes of c5 in one call (run once; the tests below check them
    against the oracle eight at a time)."""
    w = inputs.WORKLOADS["c5"]
    wb, k, v, mask, noise = inputs.make_workload_inputs(w)
    log("[c5] preparing")
    ctx = pi_ae.Context(w.cfg, wb, w.batch, w.prefix_len)
    x = Run(k, v, mask, noise).sample(ctx)
    ctx.close()
    assert np.all(np.isfinite(x))
    return w, wb, k, v, mask, noise, x, O.Weights(wb, w.cfg)


@pytest.mark.parametrize("group", range(4))
def test_c5_every_episode(c5_run, group):
    """All 32 episodes of the batched call, each against the oracle run on that
    episode alone (episodes are independent, so that is the exact reference)."""
    w, wb, k, v, mask, noise, x, W = c5_run
    for b in range(8 * group, 8 * group + 8):
        t0 = time.time()
        x_ref = O.sample(wb, w.cfg, k[:, b:b + 1], v[:, b:b + 1], mask[b:b + 1], noise[b:b + 1], weights=W)
        log(f"[c5] episode {b} oracle {time.time() - t0:.1f}s")
        check_actions(x[b:b + 1], x_ref, noise[b:b + 1], f"c5[{b}]")


# ------------------------------------------------------------------ edge cases
SMALL = inputs.ExpertConfig(num_layers=2, num_steps=2, dt=-0.5)


@pytest.fixture(scope="module")
def small_ctx():
    wb = inputs.make_weights(SMALL, seed=5, cache=False)
    return wb, pi_ae.Context(SMALL, wb, max_batch=4, max_prefix_len=96)


def test_ragged_masks_and_batch(small_ctx):
    """Per-episode masks with holes, different valid counts, and no prefix at all."""
    wb, ctx = small_ctx
    B, P = 3, 70
    k, v = inputs.make_prefix_kv(SMALL, B, P, seed=7)
    rng = np.random.default_rng(8)
    mask = (rng.random((B, P)) < 0.7).astype(np.uint8)
    mask[2] = 0  # an episode with every prefix key masked
    noise = inputs.make_noise(SMALL, B, seed=9)
    x = Run(k, v, mask, noise).sample(ctx)
    x_ref = O.sample(wb, SMALL, k, v, mask, noise)
    check_actions(x, x_ref, noise, "ragged")
    # no prefix: P = 0, NULL k/v
    k0 = np.zeros((SMALL.num_layers, 2, 0, 256), np.uint16)
    noise2 = noise[:2].copy()
    run0 = Run(None, None, None, noise2)
    out = torch.empty_like(run0.dnoise)
    ctx.sample(None, None, None, run0.dnoise, out, 2, 0)
    torch.cuda.synchronize()
    check_actions(out.cpu().numpy(), O.sample(wb, SMALL, k0, k0, None, noise2), noise2, "no-prefix")


def test_many_episodes_ragged_masks():
    """Nine episodes (288 query blocks of 16 rows): the attention kernel that
    shares each K/V block through LDS across the waves of a workgroup, with
    ragged masks (holes, a fully masked prefix), masked garbage, and the
    tiled GEMMs; every episode against the oracle."""
    wb = inputs.make_weights(SMALL, seed=5, cache=False)
    ctx = pi_ae.Context(SMALL, wb, max_batch=9, max_prefix_len=100)
    B, P = 9, 100
    k, v = inputs.make_prefix_kv(SMALL, B, P, seed=21)
    rng = np.random.default_rng(22)
    mask = (rng.random((B, P)) < 0.6).astype(np.uint8)
    mask[3] = 0
    mask[5, :] = 1
    noise = inputs.make_noise(SMALL, B, seed=23)
    x = Run(k, v, mask, noise).sample(ctx)
    x_ref = O.sample(wb, SMALL, k, v, mask, noise)
    for b in range(B):
        check_actions(x[b:b + 1], x_ref[b:b + 1], noise[b:b + 1], f"many[{b}]")
    k2, v2 = k.copy(), v.copy()
    k2[:, mask == 0] = inputs.f32_to_bf16_bits(np.array([3e4], np.float32))[0]
    v2[:, mask == 0] = np.uint16(0x7FC0)  # NaN
    np.testing.assert_array_equal(Run(k2, v2, mask, noise).sample(ctx), x)
    # an odd number of 32-key blocks (70 prefix + 63 suffix keys: 5 blocks)
    P2 = 70
    k3, v3 = np.ascontiguousarray(k[:, :, :P2]), np.ascontiguousarray(v[:, :, :P2])
    mask3 = np.ascontiguousarray(mask[:, :P2])
    x3 = Run(k3, v3, mask3, noise).sample(ctx)
    x3_ref = O.sample(wb, SMALL, k3, v3, mask3, noise)
    for b in (0, 3, 8):
        check_actions(x3[b:b + 1], x3_ref[b:b + 1], noise[b:b + 1], f"many-odd[{b}]")
    ctx.close()


def test_masked_garbage_batch_independence_and_repeatability(small_ctx):
    """Exact invariances.  Up to 128 rows (2 episodes here) the weight-streaming
    GEMMs run; above that the tiled GEMMs, whose K accumulation order differs,
    so bitwise comparisons stay within one path and the two paths are compared
    to the oracle's tolerance."""
    wb, ctx = small_ctx
    B, P = 4, 96
    k, v = inputs.make_prefix_kv(SMALL, B, P, seed=10)
    mask = inputs.make_pad_mask(B, P, [96, 80, 33, 1])
    noise = inputs.make_noise(SMALL, B, seed=11)
    base = Run(k, v, mask, noise).sample(ctx)  # 252 rows: tiled path
    # garbage (huge values, NaN) in masked prefix positions changes nothing
    k2, v2 = k.copy(), v.copy()
    k2[:, mask == 0] = inputs.f32_to_bf16_bits(np.array([3e4], np.float32))[0]
    v2[:, mask == 0] = np.uint16(0x7FC0)  # NaN
    np.testing.assert_array_equal(Run(k2, v2, mask, noise).sample(ctx), base)
    # permuting the episodes permutes the outputs (rows are independent)
    perm = np.array([2, 0, 3, 1])
    out = Run(np.ascontiguousarray(k[:, perm]), np.ascontiguousarray(v[:, perm]), mask[perm].copy(),
              noise[perm].copy()).sample(ctx)
    np.testing.assert_array_equal(out, base[perm])
    # weight-streaming path: a pair of episodes equals each episode alone
    pair = Run(np.ascontiguousarray(k[:, 1:3]), np.ascontiguousarray(v[:, 1:3]), mask[1:3].copy(),
               noise[1:3].copy()).sample(ctx)
    for i, b in enumerate([1, 2]):
        alone = Run(np.ascontiguousarray(k[:, b:b + 1]), np.ascontiguousarray(v[:, b:b + 1]),
                    mask[b:b + 1].copy(), noise[b:b + 1].copy()).sample(ctx)
        np.testing.assert_array_equal(alone, pair[i:i + 1])
        # and the tiled path agrees with it to the oracle tolerance
        check_actions(base[b:b + 1], alone.astype(np.float64), noise[b:b + 1], f"tiled-vs-streaming[{b}]")
    # graph replays with eager work in between are bitwise repeatable
    run = Run(k, v, mask, noise)
    for _ in range(3):
        torch.randn(1 << 20, device="cuda").sum().item()
        np.testing.assert_array_equal(run.sample(ctx), base)


def test_in_place_zero_batch_and_errors(small_ctx):
    wb, ctx = small_ctx
    B, P = 2, 40
    k, v = inputs.make_prefix_kv(SMALL, B, P, seed=12)
    noise = inputs.make_noise(SMALL, B, seed=13)
    run = Run(k, v, None, noise)
    ref = run.sample(ctx)
    buf = run.dnoise.clone()
    ctx.sample(run.dk, run.dv, None, buf, buf, B, P)  # actions aliases noise
    torch.cuda.synchronize()
    np.testing.assert_array_equal(buf.cpu().numpy(), ref)
    ctx.sample(run.dk, run.dv, None, run.dnoise, run.dnoise, 0, P)  # batch 0: nothing happens
    # limits the library checks (buffers large enough for the binding's own checks)
    L, T = SMALL.num_layers, SMALL.chunk_len
    big_kv = torch.zeros(L * 5 * 97 * 256, dtype=torch.int16, device="cuda")
    big_x = torch.zeros(5 * T * 32, dtype=torch.float32, device="cuda")
    with pytest.raises(pi_ae.PiAeError) as e:
        ctx.sample(big_kv, big_kv, None, big_x, big_x, 5, P)
    assert e.value.status == pi_ae.PI_AE_EINVAL
    with pytest.raises(pi_ae.PiAeError):
        ctx.sample(big_kv, big_kv, None, big_x, big_x, B, 97)
    # what the binding refuses before the call: not contiguous, too small, wrong dtype, host memory
    with pytest.raises(ValueError):
        ctx.sample(run.dk, run.dv, None, run.dnoise[:, :, 1:], buf, B, P)
    with pytest.raises(ValueError):
        ctx.sample(run.dk, run.dv, None, run.dnoise[:1], buf, B, P)
    with pytest.raises(TypeError):
        ctx.sample(run.dk.float(), run.dv, None, run.dnoise, buf, B, P)
    with pytest.raises(ValueError):
        ctx.sample(run.dk, run.dv, None, run.dnoise.cpu(), buf, B, P)
    mis = torch.empty(run.dnoise.numel() + 1, device="cuda")[1:]
    with pytest.raises(pi_ae.PiAeError) as e:
        ctx.sample(run.dk, run.dv, None, run.dnoise, mis, B, P)
    assert "aligned" in str(e.value)


# ------------------------------------------------------------------ pi0 variant
def test_pi0_step_input_and_end_to_end():
    """pi0 (action-time encoder, RMS norm scales): the step input h of step 0
    (the encoder's folded input layer, SiLU, output layer) against the
    oracle's unfolded encoder, then the whole reduced loop."""
    w = inputs.WORKLOADS["c1pi0"]
    wb, k, v, mask, noise = inputs.make_workload_inputs(w)
    ctx = pi_ae.Context(w.cfg, wb, w.batch, w.prefix_len)
    run = Run(k, v, mask, noise)
    h0 = ctx.probe(run.dk, run.dv, run.dmask, run.dnoise, 1, run.P, 0, 0, 0, 0)
    W = O.Weights(wb, w.cfg)
    t = O.timesteps(w.cfg.num_steps, w.cfg.t0, w.cfg.dt)[0]
    ref = O.encoder_pi0(W, noise[0].astype(np.float64), t)
    e = rel_l2(h0, ref)
    log(f"[c1pi0] step input h: rel_l2={e:.3e}")
    assert e < 2e-2
    check_actions(run.sample(ctx), O.sample(wb, w.cfg, k, v, mask, noise), noise, "c1pi0")
    ctx.close()


def test_pi0_many_rows_tiled_path():
    """pi0 with enough rows (3 episodes x 63 = 189) for the tiled GEMMs and the
    tiled encoder output layer; ragged masks; every episode against the oracle."""
    cfg = inputs.WORKLOADS["c1pi0"].cfg
    B, P = 3, 100
    wb = inputs.make_weights(cfg)
    k, v = inputs.make_prefix_kv(cfg, B, P, seed=7)
    mask = inputs.make_pad_mask(B, P, [100, 57, 3])
    noise = inputs.make_noise(cfg, B, seed=8)
    ctx = pi_ae.Context(cfg, wb, B, P)
    x = Run(k, v, mask, noise).sample(ctx)
    ref = O.sample(wb, cfg, k, v, mask, noise)
    for b in range(B):
        check_actions(x[b], ref[b], noise[b], f"pi0-tiled[{b}]")
    ctx.close()


# ------------------------------------------------------------------ every shape the ABI accepts
def _ragged_case(cfg, B, P, seed):
    k, v = inputs.make_prefix_kv(cfg, B, P, seed=seed)
    rng = np.random.default_rng(seed + 1)
    mask = (rng.random((B, P)) < 0.8).astype(np.uint8) if P else None
    noise = inputs.make_noise(cfg, B, seed=seed + 2)
    return k, v, mask, noise


@pytest.mark.parametrize("B,T", [(1, 1), (1, 64), (1, 65), (1, 128), (1, 129), (1, 256), (2, 64), (3, 1)])
def test_chunk_lengths(B, T):
    """Chunk lengths across the ABI's range [1, 256], on both sides of the
    switch from the weight-streaming GEMMs (up to 128 rows) to the tiled ones
    (129 rows on), at batch 1 and above; 2 layers, 2 steps, holed masks."""
    cfg = SMALL.replace(chunk_len=T)
    wb = inputs.make_weights(cfg, seed=31, cache=False)
    P = 100
    ctx = pi_ae.Context(cfg, wb, max_batch=B, max_prefix_len=P)
    k, v, mask, noise = _ragged_case(cfg, B, P, seed=40 + T)
    x = Run(k, v, mask, noise).sample(ctx)
    x_ref = O.sample(wb, cfg, k, v, mask, noise)
    for b in range(B):
        check_actions(x[b:b + 1], x_ref[b:b + 1], noise[b:b + 1], f"T={T} B={B} [{b}]")
    ctx.close()


def test_without_final_norm():
    """final_norm = 0: action_out_proj reads the residual stream directly."""
    w = inputs.WORKLOADS["c1"]
    cfg = w.cfg.replace(final_norm=False)
    wb, k, v, mask, noise = inputs.make_workload_inputs(w)
    ctx = pi_ae.Context(cfg, wb, w.batch, w.prefix_len)
    x = Run(k, v, mask, noise).sample(ctx)
    check_actions(x, O.sample(wb, cfg, k, v, mask, noise), noise, "c1 final_norm=0")
    ctx.close()


def test_longest_prefixes():
    """Prefixes of 4096 and of the ABI's maximum 8192 keys (batch 1, 2 layers,
    1 step), with pads in the middle of the prefix."""
    cfg = inputs.WORKLOADS["c1"].cfg
    wb = inputs.make_weights(cfg)
    ctx = pi_ae.Context(cfg, wb, 1, 8192)
    for P in (4096, 8192):
        k, v = inputs.make_prefix_kv(cfg, 1, P, seed=P)
        mask = np.ones((1, P), np.uint8)
        mask[0, P // 3:P // 3 + 100] = 0
        noise = inputs.make_noise(cfg, 1, seed=P + 1)
        x = Run(k, v, mask, noise).sample(ctx)
        check_actions(x, O.sample(wb, cfg, k, v, mask, noise), noise, f"P={P}")
    ctx.close()


def test_largest_batch():
    """The ABI's largest call: 1024 episodes x 64 actions (65536 rows per GEMM),
    2 layers, 1 step.  Eight distinct episodes are repeated over the batch:
    each of the eight against the oracle, and every repeat bitwise equal to
    its first occurrence (episodes are independent and every row takes the
    same arithmetic)."""
    cfg = SMALL.replace(chunk_len=64, num_steps=1, dt=-1.0)
    wb = inputs.make_weights(cfg, seed=51, cache=False)
    B, P, U = 1024, 40, 8
    ctx = pi_ae.Context(cfg, wb, max_batch=B, max_prefix_len=P)
    k8, v8, mask8, noise8 = _ragged_case(cfg, U, P, seed=60)
    rep = np.arange(B) % U
    k, v = np.ascontiguousarray(k8[:, rep]), np.ascontiguousarray(v8[:, rep])
    x = Run(k, v, np.ascontiguousarray(mask8[rep]), np.ascontiguousarray(noise8[rep])).sample(ctx)
    ctx.close()
    x_ref = O.sample(wb, cfg, k8, v8, mask8, noise8)
    for b in range(U):
        check_actions(x[b:b + 1], x_ref[b:b + 1], noise8[b:b + 1], f"B=1024 [{b}]")
    np.testing.assert_array_equal(x, x[rep])
