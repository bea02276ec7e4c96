"""pi_ae_sample_noalloc (the allocation-free variant of pi_ae_sample) through
the C-ABI: two calls in a row on one context, the second with a smaller
input, each against pi_ae_sample on the same inputs (the same kernels in the
same order: bitwise equal) and against the oracle to the target's tolerance
(relative L2 <= 1e-2, max-abs <= 5e-2 on the final actions); and the limits,
checked on the host before anything is enqueued."""
import numpy as np
import pytest
import torch

from flow_matching_action_amd import inputs
from flow_matching_action_amd import pi_ae
from oracle import pi_ae_oracle as O

pytestmark = pytest.mark.gpu


def _dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _check(x, ref, noise, tag):
    e = float(np.linalg.norm(x - ref) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(x - ref)))
    d = float(np.linalg.norm((x - noise) - (ref - noise)) / np.linalg.norm(ref - noise))
    print(f"[{tag}] rel_l2={e:.3e} max_abs={mx:.3e} delta_rel_l2={d:.3e}", flush=True)
    assert np.all(np.isfinite(x)) and e <= 1e-2 and mx <= 5e-2 and d <= 2e-2


def test_noalloc_matches_sample_on_two_calls():
    assert torch.cuda.is_available()
    w = inputs.WORKLOADS["c2"]
    cfg = w.cfg
    wb = inputs.make_weights(cfg)
    ctx = pi_ae.Context(cfg, wb, 1, 256)
    try:
        for P, holes in ((256, False), (100, True)):
            print(f"step: noalloc call, 18 layers x 10 steps, prefix {P}", flush=True)
            k, v = inputs.make_prefix_kv(cfg, 1, P, seed=300 + P)
            mask = np.ones((1, P), np.uint8)
            if holes:
                mask[0, 20:35] = 0
                mask[0, 90:] = 0
            noise = inputs.make_noise(cfg, 1, seed=400 + P)
            dk, dv, dm, dn = _dev(k), _dev(v), _dev(mask), _dev(noise)
            a_ref = torch.empty_like(dn)
            ctx.sample(dk, dv, dm, dn, a_ref, 1, P)
            a_na = torch.full_like(dn, float("nan"))
            ctx.sample_noalloc(dk, dv, dm, dn, a_na, 1, P)
            torch.cuda.synchronize()
            x_ref, x = a_ref.cpu().numpy(), a_na.cpu().numpy()
            np.testing.assert_array_equal(x, x_ref)
            _check(x, O.sample(wb, cfg, k, v, mask, noise), noise, f"noalloc P={P}")
    finally:
        ctx.close()


def test_noalloc_limits_checked_before_enqueue():
    """Calls past the fixed array's limits return PI_AE_EINVAL before anything
    is enqueued: more than 64 rows, or more packed K/V than the array holds
    (4 layers x 258 key blocks x 16 KiB x 2 = 33 MiB > 24 MiB)."""
    cfg = inputs.WORKLOADS["c1"].cfg.replace(num_layers=4)
    wb = {n: np.zeros(sh, np.uint16) for n, sh in inputs.weight_shapes(cfg)}
    ctx = pi_ae.Context(cfg, wb, 2, 8192)
    try:
        x = torch.zeros(2 * cfg.chunk_len * 32, device="cuda")
        kv = torch.zeros(cfg.num_layers * 2 * 8192 * 256, dtype=torch.int16, device="cuda")
        with pytest.raises(pi_ae.PiAeError) as e:
            ctx.sample_noalloc(kv, kv, None, x, x, 2, 16)          # 2 x 63 = 126 rows
        assert e.value.status == pi_ae.PI_AE_EINVAL and "64" in str(e.value)
        with pytest.raises(pi_ae.PiAeError) as e:
            ctx.sample_noalloc(kv, kv, None, x, x, 1, 8192)
        assert e.value.status == pi_ae.PI_AE_EINVAL and "fixed array" in str(e.value)
        torch.cuda.synchronize()
        assert torch.all(x == 0)                                    # nothing ran
    finally:
        ctx.close()
