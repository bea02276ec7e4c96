"""Robustness of the library objects on the GPU: the guard bytes around every
device allocation are intact after calls of every shape class (and the check
sees a changed guard), and an allocation that fails at any point of a
preparation (PI_AE_FAIL_ALLOC=N) returns PI_AE_ENOMEM and frees everything
allocated before it."""
import os

import numpy as np
import pytest
import torch

from flow_matching_action_amd import inputs
from flow_matching_action_amd import pi_ae

pytestmark = pytest.mark.gpu


def _dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


SMALL = inputs.ExpertConfig(num_layers=2, num_steps=2, dt=-0.5)


def test_guards_intact_after_calls():
    assert torch.cuda.is_available()
    wb = inputs.make_weights(SMALL, seed=5, cache=False)
    ctx = pi_ae.Context(SMALL, wb, max_batch=4, max_prefix_len=96)
    try:
        for B, P in ((1, 96), (2, 40), (4, 96), (3, 0)):   # streaming and tiled GEMMs, the key split, no prefix
            print(f"step: expert B={B} P={P}", flush=True)
            k, v = inputs.make_prefix_kv(SMALL, B, P, seed=B + P)
            mask = (np.random.default_rng(P).random((B, P)) < 0.7).astype(np.uint8) if P else None
            noise = _dev(inputs.make_noise(SMALL, B, seed=B))
            out = torch.empty_like(noise)
            ctx.sample(_dev(k) if P else None, _dev(v) if P else None, _dev(mask), noise, out, B, P)
        torch.cuda.synchronize()
        assert pi_ae.check_guards(ctx) == -1
        with pytest.raises(pi_ae.PiAeError) as e:
            pi_ae.check_guards(ctx, corrupt=3)
        assert e.value.status == pi_ae.PI_AE_ESTATE and "allocation 3" in str(e.value)
    finally:
        ctx.close()
    pcfg = inputs.PrefillConfig(num_layers=2)
    pf = pi_ae.Prefill(pcfg, inputs.make_prefill_weights(pcfg), 2, 40)
    try:
        print("step: prefill B=2 P=40", flush=True)
        emb = _dev(inputs.make_prefix_embeddings(pcfg, 2, 40))
        pf.run(emb, _dev(inputs.make_pad_mask(2, 40, [40, 31])), 2, 40)
        torch.cuda.synchronize()
        assert pi_ae.check_guards(pf) == -1
    finally:
        pf.close()
    vcfg = inputs.VisionConfig(num_layers=1)
    vis = pi_ae.Vision(vcfg, inputs.make_vision_weights(vcfg), 2)
    try:
        print("step: vision 2 views", flush=True)
        tok = torch.empty(2 * 256 * 2048, dtype=torch.int16, device="cuda")
        vis.encode(_dev(inputs.make_images(vcfg, 2)), 2, tok)
        torch.cuda.synchronize()
        assert pi_ae.check_guards(vis) == -1
    finally:
        vis.close()


@pytest.mark.parametrize("kind", ["expert", "prefill", "vision"])
def test_every_failed_allocation_frees_what_came_before(kind):
    """PI_AE_FAIL_ALLOC=n for n = 1, 2, ... until the preparation succeeds: each
    failure returns PI_AE_ENOMEM, and the device bytes the library holds (its
    own exact count: the device-wide free memory moves by tens of MB between
    identical attempts as the HIP runtime caches and returns memory) are back
    where they were before the attempt."""
    if kind == "expert":
        cfg, w = SMALL, inputs.make_weights(SMALL, seed=5, cache=False)
        make = lambda: pi_ae.Context(cfg, w, 2, 64)
    elif kind == "prefill":
        cfg = inputs.PrefillConfig(num_layers=2)
        w = inputs.make_prefill_weights(cfg)
        make = lambda: pi_ae.Prefill(cfg, w, 1, 64)
    else:
        cfg = inputs.VisionConfig(num_layers=1)
        w = inputs.make_vision_weights(cfg)
        make = lambda: pi_ae.Vision(cfg, w, 1)
    held = pi_ae.live_device_bytes()
    obj = make()
    assert pi_ae.live_device_bytes() > held
    obj.close()
    assert pi_ae.live_device_bytes() == held
    try:
        for n in range(1, 200):
            os.environ["PI_AE_FAIL_ALLOC"] = str(n)
            try:
                obj = make()
            except pi_ae.PiAeError as e:
                assert e.status == pi_ae.PI_AE_ENOMEM and "injected" in str(e), str(e)
                assert pi_ae.live_device_bytes() == held, (n, pi_ae.live_device_bytes() - held)
                continue
            obj.close()  # n is past the last allocation: preparation succeeded
            print(f"[{kind}] each of the {n - 1} allocation failures returned ENOMEM and freed everything",
                  flush=True)
            assert n > 5
            break
        else:
            raise AssertionError("preparation never succeeded")
    finally:
        os.environ.pop("PI_AE_FAIL_ALLOC", None)
    assert pi_ae.live_device_bytes() == held
