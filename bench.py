"""Benchmark of the action-expert denoise loop on one MI355X.

One bench step = one pi_ae_sample call: the whole 10-step flow-matching loop of
the 18-layer expert over one batch (inputs resident in HBM).  Prints ONE JSON
line.  Default workload: c5, the largest configuration of the loop that fits
one GPU (32 episodes x 50 actions, 712 prefix keys each: the MFMA-bound
regime), with the batch-1 configuration c2 (1 camera view, 256 prefix keys,
chunk 63: the weight-streaming regime) timed in the same run and reported in
the nested "batch1" block.

  python bench.py [--steps K] [--warmup W] [--workload c1..c5|c1pi0|c2pi0] [--no-cpu] [--no-batch1]

Reported beside the throughput:
  * "roofline": the kernel with the largest share of the loop's kernel time
    (durations timed live inside the loop with a HIP event pair bound to each
    launch of that kernel), against the roof its own arithmetic intensity puts
    it under (HBM for intensity below the ridge of 2.5 PFLOP/s / 8 TB/s, bf16
    MFMA above); "traffic" = its HBM bytes per launch from the rocprofv3
    FETCH_SIZE / WRITE_SIZE counters committed under profiles/, when they were
    taken on the current kernel source;
  * "whole_loop_roofline_frac" and "roofline_by_kernel" (every kernel, both
    roofs, its share of the kernel time);
  * "floors": a plain streaming read, the per-kernel boundary of a replayed
    graph of empty kernels and a grid-wide barrier inside one kernel, measured
    by the library's diagnostics in the same run;
  * "cpu_baseline": the CPU oracle timed on this host on a bounded sample.

Other workloads: p1 / p2 / p3 time the VLM prefix prefill (one step = one
pi_ae_vlm_prefill call: 17 full Gemma-2B-shaped layers and the last layer's K/V
over 256 / 512 / 816 prefix tokens), reported as prefix tokens/s; s1 / s3 the
vision encoder alone (1 / 3 views -> 256 tokens each), views/s; f1 / f2 / f3
one whole inference at the shapes of the pages' Table 1 (1 / 2 / 3 views,
empty prompt, a 63-action chunk, 10 steps: pi_ae_inference_run, the vision
encoder, the prefill and the loop as one graph); e1 / e2 / e3 the prefill of 1
/ 2 / 3 views followed by the 10-step loop (pi_ae_pipeline_run, one graph),
inferences/s.

Counter summaries: `--pmc-summary` turns the CSV output of rocprofv3 counter
runs (FETCH_SIZE, WRITE_SIZE over whole sample calls, and over the plain copy
of `--calibrate-copy`) into profiles/hbm_counters_<workload>.json, which the
default run reads for "traffic".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA

# bf16 weight bytes streamed per launch of each phase's kernel (one layer)
PHASE_WEIGHT_BYTES = {1: 2560 * 1024 * 2, 3: 1024 * 2048 * 2, 4: 8192 * 1024 * 2, 5: 1024 * 4096 * 2}
PHASE_NAMES = {0: "k_io", 1: "k_gemm<qkv>", 2: "k_attn", 3: "k_gemm<o>", 4: "k_gemm<gate_up>", 5: "k_gemm<down>"}
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "flow_matching_action_amd", "csrc", "pi_ae_kernels.hip")


def algorithmic_bytes_per_step(w) -> float:
    """Weights streamed once per Euler step + each valid prefix K/V once per layer."""
    cfg = w.cfg
    per_layer = sum(PHASE_WEIGHT_BYTES.values())
    io = 2 * 32 * 1024 * 2
    if getattr(cfg, "variant", 0) == 1:  # pi0: the action-time encoder's output layer
        io += 1024 * 1024 * 2
    kv = cfg.num_layers * w.batch * w.n_valid * 256 * 2 * 2
    return cfg.num_layers * per_layer + io + kv


def algorithmic_flops_per_step(w) -> float:
    cfg = w.cfg
    M = w.batch * cfg.chunk_len
    gemm = 2 * M * (1024 * 2560 + 2048 * 1024 + 1024 * 8192 + 4096 * 1024) * cfg.num_layers
    gemm += 2 * M * (32 * 1024 * 2)
    if getattr(cfg, "variant", 0) == 1:
        gemm += 2 * M * 1024 * 1024
    attn = 4 * 8 * cfg.chunk_len * (w.n_valid + cfg.chunk_len) * 256 * w.batch * cfg.num_layers
    return gemm + attn


# VLM prefill: per-launch algorithmic bytes (bf16 weights) and flops per row
VLM_PHASE_NAMES = {1: "k_gemm<vlm qkv>", 2: "k_attn<vlm>", 3: "k_gemm<vlm o>", 4: "k_gemm<vlm gate_up>",
                   5: "k_gemm<vlm down>"}
VLM_PHASE_NK = {1: (2560, 2048), 3: (2048, 2048), 4: (32768, 2048), 5: (2048, 16384)}  # (N, K) per layer


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def host_blas():
    """(threads the BLAS pool uses, a description of the BLAS library)."""
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        desc = "; ".join(f"{i.get('internal_api', '?')} {i.get('version', '?')} ({i.get('threading_layer', '?')}, "
                         f"{i.get('num_threads', '?')} threads)" for i in info)
        return int(threads), desc
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1, "unknown"


def cpu_baseline(w, wb, k, v, mask, noise, target_s: float = 12.0, max_chunks: int = 5):
    """The CPU oracle (fp32 mode) on a bounded sample: whole chunks of episode 0.
    Episodes are independent and the oracle runs them one after another, so
    its rate over the whole workload is that of one episode."""
    import numpy as np
    from oracle import pi_ae_oracle as O
    threads, blas = host_blas()
    W = O.Weights(wb, w.cfg, np.float32)
    args = (k[:, :1], v[:, :1], mask[:1], noise[:1])
    times = []
    t_start = time.time()
    while True:
        t0 = time.time()
        O.sample(wb, w.cfg, *args, dtype=np.float32, weights=W)
        times.append(time.time() - t0)
        if time.time() - t_start >= target_s or len(times) >= max_chunks:
            break
    per_chunk = statistics.median(times)
    return {"value": round(w.cfg.num_steps / per_chunk, 3), "unit": "denoise steps/s", "cores": int(threads),
            "kind": "oracle", "blas": blas, "affinity_cores": len(os.sched_getaffinity(0)),
            "sample": f"{len(times)} full {w.cfg.num_steps}-step chunk(s) of episode 0 of this workload "
                      f"(T={w.cfg.chunk_len}, {w.n_valid} prefix keys), NumPy fp32, median "
                      f"{per_chunk * 1e3:.0f} ms/chunk; episodes run one after another, so this is also "
                      f"its rate over all {w.batch} episode(s)"}


COPY_BYTES = 256 << 20  # fp32 source read once and destination written once per launch


def calibrate_copy(torch):
    """A plain elementwise copy (dst = src * 1) of COPY_BYTES each way, 3 launches:
    the reference that scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy": True, "read_bytes": COPY_BYTES, "write_bytes": COPY_BYTES, "launches": 3}),
          flush=True)


def prefill_cpu_baseline(w, wb, emb, mask, target_layers: int = 2):
    """The prefill oracle (fp32) on a bounded sample: the first two layers of
    episode 0, scaled to the whole prefill (17 full layers + the last K/V)."""
    import numpy as np
    from oracle import prefill_oracle as PO
    threads, blas = host_blas()
    cfg = w.cfg
    t0 = time.time()
    PO.prefill(wb, cfg, emb[:1], mask[:1], dtype=np.float32, layers=target_layers)
    per_layer = (time.time() - t0) / target_layers
    full = per_layer * (cfg.num_layers - 1) + per_layer * 0.05  # the last layer's K/V: ~5% of a layer's MACs
    return {"value": round(w.prefix_len / full, 1), "unit": "prefix tokens/s", "cores": int(threads),
            "kind": "oracle", "blas": blas, "affinity_cores": len(os.sched_getaffinity(0)),
            "sample": f"layers 0-{target_layers - 1} of episode 0 (NumPy fp32), {per_layer * 1e3:.0f} ms per layer, "
                      f"scaled to {cfg.num_layers - 1} full layers + the last layer's K/V"}


def bench_prefill(args, np, torch):
    from flow_matching_action_amd import inputs, pi_ae
    w = inputs.PREFILL_WORKLOADS[args.workload]
    cfg, B, P = w.cfg, w.batch, w.prefix_len
    print(f"bench: workload {w.name}: {w.description}", file=sys.stderr, flush=True)
    wb = inputs.make_prefill_weights(cfg)
    emb = inputs.make_prefix_embeddings(cfg, B, P)
    mask = inputs.make_pad_mask(B, P, w.n_valid)
    pf = pi_ae.Prefill(cfg, wb, B, P)
    dev = torch.device("cuda:0")
    de = torch.from_numpy(emb.view(np.int16)).to(dev)
    dm = torch.from_numpy(mask).to(dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        pf.run(de, dm, B, P, stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        pf.run(de, dm, B, P, stream)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms_per_step = wall * 1e3 / args.steps
    median_us = statistics.median(per_call_ms) * 1e3
    p99_us = float(np.percentile(per_call_ms, 99)) * 1e3
    print(f"bench: {ms_per_step * 1e3:.1f} us/prefill (median {median_us:.1f}, p99 {p99_us:.1f})",
          file=sys.stderr, flush=True)
    phase_us = {ph: pf.time_phase(de, dm, B, P, ph, args.kernel_chunks, stream) for ph in range(1, 6)}
    print("bench: per-launch us " + ", ".join(f"{VLM_PHASE_NAMES[p]}={t:.2f}" for p, t in phase_us.items()),
          file=sys.stderr, flush=True)
    L, M = cfg.num_layers, B * P
    nv = w.n_valid
    alg_bytes = {ph: n * k * 2 for ph, (n, k) in VLM_PHASE_NK.items()}
    alg_flops = {ph: 2 * M * n * k for ph, (n, k) in VLM_PHASE_NK.items()}
    alg_bytes[2] = B * nv * 256 * 2 * 2
    alg_flops[2] = 4 * 8 * P * nv * 256 * B
    launches = {1: L, 2: L - 1, 3: L - 1, 4: L - 1, 5: L - 1}
    # whole prefill: 17 full layers + the last layer's K/V columns (512 of 2560)
    bytes_call = sum(alg_bytes[ph] * (L - 1) for ph in (1, 2, 3, 4, 5)) + 512 * 2048 * 2
    flops_call = sum(alg_flops[ph] * (L - 1) for ph in (1, 2, 3, 4, 5)) + 2 * M * 512 * 2048
    call_s = ms_per_step * 1e-3
    t_hbm, t_mfma = bytes_call / (HBM_PEAK_GBS * 1e9), flops_call / (MFMA_BF16_PEAK_TFS * 1e12)
    dom = 4
    sec = phase_us[dom] * 1e-6
    if alg_flops[dom] / (MFMA_BF16_PEAK_TFS * 1e12) >= alg_bytes[dom] / (HBM_PEAK_GBS * 1e9):
        a = alg_flops[dom] / sec / 1e12
        roof = {"kernel": VLM_PHASE_NAMES[dom], "bound": "mfma", "achieved": round(a, 1), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(a / MFMA_BF16_PEAK_TFS, 4), "traffic": None}
    else:
        a = alg_bytes[dom] / sec / 1e9
        roof = {"kernel": VLM_PHASE_NAMES[dom], "bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4), "traffic": None}
    by_kernel = {}
    for ph in range(1, 6):
        sec = phase_us[ph] * 1e-6
        gbs, tfs = alg_bytes[ph] / sec / 1e9, alg_flops[ph] / sec / 1e12
        by_kernel[VLM_PHASE_NAMES[ph]] = {
            "us": round(phase_us[ph], 3), "alg_bytes": alg_bytes[ph], "GB/s": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "alg_flops": alg_flops[ph], "TFLOP/s": round(tfs, 2),
            "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
            "time_share": round(phase_us[ph] * launches[ph] / (ms_per_step * 1e3), 4)}
    cpu = None if args.no_cpu else prefill_cpu_baseline(w, wb, emb, mask)
    pf.close()
    line = {
        "metric": "VLM prefix prefill: prefix tokens/s (18-layer Gemma-2B-shaped VLM filling the expert's KV cache)",
        "value": round(B * P / call_s, 1),
        "unit": "prefix tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "batch": B, "prefix_len": P, "valid_prefix": nv,
                   "layers": L},
        "us_per_prefill": {"mean": round(ms_per_step * 1e3, 1), "median": round(median_us, 1),
                           "p99": round(p99_us, 1)},
        "whole_prefill_roofline": {"hbm_us": round(t_hbm * 1e6, 1), "mfma_us": round(t_mfma * 1e6, 1),
                                   "frac": round(max(t_hbm, t_mfma) / call_s, 4)},
        "per_launch_us": {VLM_PHASE_NAMES[p]: round(t, 3) for p, t in phase_us.items()},
        "roofline": roof,
        "roofline_by_kernel": by_kernel,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


PIPELINES = {"e1": ("p1", "c2"), "e2": ("p2", "c3"), "e3": ("p3", "c4")}

# vision encoder: per-launch algorithmic flops (unpadded shapes) and bf16 weight bytes per view of 256 tokens
VIS_PHASE_NAMES = {0: "k_gemm<vis patch>", 1: "k_vis_ln", 2: "k_gemm<vis qkv>", 3: "k_vis_attn",
                   4: "k_gemm<vis o>+k_vis_res_ln", 5: "k_gemm<vis fc1>", 6: "k_gemm<vis fc2>+k_vis_res_ln",
                   7: "k_gemm<vis proj>"}
VIS_NK = {0: (1152, 588), 2: (3456, 1152), 4: (1152, 1152), 5: (4304, 1152), 6: (1152, 4304), 7: (2048, 1152)}


def _timed_calls(run, torch, stream, steps, warmup):
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        run()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return wall * 1e3 / steps, statistics.median(per), max(per)


def bench_vision(args, np, torch):
    from flow_matching_action_amd import inputs, pi_ae
    V = {"s1": 1, "s3": 3}[args.workload]
    cfg = inputs.VisionConfig()
    print(f"bench: vision encoder, {V} view(s) of 224x224 -> {256 * V} tokens", file=sys.stderr, flush=True)
    vis = pi_ae.Vision(cfg, inputs.make_vision_weights(cfg), V)
    dev = torch.device("cuda:0")
    imgs = torch.from_numpy(inputs.make_images(cfg, V).view(np.int16)).to(dev)
    tok = torch.empty(V * 256 * 2048, dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    ms, med, mx = _timed_calls(lambda: vis.encode(imgs, V, tok, stream), torch, stream, args.steps, args.warmup)
    print(f"bench: {ms * 1e3:.1f} us/encode (median {med * 1e3:.1f})", file=sys.stderr, flush=True)
    phase_us = {ph: vis.time_phase(imgs, V, tok, ph, args.kernel_chunks, stream) for ph in range(8)}
    print("bench: per-launch us " + ", ".join(f"{VIS_PHASE_NAMES[p]}={t:.2f}" for p, t in phase_us.items()),
          file=sys.stderr, flush=True)
    vis.close()
    M, L = 256 * V, cfg.num_layers
    flops = {ph: 2 * M * n * k for ph, (n, k) in VIS_NK.items()}
    flops[3] = 4 * cfg.num_heads * 256 * 256 * cfg.head_dim * V
    wbytes = {ph: n * k * 2 for ph, (n, k) in VIS_NK.items()}
    per_call = flops[0] + flops[7] + L * (flops[2] + flops[3] + flops[4] + flops[5] + flops[6])
    bytes_call = wbytes[0] + wbytes[7] + L * (wbytes[2] + wbytes[4] + wbytes[5] + wbytes[6])
    dom = 5
    a = flops[dom] / (phase_us[dom] * 1e-6) / 1e12
    roof = {"kernel": VIS_PHASE_NAMES[dom], "bound": "mfma", "achieved": round(a, 1), "peak": MFMA_BF16_PEAK_TFS,
            "unit": "TFLOP/s", "frac": round(a / MFMA_BF16_PEAK_TFS, 4), "traffic": None}
    t_mfma, t_hbm = per_call / (MFMA_BF16_PEAK_TFS * 1e12), bytes_call / (HBM_PEAK_GBS * 1e9)
    line = {
        "metric": "vision encoder: views/s (27-layer SigLIP-shaped, 224x224 -> 256 tokens per view)",
        "value": round(V / (ms * 1e-3), 1), "unit": "views/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: {V} view(s), 27 layers, width 1152, 16 heads x 72, MLP 4304",
                   "views": V},
        "us_per_encode": {"mean": round(ms * 1e3, 1), "median": round(med * 1e3, 1)},
        "whole_encode_roofline": {"hbm_us": round(t_hbm * 1e6, 1), "mfma_us": round(t_mfma * 1e6, 1),
                                  "frac": round(max(t_hbm, t_mfma) / (ms * 1e-3), 4)},
        "per_launch_us": {VIS_PHASE_NAMES[p]: round(t, 3) for p, t in phase_us.items()},
        "roofline": roof, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_full(args, np, torch):
    """Table 1 shapes: V views (256 tokens each), empty prompt, chunk 63, 10 steps."""
    from flow_matching_action_amd import inputs, pi_ae
    V = {"f1": 1, "f2": 2, "f3": 3}[args.workload]
    P = 256 * V
    vcfg, pcfg, ecfg = inputs.VisionConfig(), inputs.PrefillConfig(), inputs.ExpertConfig()
    print(f"bench: full inference, {V} view(s), empty prompt, chunk 63, 10 steps", file=sys.stderr, flush=True)
    vis = pi_ae.Vision(vcfg, inputs.make_vision_weights(vcfg), V)
    pf = pi_ae.Prefill(pcfg, inputs.make_prefill_weights(pcfg), 1, P)
    ctx = pi_ae.Context(ecfg, inputs.make_weights(ecfg), 1, P)
    inf = pi_ae.Inference(vis, pf, ctx)
    dev = torch.device("cuda:0")
    imgs = torch.from_numpy(inputs.make_images(vcfg, V).view(np.int16)).to(dev)
    dn = torch.from_numpy(inputs.make_noise(ecfg, 1)).to(dev)
    out = torch.empty_like(dn)
    stream = torch.cuda.current_stream()

    def run():
        inf.run(imgs, V, None, 0, None, dn, out, stream)

    ms, med, mx = _timed_calls(run, torch, stream, args.steps, args.warmup)
    print(f"bench: {ms * 1e3:.1f} us/inference (median {med * 1e3:.1f})", file=sys.stderr, flush=True)
    inf.close()
    ctx.close()
    pf.close()
    vis.close()
    line = {
        "metric": "inferences/s (vision encoder + VLM prefix prefill + 10-step denoise loop, one graph)",
        "value": round(1 / (ms * 1e-3), 2), "unit": "inferences/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: {V} view(s) x 256 tokens, empty prompt, chunk 63 x 32, 10 steps",
                   "views": V, "prefix_len": P, "chunk_len": ecfg.chunk_len, "euler_steps": ecfg.num_steps},
        "ms_per_inference": {"mean": round(ms, 3), "median": round(med, 3)},
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_pipeline(args, np, torch):
    from flow_matching_action_amd import inputs, pi_ae
    pw = inputs.PREFILL_WORKLOADS[PIPELINES[args.workload][0]]
    ew = inputs.WORKLOADS[PIPELINES[args.workload][1]]
    B, P = pw.batch, pw.prefix_len
    print(f"bench: pipeline {args.workload}: {pw.description}, then {ew.description}", file=sys.stderr, flush=True)
    pf = pi_ae.Prefill(pw.cfg, inputs.make_prefill_weights(pw.cfg), B, P)
    ctx = pi_ae.Context(ew.cfg, inputs.make_weights(ew.cfg), B, P)
    pipe = pi_ae.Pipeline(pf, ctx)
    dev = torch.device("cuda:0")
    de = torch.from_numpy(inputs.make_prefix_embeddings(pw.cfg, B, P).view(np.int16)).to(dev)
    dm = torch.from_numpy(inputs.make_pad_mask(B, P, pw.n_valid)).to(dev)
    dn = torch.from_numpy(inputs.make_noise(ew.cfg, B)).to(dev)
    out = torch.empty_like(dn)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        pipe.run(de, dm, dn, out, B, P, stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        pipe.run(de, dm, dn, out, B, P, stream)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = wall * 1e3 / args.steps
    med, p99 = statistics.median(per_call_ms), float(np.percentile(per_call_ms, 99))
    print(f"bench: {ms * 1e3:.1f} us/inference (median {med * 1e3:.1f}, p99 {p99 * 1e3:.1f})", file=sys.stderr, flush=True)
    pipe.close()
    ctx.close()
    pf.close()
    line = {
        "metric": "inferences/s (VLM prefix prefill + 10-step denoise loop, one graph; no vision encoder)",
        "value": round(B / (ms * 1e-3), 2), "unit": "inferences/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: {pw.description}; then {ew.description}", "batch": B,
                   "prefix_len": P, "valid_prefix": pw.n_valid, "chunk_len": ew.cfg.chunk_len,
                   "vlm_layers": pw.cfg.num_layers, "expert_layers": ew.cfg.num_layers,
                   "euler_steps": ew.cfg.num_steps},
        "ms_per_inference": {"mean": round(ms, 3), "median": round(med, 3), "p99": round(p99, 3)},
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def expert_kernel_table(w, phase_us, us_per_chunk):
    """Every phase kernel of the loop against both roofs.

    Algorithmic work per launch: the bf16 weights it streams (attention: the
    valid prefix K/V) and 2 M N K flops of its GEMM (attention: 4 H T (P_v + T)
    d per episode).  A kernel's roof is the one its intensity puts it under.
    The event pair bound to each timed launch reads about 1 us more than the
    dispatch itself, so the shares are those of the summed event times
    (normalised to 1), and the per-launch overhead this implies is reported."""
    cfg = w.cfg
    M = w.batch * cfg.chunk_len
    launches = {0: cfg.num_steps + 1, **{ph: cfg.num_steps * cfg.num_layers for ph in range(1, 6)}}
    alg_bytes = dict(PHASE_WEIGHT_BYTES)
    alg_bytes[0] = 2 * 32 * 1024 * 2
    alg_bytes[2] = w.batch * w.n_valid * 256 * 2 * 2
    alg_flops = {0: 2 * M * 32 * 1024 * 2, 1: 2 * M * 1024 * 2560, 3: 2 * M * 2048 * 1024, 4: 2 * M * 1024 * 8192,
                 5: 2 * M * 4096 * 1024, 2: 4 * 8 * cfg.chunk_len * (w.n_valid + cfg.chunk_len) * 256 * w.batch}
    total = sum(phase_us[ph] * launches[ph] for ph in range(6))
    n_launch = sum(launches.values())
    rows = {}
    for ph in range(6):
        sec = phase_us[ph] * 1e-6
        gbs, tfs = alg_bytes[ph] / sec / 1e9, alg_flops[ph] / sec / 1e12
        mfma_bound = alg_flops[ph] / (MFMA_BF16_PEAK_TFS * 1e12) >= alg_bytes[ph] / (HBM_PEAK_GBS * 1e9)
        rows[PHASE_NAMES[ph]] = {
            "us": round(phase_us[ph], 3), "launches_per_chunk": launches[ph],
            "alg_bytes": alg_bytes[ph], "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "alg_flops": alg_flops[ph], "TFLOP/s": round(tfs, 2), "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
            "bound": "mfma" if mfma_bound else "hbm",
            "share": round(phase_us[ph] * launches[ph] / total, 4)}
    overhead = (total - us_per_chunk) / n_launch
    return rows, round(overhead, 3)


def load_counters(workload: str):
    path = os.path.join(PROFILES, f"hbm_counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    return c if c.get("kernel_source_sha256_16") == kernel_source_hash() else None


def expert_roofline(w, rows):
    """The roofline object for the kernel with the largest share."""
    name = max(rows, key=lambda n: rows[n]["share"])
    r = rows[name]
    if r["bound"] == "mfma":
        roof = {"kernel": name, "bound": "mfma", "achieved": r["TFLOP/s"], "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": r["mfma_frac"]}
    else:
        roof = {"kernel": name, "bound": "hbm", "achieved": r["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": r["hbm_frac"]}
    counters = load_counters(w.name)
    roof["traffic"] = None
    if counters and name in counters.get("kernels", {}):
        roof["traffic"] = counters["kernels"][name]["hbm_bytes_per_launch"]
    roof["share"] = r["share"]
    return roof, counters


def run_expert(args, np, torch, w, cpu_s: float, phase_timing: bool = True):
    """Time one expert workload; returns the fields of its bench line."""
    from flow_matching_action_amd import inputs, pi_ae
    cfg = w.cfg
    wb, k, v, mask, noise = inputs.make_workload_inputs(w)
    print(f"bench: workload {w.name}: {w.description}", file=sys.stderr, flush=True)
    ctx = pi_ae.Context(cfg, wb, w.batch, w.prefix_len)
    dev = torch.device("cuda:0")
    dk = torch.from_numpy(k.view(np.int16)).to(dev)
    dv = torch.from_numpy(v.view(np.int16)).to(dev)
    dm = torch.from_numpy(mask).to(dev)
    dn = torch.from_numpy(noise).to(dev)
    out = torch.empty_like(dn)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        ctx.sample(dk, dv, dm, dn, out, w.batch, w.prefix_len, stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        ctx.sample(dk, dv, dm, dn, out, w.batch, w.prefix_len, stream)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms_per_step = wall * 1e3 / args.steps
    median_us = statistics.median(per_call_ms) * 1e3
    p99_us = float(np.percentile(per_call_ms, 99)) * 1e3
    print(f"bench: {w.name}: {ms_per_step * 1e3:.1f} us/chunk (median {median_us:.1f}, p99 {p99_us:.1f})",
          file=sys.stderr, flush=True)
    res = {"ms_per_step": round(ms_per_step, 4),
           "value": round(cfg.num_steps * w.batch / (ms_per_step * 1e-3), 1),
           "config": {"workload": f"{w.name}: {w.description}", "batch": w.batch, "chunk_len": cfg.chunk_len,
                      "prefix_len": w.prefix_len, "valid_prefix": w.n_valid, "layers": cfg.num_layers,
                      "euler_steps": cfg.num_steps},
           "us_per_chunk": {"mean": round(ms_per_step * 1e3, 1), "median": round(median_us, 1),
                            "p99": round(p99_us, 1)}}
    chunk_s = ms_per_step * 1e-3
    if w.batch * cfg.chunk_len < 129:
        res["whole_loop_roofline"] = {"bound": "hbm", "alg_bytes_per_chunk": algorithmic_bytes_per_step(w) * cfg.num_steps,
                                      "frac": round(algorithmic_bytes_per_step(w) * cfg.num_steps / chunk_s /
                                                    (HBM_PEAK_GBS * 1e9), 4)}
    else:
        res["whole_loop_roofline"] = {"bound": "mfma", "alg_flops_per_chunk": algorithmic_flops_per_step(w) * cfg.num_steps,
                                      "frac": round(algorithmic_flops_per_step(w) * cfg.num_steps / chunk_s /
                                                    (MFMA_BF16_PEAK_TFS * 1e12), 4)}
    res["whole_loop_roofline_frac"] = res["whole_loop_roofline"]["frac"]
    if phase_timing:
        phase_us = {ph: ctx.time_phase(dk, dv, dm, dn, out, w.batch, w.prefix_len, ph, args.kernel_chunks, stream)
                    for ph in range(6)}
        print("bench: per-launch us " + ", ".join(f"{PHASE_NAMES[p]}={t:.2f}" for p, t in phase_us.items()),
              file=sys.stderr, flush=True)
        rows, overhead = expert_kernel_table(w, phase_us, ms_per_step * 1e3)
        roof, counters = expert_roofline(w, rows)
        res["roofline"] = roof
        res["roofline_by_kernel"] = rows
        res["event_timing_overhead_us_per_launch"] = overhead
        if counters:
            res["hbm_traffic_per_chunk"] = counters.get("chunk")
    ctx.close()
    if cpu_s > 0:
        res["cpu_baseline"] = cpu_baseline(w, wb, k, v, mask, noise, target_s=cpu_s)
    else:
        res["cpu_baseline"] = None
    return res


def machine_floors(pi_ae, stream, chunk_kernels: int):
    """The floors under the batch-1 design, measured on this GPU now."""
    read = pi_ae.stream_read_gbps(2 << 30, 5, stream)
    boundary = pi_ae.graph_floor_us(200, 256, stream)
    flags = pi_ae.grid_sync_us(2000, 0, stream)
    counters = pi_ae.grid_sync_us(2000, 1, stream)
    return {"stream_read_GBps": round(read, 1),
            "graph_boundary_us_per_kernel": round(boundary, 3),
            "grid_sync_us_per_round": {"flags": round(flags, 3), "xcd_counters": round(counters, 3)},
            "kernels_per_chunk": chunk_kernels,
            "boundary_floor_us_per_chunk": round(boundary * chunk_kernels, 1)}


def pmc_summary(args):
    """profiles/hbm_counters_<workload>.json from rocprofv3 counter CSVs: per
    kernel the mean HBM bytes per dispatch, and the bytes of one whole sample
    call (every dispatch of the run divided by the number of calls), each
    counter scaled by what it reads for the plain copy of --calibrate-copy."""
    import csv
    import glob

    def rows(d, counter):
        out = []
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") == counter:
                        out.append((int(r.get("Dispatch_Id", len(out))), r["Kernel_Name"], float(r["Counter_Value"])))
        if not out:
            raise SystemExit(f"no {counter} rows under {d}")
        out.sort()
        # O and down projections share one kernel at many rows: every layer
        # dispatches O first, so alternate occurrences of that kernel are O, down
        named, seen = [], {}
        for _, kname, v in out:
            n = phase_name(kname)
            if n == "k_gemm<o|down>":
                i = seen.get(n, 0)
                seen[n] = i + 1
                n = "k_gemm<o>" if i % 2 == 0 else "k_gemm<down>"
            named.append((n, v))
        return named

    def phase_name(kname):
        for short in ("k_io", "k_pack", "k_args"):
            if kname.startswith("pi_ae::" + short):
                return short
        if "k_attn" in kname:
            return "k_attn"
        if "k_gemm_sq" in kname or "k_gemm_wide" in kname or "k_gemm<4, 2, 4, 8, 1," in kname:
            return "k_gemm<gate_up>"
        if any(t in kname for t in ("k_gemm_big32<4, 1, 2, 0,", "k_gemm<2, 2, 4, 8, 0,", "k_gemm<4, 2, 4, 8, 0,")):
            return "k_gemm<qkv>"
        if "k_gemm<1, 1, 8, 8, 2," in kname or "k_gemm<4, 1, 8, 8, 2," in kname:
            return "k_gemm<o>"
        if "k_gemm<1, 1, 8, 16, 2," in kname or "k_gemm<4, 1, 8, 16, 2," in kname:
            return "k_gemm<down>"
        if "k_gemm_big32<4, 1, 2, 2," in kname:
            return "k_gemm<o|down>"
        return kname

    fetch, write = rows(args.pmc_fetch, "FETCH_SIZE"), rows(args.pmc_write, "WRITE_SIZE")
    cf = [v for n, v in rows(args.pmc_copy_fetch, "FETCH_SIZE") if "elementwise" in n]
    cw = [v for n, v in rows(args.pmc_copy_write, "WRITE_SIZE") if "elementwise" in n]
    if not cf or not cw:
        raise SystemExit("no elementwise copy dispatches in the calibration runs")
    kib = COPY_BYTES / 1024
    f_fac, w_fac = kib / statistics.median(cf), kib / statistics.median(cw)
    calls = args.steps + args.warmup
    per = {}
    for which, data, fac in (("read", fetch, f_fac), ("write", write, w_fac)):
        for name, v in data:
            per.setdefault(name, {}).setdefault(which, []).append(v * 1024 * fac)
    kernels = {}
    for n, d in per.items():
        r = statistics.mean(d.get("read", [0.0]))
        wr = statistics.mean(d.get("write", [0.0]))
        kernels[n] = {"dispatches": len(d.get("read", [])), "hbm_read_bytes_per_launch": int(r),
                      "hbm_write_bytes_per_launch": int(wr), "hbm_bytes_per_launch": int(r + wr)}
    read_total = sum(v * 1024 * f_fac for _, v in fetch) / calls
    write_total = sum(v * 1024 * w_fac for _, v in write) / calls
    from flow_matching_action_amd import inputs
    w = inputs.WORKLOADS[args.workload]
    alg = algorithmic_bytes_per_step(w) * w.cfg.num_steps
    out = {"workload": args.workload, "kernel_source_sha256_16": kernel_source_hash(),
           "sample_calls": calls, "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4),
           "kernels": kernels,
           "chunk": {"hbm_read_bytes": int(read_total), "hbm_write_bytes": int(write_total),
                     "hbm_bytes": int(read_total + write_total), "algorithmic_bytes": int(alg),
                     "ratio_to_algorithmic": round((read_total + write_total) / alg, 3)}}
    path = os.path.join(PROFILES, f"hbm_counters_{args.workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c5",
                    choices=["c1", "c2", "c3", "c4", "c5", "c1pi0", "c2pi0", "p1", "p2", "p3", "e1", "e2", "e3",
                             "s1", "s3", "f1", "f2", "f3"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-batch1", action="store_true", help="c5 only: skip the nested batch-1 (c2) block")
    ap.add_argument("--no-floors", action="store_true", help="skip the machine floors")
    ap.add_argument("--only-sample", action="store_true",
                    help="only the timed sample calls (no per-kernel passes, no CPU, no floors): for counter runs")
    ap.add_argument("--kernel-chunks", type=int, default=2,
                    help="whole loop passes over which each kernel's in-loop duration is averaged")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain elementwise copy of known size (HBM counter calibration)")
    ap.add_argument("--pmc-summary", action="store_true",
                    help="write profiles/hbm_counters_<workload>.json from rocprofv3 counter CSV directories")
    ap.add_argument("--pmc-fetch")
    ap.add_argument("--pmc-write")
    ap.add_argument("--pmc-copy-fetch")
    ap.add_argument("--pmc-copy-write")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: every path here runs on exactly one GPU (there is no multi-GPU path); --gpus must be 1",
              file=sys.stderr)
        sys.exit(2)
    if args.pmc_summary:
        pmc_summary(args)
        return

    import numpy as np
    import torch

    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    if args.workload.startswith("p"):
        bench_prefill(args, np, torch)
        return
    if args.workload.startswith("e"):
        bench_pipeline(args, np, torch)
        return
    if args.workload.startswith("s"):
        bench_vision(args, np, torch)
        return
    if args.workload.startswith("f"):
        bench_full(args, np, torch)
        return

    from flow_matching_action_amd import inputs, pi_ae

    w = inputs.WORKLOADS[args.workload]
    quick = args.only_sample
    main_res = run_expert(args, np, torch, w, cpu_s=0 if (args.no_cpu or quick) else 12.0, phase_timing=not quick)
    line = {
        "metric": "denoise steps/s (10-step action chunk, 18-layer expert); us per chunk; roofline fraction",
        "value": main_res["value"],
        "unit": "denoise steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": main_res["config"],
    }
    for key in ("us_per_chunk", "whole_loop_roofline_frac", "whole_loop_roofline", "roofline", "roofline_by_kernel",
                "event_timing_overhead_us_per_launch", "hbm_traffic_per_chunk"):
        if key in main_res:
            line[key] = main_res[key]
    if w.name == "c5" and not (args.no_batch1 or quick):
        b1 = run_expert(args, np, torch, inputs.WORKLOADS["c2"], cpu_s=0 if args.no_cpu else 4.0)
        line["batch1"] = {k: b1[k] for k in ("value", "ms_per_step", "config", "us_per_chunk", "whole_loop_roofline",
                                              "roofline", "roofline_by_kernel", "event_timing_overhead_us_per_launch",
                                              "cpu_baseline") if k in b1}
        if "hbm_traffic_per_chunk" in b1:
            line["batch1"]["hbm_traffic_per_chunk"] = b1["hbm_traffic_per_chunk"]
        line["batch1"]["unit"] = "denoise steps/s"
    if not (args.no_floors or quick):
        L, S = w.cfg.num_layers, w.cfg.num_steps
        line["floors"] = machine_floors(pi_ae, torch.cuda.current_stream(), 1 + S * (1 + 5 * L) + 1)
    line["cpu_baseline"] = main_res["cpu_baseline"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
