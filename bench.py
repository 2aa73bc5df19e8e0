#!/usr/bin/env python3
"""Throughput of block-wise cached decoding with confidence-aware parallel
unmasking on one MI355X.

A step is one whole decode of the workload (every block: cache refresh,
cached forwards, confidence scoring, selection, commit) through fdllm_decode,
starting from the same prompt with the generated positions masked. The
default workload is the LLaDA-8B-shaped random-init bf16 model (32 layers,
d 4096, 32 x 128 heads, SwiGLU 12288, vocab 126464) on a 512-token uniform
random prompt, gen_length 256, block 32, steps 256, PrefixCache, tau 0.9.

Prints one JSON line: generated tokens/s, the roofline of the dominant
kernel (achieved algorithmic bytes / launch time from hipEvents recorded on
the launch stream during the timed steps, against 8 TB/s HBM) and the CPU
oracle on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3
EVENT_STRIDE = 4  # timed decodes: events around every 4th launch of the dominant kernel


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    of this workload, or None when it is absent or the kernel sources
    changed since the counters were taken."""
    from block_wise_kv_amd.profiling import family, source_hash

    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    fam = family(kernel)
    if (t.get("source_hash") or {}).get(fam) != source_hash(fam):
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def roofline_of(prof: dict, workload: str, bf16: bool):
    """Roofline of the kernel variant with the largest total launch time:
    bound by MFMA when its algorithmic FLOPs per byte exceed the machine
    balance, else by HBM."""
    if not prof:
        return None
    kernel, (n, ms, nbytes, flops) = max(prof.items(), key=lambda kv: kv[1][1])
    peak_tf = MFMA_BF16_PEAK_TFLOPS if bf16 else MFMA_F32_PEAK_TFLOPS
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9)
    sec = ms * 1e-3
    tr = traffic_for(kernel, workload)
    common = {"kernel": kernel, "launches": n, "avg_launch_us": round(ms / n * 1e3, 2),
              "bytes_per_launch": round(nbytes / n), "flops_per_launch": round(flops / n),
              "traffic": tr, "share_of_kernel_time": round(ms / sum(v[1] for v in prof.values()), 4)}
    if flops / nbytes > ridge:
        achieved = flops / sec / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(achieved / peak_tf, 4), **common,
                "hbm_GBps": round(nbytes / sec / 1e9, 1)}
    achieved = nbytes / sec / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), **common,
            "mfma_TFLOPs": round(flops / sec / 1e12, 1)}


def cpu_baseline(wl, weights, nfe: int):
    """Times the oracle (float64, host cores) on one PrefixCache step of the
    final block and extrapolates NFE steps of that cost to tokens/s."""
    import numpy as np

    from block_wise_kv_amd import synth
    from oracle import decode as od
    from oracle import model as om

    shape, st = wl.model, wl.decode
    P, L, B = st.prompt_len, st.gen_length, st.block_size
    N = P + L
    m = om.Model(shape, weights)
    prompt = synth.make_prompt(shape, P, wl.seed_p)[0]
    x = np.concatenate([prompt.astype(np.int64), np.full(L, shape.mask_id)])
    flags = np.zeros(N, np.uint8)
    flags[N - B:] = 1
    # a stale cache of the right shape (its values do not change the work done)
    cache = [(np.zeros((N, shape.n_kv_heads, shape.head_dim)),
              np.zeros((N, shape.n_kv_heads, shape.head_dim))) for _ in range(shape.n_layers)]
    s = N - B
    r1 = s + B
    t0 = time.perf_counter()
    h, _ = m.forward_cached(x, s, r1, cache)
    z = m.logits(h[:B])
    c, a = od.confidence(z)
    if st.sampling:
        from oracle import sampling as smp
        smp.tau_leap_step(z, flags[s:s + B], s, 0, st.steps // (L // B), st.seed)
    else:
        od.select_rule(c, flags[s:s + B], st.threshold, 1, st.factor, st.topk)
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {
        "value": L / (dt * nfe), "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": (f"one PrefixCache step of the final block ({B} rows x {shape.n_layers} layers "
                   f"over a {N}-row cache, LM head over {shape.vocab} ids, selection) in float64 "
                   f"took {dt:.2f} s on {cores} host cores; value = gen_length / ({nfe} forwards "
                   f"x that time), the decode's forward count from the GPU run (refresh forwards, "
                   f"which cost the oracle more, are priced like this step)"),
    }


def step_bytes(shape, batch: int, block: int, kv_rows: int) -> int:
    """Algorithmic HBM bytes of one cached block step: every layer's
    weights, the LM head, the K/V of all kv_rows cache rows read and the
    fresh K/V of the block rows written (the norm gains are not counted)."""
    es = 2 if shape.dtype == "bf16" else 4
    d, qd, kvd, f = shape.d_model, shape.n_heads * shape.head_dim, shape.n_kv_heads * shape.head_dim, shape.ffn_dim
    layer_w = ((qd + 2 * kvd) * d + d * qd + 2 * f * d + f * d) * es
    kv_read = batch * kvd * kv_rows * es * 2
    kv_write = batch * block * kvd * es * 2
    return shape.n_layers * (layer_w + kv_read + kv_write) + shape.vocab * d * es


def step_roofline(F, torch, model, cache, x_final, wl, reps: int = 10):
    """One cached block step at the shape of the decode's last block (rows
    [N - B, N), the same rows for PrefixCache and DualCache), timed with
    events around the block forward and the fused LM head + selection only
    (ids and flags are restored outside the events before every call).
    Algorithmic bytes: every layer's weights, the LM head, the K/V of all N
    cache rows read and the fresh K/V of the block rows written."""
    shape, st = wl.model, wl.decode
    b, B = st.batch, st.block_size
    N = st.prompt_len + st.gen_length
    s = N - B
    d = shape.d_model
    nbytes = step_bytes(shape, b, B, N)
    x0 = x_final.clone()
    f0 = torch.zeros_like(x0, dtype=torch.uint8)
    f0[:, s:] = 1
    x, fl = x0.clone(), f0.clone()
    hidden = torch.empty(b * B * d, dtype=torch.float32, device="cuda")
    counts = torch.zeros(b, 2, dtype=torch.int32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps + 2)]
    for i in range(reps + 2):
        x.copy_(x0)
        fl.copy_(f0)
        ev[i][0].record()
        F.fdllm_block_forward(model.handle, cache.handle, x, b, N, s, N, s, B, hidden)
        F.fdllm_confidence_unmask(model.handle, cache.handle, hidden, x, fl, b, N, s, B, st.threshold, 0,
                                  st.steps // (st.gen_length // B), counts=counts)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(c) for a, c in ev[2:]) / reps  # the first two calls warm up
    floor_ms = nbytes / (HBM_PEAK_GBS * 1e9) * 1e3
    return {"rows": b * B, "kv_rows": N, "ms": round(ms, 4), "bytes": nbytes,
            "achieved_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "floor_ms": round(floor_ms, 4),
            "frac": round(floor_ms / ms, 4),
            "what": "one cached block step (block forward + LM head + selection) at the last block, "
                    "event-timed, against weights + LM head + K/V read + fresh K/V written at 8 TB/s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llada8b_prefix_gen256")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="do not time launches with events")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the decoding hot path on one GPU; runs on several GPUs are not part "
              "of this build (independent sequences would shard one per GPU with no exchange). "
              "Use --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from block_wise_kv_amd import fdllm as F
    from block_wise_kv_amd import synth
    from block_wise_kv_amd.runtime import GPUCache, GPUModel, decode_params

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    shape, st = wl.model, wl.decode
    P, L = st.prompt_len, st.gen_length
    N = P + L
    b = st.batch

    log(f"workload {wl.name}: {shape.n_params() / 1e9:.2f} B params, N={N}")
    t0 = time.time()
    weights = synth.make_weights(shape, wl.seed_w, threads=min(16, os.cpu_count() or 1))
    log(f"weights generated in {time.time() - t0:.1f} s")
    model = GPUModel(shape, weights, max_seq_len=N)
    cache = GPUCache(model, b, N)
    log("model packed and cache created on the GPU")
    prompt = synth.make_prompt(shape, P, wl.seed_p, batch=b)
    x0, f0 = synth.initial_sequence(shape, prompt, L)
    x0d = torch.from_numpy(x0).cuda()
    f0d = torch.from_numpy(f0).cuda()
    x = torch.empty_like(x0d)
    fl = torch.empty_like(f0d)
    params = decode_params(st)
    stream = torch.cuda.current_stream()

    def one_step():
        x.copy_(x0d)
        fl.copy_(f0d)
        return F.fdllm_decode(model.handle, cache.handle, x, fl, b, P, params)

    # The last warm-up decode is timed launch by launch (events around every
    # kernel) for the per-kernel breakdown and to find the dominant kernel;
    # the timed decodes then carry events only around every EVENT_STRIDE-th
    # launch of that kernel, which keeps their perturbation small.
    full = {}
    for i in range(args.warmup):
        last = i == args.warmup - 1 and not args.no_profile
        if last:
            F.fdllm_cache_profile_select(cache.handle, None, 1)
            F.fdllm_cache_profile_enable(cache.handle, True)
            F.fdllm_cache_profile_read(cache.handle, reset=True)
        s = one_step()
        if last:
            full = F.fdllm_cache_profile_read(cache.handle, reset=True)
            F.fdllm_cache_profile_enable(cache.handle, False)
        log(f"warmup {i}: nfe {s.nfe}")
    torch.cuda.synchronize()
    dominant = max(full.items(), key=lambda kv: kv[1][1])[0] if full else None
    if dominant:
        F.fdllm_cache_profile_select(cache.handle, dominant, EVENT_STRIDE)
        F.fdllm_cache_profile_enable(cache.handle, True)
        F.fdllm_cache_profile_read(cache.handle, reset=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    stats = []
    for i in range(args.steps):
        stats.append(one_step().as_dict(L // st.block_size))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    log(f"timed {args.steps} decodes in {elapsed:.3f} s; nfe {[s['nfe'] for s in stats]}")
    assert not fl.any().item(), "positions left masked"
    prof = F.fdllm_cache_profile_read(cache.handle) if dominant else {}
    F.fdllm_cache_profile_enable(cache.handle, False)
    F.fdllm_cache_profile_select(cache.handle, None, 1)
    del stream

    ms_per_step = elapsed / args.steps * 1e3
    value = b * L * args.steps / elapsed
    roofline = roofline_of(prof, wl.name, shape.dtype == "bf16")
    if roofline:
        roofline["sampled"] = f"every {EVENT_STRIDE}th launch of {dominant} in the timed decodes"
        roofline["share_of_kernel_time"] = round(full[dominant][1] / sum(v[1] for v in full.values()), 4)
    e2e = None
    if full:
        total_bytes = sum(v[2] for v in full.values())
        kernel_ms = sum(v[1] for v in full.values())
        floor_ms = total_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
        e2e = {"source": "last warm-up decode, every launch timed",
               "algorithmic_bytes_per_step": round(total_bytes),
               "bytes_floor_ms": round(floor_ms, 3), "frac_of_bytes_roofline": round(floor_ms / ms_per_step, 4),
               "kernel_busy_ms_per_step": round(kernel_ms, 3),
               "kernels": {k: {"launches": v[0], "ms": round(v[1], 3), "GBps": round(v[2] / (v[1] * 1e-3) / 1e9, 1),
                               "TFLOPs": round(v[3] / (v[1] * 1e-3) / 1e12, 1)}
                           for k, v in sorted(full.items(), key=lambda kv: -kv[1][1])}}

    step = step_roofline(F, torch, model, cache, x, wl) if not st.sampling else None
    if step:
        log(f"cached block step: {step['ms']} ms, {step['frac']} of the bytes roofline")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(wl, weights, int(np.mean([s["nfe"] for s in stats])))
        log(f"cpu baseline {cpu['value']:.4f} tokens/s")

    out = {
        "metric": "generated tokens/sec (LLaDA-8B-shape, gen 256/512) + % of HBM roofline",
        "value": round(value, 3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": b, "prompt_len": P, "gen_length": L,
                   "block_size": st.block_size,
                   "steps": st.steps, "cache": "dual" if st.dual_cache else ("prefix" if st.use_cache else "none"),
                   "threshold": st.threshold, "logit_scale": shape.logit_scale,
                   **({"selection": "tau-leaping sampling", "seed": st.seed} if st.sampling else
                      {"selection": "topk", "topk": st.topk} if st.topk > 0 else
                      {"selection": "factor", "factor": st.factor} if st.factor > 0 else
                      {"selection": "threshold"}),
                   **({"refresh_interval": st.refresh_interval} if st.refresh_interval > 0 else {})},
        "roofline": roofline, "cpu_baseline": cpu, "e2e": e2e, "block_step": step,
        "decode": {"nfe": stats[-1]["nfe"], "refreshes": stats[-1]["refreshes"],
                   "cached_steps": stats[-1]["cached_steps"], "steps_per_block": stats[-1]["steps_per_block"]},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
