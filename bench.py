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
the launch stream during the timed steps, against 8 TB/s HBM), the whole
decode against the bytes-only and the combined max(bytes, FLOPs) roofline
and against a streaming-read kernel measured in the same run, and the CPU
oracle on a bounded sample (plus the tiny workload end to end on both).

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
    balance, else by HBM. frac_combined is the sum over its launches of
    max(bytes / HBM peak, FLOPs / MFMA peak) over their summed time."""
    if not prof:
        return None
    kernel, (n, ms, nbytes, flops, floor_ms) = max(prof.items(), key=lambda kv: kv[1][1])
    peak_tf = MFMA_BF16_PEAK_TFLOPS if bf16 else MFMA_F32_PEAK_TFLOPS
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9)
    sec = ms * 1e-3
    tr = traffic_for(kernel, workload)
    common = {"kernel": kernel, "launches": n, "avg_launch_us": round(ms / n * 1e3, 2),
              "bytes_per_launch": round(nbytes / n), "flops_per_launch": round(flops / n),
              "traffic": tr, "share_of_kernel_time": round(ms / sum(v[1] for v in prof.values()), 4),
              "frac_combined": round(floor_ms / ms, 4)}
    if flops / nbytes > ridge:
        achieved = flops / sec / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(achieved / peak_tf, 4), **common,
                "hbm_GBps": round(nbytes / sec / 1e9, 1)}
    achieved = nbytes / sec / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), **common,
            "mfma_TFLOPs": round(flops / sec / 1e12, 1)}


def oracle_threads() -> int:
    """Threads the oracle's arithmetic runs on: the BLAS pool numpy calls
    (threadpoolctl's report) and torch's intra-op pool (its bf16 widening),
    whichever is larger, capped by the cores this process may use."""
    import torch
    n = torch.get_num_threads()
    try:
        from threadpoolctl import threadpool_info
        n = max([n] + [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"])
    except ImportError:
        pass
    return min(n, len(os.sched_getaffinity(0)))


def forward_plan(st, stats_blocks):
    """The decode's forwards as (kind, rows) from its steps per block: a
    full forward over N rows at each block's first step and at refresh-
    interval steps, else a cached forward over [s, N) (PrefixCache) or
    [s, s + B) (DualCache), or a full forward without a cache."""
    P, L, B = st.prompt_len, st.gen_length, st.block_size
    N = P + L
    out = []
    for k, n in enumerate(stats_blocks):
        s = P + k * B
        for t in range(n):
            r = st.refresh_interval
            if t == 0 or not st.use_cache or (r > 0 and t % r == 0):
                out.append(("full", N))
            else:
                out.append(("cached", B if st.dual_cache else N - s))
    return out


def cpu_baseline(wl, weights, stats_blocks, layers: int = 6):
    """Times the oracle (float64, host cores) on a bounded sample of the
    decode and prices the decode's own forwards with it: `layers` layers of
    a full forward over all N rows, the same layers of a cached forward at
    the smallest and the largest row count the decode's cached steps use
    (cost taken linear in the rows between them), and the LM head over the
    block rows with the confidences and the selection. Every forward of the
    GPU run (from its steps per block) then costs n_layers / layers times
    its sampled layers plus one LM head and selection."""
    import dataclasses

    import numpy as np

    from block_wise_kv_amd import synth
    from oracle import decode as od
    from oracle import model as om

    shape, st = wl.model, wl.decode
    P, L, B = st.prompt_len, st.gen_length, st.block_size
    N = P + L
    plan = forward_plan(st, stats_blocks)
    layers = min(layers, shape.n_layers)
    sub = om.Model(dataclasses.replace(shape, n_layers=layers), weights)
    full = om.Model(shape, weights)
    prompt = synth.make_prompt(shape, P, wl.seed_p)[0]
    x = np.concatenate([prompt.astype(np.int64), np.full(L, shape.mask_id)])
    flags = np.zeros(N, np.uint8)
    flags[N - B:] = 1
    t0 = time.perf_counter()
    hf, cache, _ = sub.forward_full(x)
    t_full = (time.perf_counter() - t0) / layers
    rows = sorted({m for k, m in plan if k == "cached"}) or [B]
    lo, hi = rows[0], rows[-1]
    t_rows = {}
    for m in sorted({lo, hi}):
        t0 = time.perf_counter()
        sub.forward_cached(x, N - m, N, cache)
        t_rows[m] = (time.perf_counter() - t0) / layers
    t0 = time.perf_counter()
    z = full.logits(hf[N - B:])
    c, _ = od.confidence(z)
    if st.sampling:
        from oracle import sampling as smp
        smp.tau_leap_step(z, flags[N - B:], N - B, 0, st.steps // (L // B), st.seed)
    else:
        od.select_rule(c, flags[N - B:], st.threshold, 1, st.factor, st.topk)
    t_head = time.perf_counter() - t0

    def t_cached(m):
        if hi == lo:
            return t_rows[lo]
        return t_rows[lo] + (m - lo) * (t_rows[hi] - t_rows[lo]) / (hi - lo)

    est = sum(shape.n_layers * (t_full if k == "full" else t_cached(m)) + t_head for k, m in plan)
    est *= st.batch  # the oracle decodes the sequences of a batch one after another
    sampled = layers * t_full + sum(layers * t_rows[m] for m in t_rows) + t_head
    cores = oracle_threads()
    return {
        "value": st.batch * L / est, "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": (f"float64 oracle on {cores} host cores: {layers} layers of a full forward over {N} rows "
                   f"({t_full:.2f} s per layer), of cached forwards over "
                   + ", ".join(f"{m} rows ({t_rows[m]:.2f} s per layer)" for m in sorted(t_rows))
                   + f", and the LM head over {B} rows with confidences and selection ({t_head:.2f} s): "
                   f"{sampled:.1f} s measured; value prices the GPU run's {len(plan)} forwards "
                   f"({sum(1 for k, _ in plan if k == 'full')} full, {sum(1 for k, _ in plan if k == 'cached')} "
                   f"cached, rows linear between the sampled counts) x {shape.n_layers} layers plus one LM head "
                   f"each: {est:.0f} s per decode"),
        "oracle_s_per_decode": round(est, 1),
    }


def tiny_end_to_end(F, torch):
    """The tiny fp32 workload (2 layers, d 256, vocab 2048, prompt 32, gen
    64, block 16, PrefixCache) decoded end to end by the float64 oracle and
    by fdllm_decode: tokens/s of each and whether the tokens agree."""
    import numpy as np

    from block_wise_kv_amd import synth
    from block_wise_kv_amd.runtime import GPUCache, GPUModel, decode_params
    from oracle import decode as od
    from oracle import model as om

    wl = synth.WORKLOADS["tiny_prefix"]
    shape, st = wl.model, wl.decode
    P, L = st.prompt_len, st.gen_length
    w = synth.make_weights(shape, wl.seed_w, threads=4)
    prompt = synth.make_prompt(shape, P, wl.seed_p)[0]
    t0 = time.perf_counter()
    xo, _, steps = od.decode(om.Model(shape, w), prompt, st)
    t_cpu = time.perf_counter() - t0
    gm = GPUModel(shape, w, max_seq_len=P + L)
    gc = GPUCache(gm, 1, P + L)
    x0, f0 = synth.initial_sequence(shape, prompt[None], L)
    best = None
    for _ in range(5):
        x, fl = torch.from_numpy(x0).cuda(), torch.from_numpy(f0).cuda()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        F.fdllm_decode(gm.handle, gc.handle, x, fl, 1, P, decode_params(st))
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
    same = bool(np.array_equal(x.cpu().numpy()[0], xo))
    del gc, gm
    return {"workload": "tiny_prefix", "oracle_tokens_per_s": round(L / t_cpu, 2),
            "gpu_tokens_per_s": round(L / best, 1), "oracle_s": round(t_cpu, 3), "gpu_ms": round(best * 1e3, 3),
            "oracle_forwards": len(steps), "tokens_equal": same}


def stream_ceiling(F, torch, nbytes: int = 4 << 30, reps: int = 10):
    """HBM read rate of the library's streaming-read kernel over a buffer
    16 times the last-level cache, best of `reps` event-timed launches."""
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    out = torch.empty(F.fdllm_stream_read_blocks(nbytes), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        F.fdllm_stream_read(buf, nbytes, out, st)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        F.fdllm_stream_read(buf, nbytes, out, st)
        b.record()
    torch.cuda.synchronize()
    best_ms = min(a.elapsed_time(b) for a, b in ev)
    del buf, out
    return round(nbytes / (best_ms * 1e-3) / 1e9, 1)


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
    peak_flops = (MFMA_BF16_PEAK_TFLOPS if shape.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS) * 1e12
    F.fdllm_cache_profile_peaks(cache.handle, HBM_PEAK_GBS * 1e9, peak_flops)
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
    log("measuring the streaming-read ceiling")
    ceiling = stream_ceiling(F, torch)
    log(f"streaming read: {ceiling} GB/s")
    if roofline and roofline["unit"] == "GB/s":
        roofline["frac_of_measured_ceiling"] = round(roofline["achieved"] / ceiling, 4)
    e2e = None
    if full:
        total_bytes = sum(v[2] for v in full.values())
        kernel_ms = sum(v[1] for v in full.values())
        floor_ms = total_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
        comb_ms = sum(v[4] for v in full.values())
        e2e = {"source": "last warm-up decode, every launch timed",
               "algorithmic_bytes_per_step": round(total_bytes),
               "algorithmic_flops_per_step": round(sum(v[3] for v in full.values())),
               "bytes_floor_ms": round(floor_ms, 3), "frac_of_bytes_roofline": round(floor_ms / ms_per_step, 4),
               "combined_floor_ms": round(comb_ms, 3),
               "frac_of_combined_roofline": round(comb_ms / ms_per_step, 4),
               "combined_floor": "sum over launches of max(bytes / 8 TB/s, FLOPs / MFMA peak)",
               "stream_read_ceiling_GBps": ceiling,
               "frac_of_bytes_roofline_at_measured_ceiling": round(
                   total_bytes / (ceiling * 1e9) * 1e3 / ms_per_step, 4),
               "kernel_busy_ms_per_step": round(kernel_ms, 3),
               "kernels": {k: {"launches": v[0], "ms": round(v[1], 3), "GBps": round(v[2] / (v[1] * 1e-3) / 1e9, 1),
                               "TFLOPs": round(v[3] / (v[1] * 1e-3) / 1e12, 1)}
                           for k, v in sorted(full.items(), key=lambda kv: -kv[1][1])}}

    step = step_roofline(F, torch, model, cache, x, wl) if not st.sampling else None
    if step:
        log(f"cached block step: {step['ms']} ms, {step['frac']} of the bytes roofline")

    if step:
        step["frac_of_measured_ceiling"] = round(step["bytes"] / (ceiling * 1e9) * 1e3 / step["ms"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(wl, weights, stats[-1]["steps_per_block"])
        log(f"cpu baseline {cpu['value']:.4f} tokens/s ({cpu['oracle_s_per_decode']} s per decode)")
        cpu["tiny_end_to_end"] = tiny_end_to_end(F, torch)
        log(f"tiny workload end to end: {cpu['tiny_end_to_end']}")

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
                   "cached_steps": stats[-1]["cached_steps"], "steps_per_block": stats[-1]["steps_per_block"],
                   "commits_per_step": stats[-1]["commits_per_step"]},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
