"""Drift of the approximate cache during a decode: how far the keys and
values a block's cached steps reuse have moved from what a fresh forward
would compute ([commentary] 3.4.2 "The Empirical Justification: Cosine
Similarity of KV Activations", Figure 3: (a) prompt tokens, (b) the masked
suffix). Reads the library through its C ABI.

    python3 -m block_wise_kv_amd.kv_drift [--workload NAME] [--blocks K] [--out FILE]

The decode runs step by step as ``fdllm_decode`` does (cache rebuilt at each
block start, cached forwards after it, the workload's selection rule). Right
after each block-start rebuild every layer's K and V are copied out; at every
later step of the block a second cache is rebuilt from the current tokens
and ``fdllm_kv_cosine`` compares the two per token. Reported per step: the
mean over layers and tokens of the K and V cosine for the prompt rows
[0, P) and for the suffix rows [e, N) (the rows the DualCache also reuses),
and the lowest per-layer mean.

With random-init weights the values say nothing about the pages' trained
models; the tool is the measurement, parity-tested against the oracle on the
tiny models.
"""
from __future__ import annotations

import argparse
import json
import sys
import time

import numpy as np

from . import fdllm as F
from . import synth


def _snapshot(cache, layer, shape):
    kp, vp, ncap = F.fdllm_cache_kv(cache.handle, layer)
    nbytes = cache.batch * shape.n_kv_heads * ncap * shape.head_dim * (2 if shape.dtype == "bf16" else 4)
    base = cache.mem.data_ptr()
    k = cache.mem[kp - base:kp - base + nbytes].clone()
    v = cache.mem[vp - base:vp - base + nbytes].clone()
    return k, v, ncap


def run(workload: str, blocks: int, torch, log=print):
    from .runtime import GPUCache, GPUModel
    wl = synth.WORKLOADS[workload]
    shape, st = wl.model, wl.decode
    if st.batch != 1:
        raise SystemExit("kv_drift runs one sequence")
    P, L, B = st.prompt_len, st.gen_length, st.block_size
    N = P + L
    K, T = L // B, st.steps // (L // B)
    weights = synth.make_weights(shape, wl.seed_w, threads=16)
    gm = GPUModel(shape, weights, max_seq_len=N)
    del weights
    ca = GPUCache(gm, 1, N)   # the decode's cache
    cb = GPUCache(gm, 1, N)   # rebuilt from the current tokens at every step
    ca.batch = cb.batch = 1
    prompt = synth.make_prompt(shape, P, wl.seed_p)[0]
    x0, f0 = synth.initial_sequence(shape, prompt[None], L)
    x = torch.from_numpy(x0).cuda()
    fl = torch.from_numpy(f0).cuda()
    hid = torch.empty(1, B, shape.d_model, device="cuda")
    counts = torch.zeros(1, 2, dtype=torch.int32, device="cuda")
    dt = F.BF16 if shape.dtype == "bf16" else F.F32
    cos = torch.empty(N * 2, device="cuda")
    rows = []
    for k in range(min(blocks, K)):
        s, e = P + k * B, P + (k + 1) * B
        snap = None
        for t in range(T):
            if t == 0:
                F.fdllm_cache_refresh(gm.handle, ca.handle, x, 1, N, s, B, hid)
                snap = [_snapshot(ca, l, shape) for l in range(shape.n_layers)]
            else:
                r1 = e if st.dual_cache else N
                F.fdllm_block_forward(gm.handle, ca.handle, x, 1, N, s, r1, s, B, hid)
            x_before = x.clone()
            F.fdllm_confidence_unmask(gm.handle, ca.handle, hid, x, fl, 1, N, s, B, st.threshold, t, T,
                                      None, None, counts, None, factor=st.factor)
            torch.cuda.synchronize()
            if t > 0:
                # the cached step just run reused the block-start K/V: compare
                # them with a fresh rebuild from the tokens it saw
                F.fdllm_cache_refresh(gm.handle, cb.handle, x_before, 1, N, s, B, hid)
                per_layer = []
                for l in range(shape.n_layers):
                    ka, va, ncap = snap[l]
                    kb, vb, _ = F.fdllm_cache_kv(cb.handle, l)
                    F.fdllm_kv_cosine(ka, va, kb, vb, 1, shape.n_kv_heads, ncap, shape.head_dim, 0, N,
                                      dt, cos)
                    c = cos.view(N, 2).cpu().numpy()
                    per_layer.append((c[:P].mean(0), c[e:].mean(0) if e < N else np.array([np.nan] * 2)))
                pk = np.array([p[0][0] for p in per_layer]); pv = np.array([p[0][1] for p in per_layer])
                sk = np.array([p[1][0] for p in per_layer]); sv = np.array([p[1][1] for p in per_layer])
                row = {"block": k, "step": t,
                       "prompt_k": round(float(pk.mean()), 6), "prompt_v": round(float(pv.mean()), 6),
                       "prompt_min_layer": round(float(np.minimum(pk, pv).min()), 6),
                       "suffix_k": round(float(np.nanmean(sk)), 6), "suffix_v": round(float(np.nanmean(sv)), 6),
                       "suffix_min_layer": round(float(np.nanmin(np.minimum(sk, sv))), 6)}
                rows.append(row)
                log(json.dumps(row))
            left = int(counts[0, 1].item())
            if left == 0:
                break
    return {"workload": workload, "blocks": min(blocks, K), "steps": rows}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="llada8b_prefix_gen256")
    ap.add_argument("--blocks", type=int, default=2)
    ap.add_argument("--out")
    a = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("kv_drift needs a GPU")
    F.lib()
    t0 = time.time()
    res = run(a.workload, a.blocks, torch, log=lambda m: print(m, file=sys.stderr, flush=True))
    res["seconds"] = round(time.time() - t0, 1)
    text = json.dumps(res, indent=1)
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text + "\n")
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
