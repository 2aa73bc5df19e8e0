"""Timing of the two standalone kernels over their sweep shapes, against the
HBM roofline (reads the library through its C ABI; no parity checks here,
those live in the GPU tests).

    python3 -m block_wise_kv_amd.kernel_sweep [--reps 20] [--out FILE]

* Block attention (bidirectional, no mask): batch 8, 32 query rows,
  32 heads x 128, KV length 1024 / 2048 / 4096 / 8192, bf16. Algorithmic
  bytes per call: K and V once (2 * b * L * H * D * 2) plus Q and O
  (2 * b * rows * H * D * 2).
* Confidence unmask with the logits as input: bf16 logits [8][32][126464],
  scale {5, 10, 20} x masked fraction {1, 0.5, 0.1} x tau {0.7, 0.9, 0.95}.
  Algorithmic bytes per call: the logits of the still-masked rows once
  (64.75 MB when every row is masked), plus ids, flags and the per-position
  outputs.

Each case rotates over enough distinct buffer sets (more than 512 MB in
all) that a call's operands are not left in the 256 MB last-level cache by
the previous call, and is timed with events on the launch stream. Values
are seeded N(0, 1) draws (times the scale for the logits) made on the GPU;
timing does not depend on them beyond the masked pattern, which is the
seeded one the parity tests use.
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np

from . import fdllm as F
from . import synth

HBM_PEAK_GBPS = 8000.0
ROTATE_BYTES = 768 << 20   # more than the 256 MB last-level cache, twice over


def _time(fn, n_sets: int, reps: int, torch, pre=None) -> float:
    """Mean ms per call over reps calls, cycling through n_sets operand sets.
    Each call is bracketed by its own pair of events, so host-side gaps and
    the optional untimed pre(i) step stay out of the figure."""
    for i in range(n_sets):
        if pre:
            pre(i)
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for r in range(reps):
        if pre:
            pre(r % n_sets)
        ev[r][0].record()
        fn(r % n_sets)
        ev[r][1].record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / reps


def attention_sweep(reps: int, torch) -> list:
    cfg = synth.SWEEP_ATTN
    b, rows, h, d = cfg["batch"], cfg["q_rows"], cfg["n_heads"], cfg["head_dim"]
    out = []
    gen = torch.Generator(device="cuda")
    for kv in cfg["kv_lens"]:
        gen.manual_seed(cfg["seed"] * 100003 + kv)
        kv_bytes = 2 * b * h * kv * d * 2
        qo_bytes = 2 * b * rows * h * d * 2
        n_sets = max(2, -(-ROTATE_BYTES // kv_bytes))
        sets = []
        for _ in range(n_sets):
            q = torch.randn(b, rows, h, d, device="cuda", generator=gen).to(torch.bfloat16)
            k = torch.randn(b, h, kv, d, device="cuda", generator=gen).to(torch.bfloat16)
            vt = torch.randn(b, h, d, kv, device="cuda", generator=gen).to(torch.bfloat16)
            o = torch.empty_like(q)
            ws = torch.zeros(F.fdllm_block_attention_workspace(b, rows, h, d, kv), dtype=torch.uint8,
                             device="cuda")
            sets.append((q, k, vt, o, ws))
        scale = 1.0 / float(np.sqrt(d))

        def call(i):
            q, k, vt, o, ws = sets[i]
            F.fdllm_block_attention(q, k, vt, o, b, rows, h, h, d, kv, F.BF16, scale, ws)

        ms = _time(call, n_sets, reps, torch)
        nbytes = kv_bytes + qo_bytes
        flops = 4.0 * b * rows * h * kv * d
        gbps = nbytes / ms / 1e6
        out.append({"kernel": "attention", "kv_len": kv, "batch": b, "q_rows": rows, "heads": h,
                    "head_dim": d, "us": round(ms * 1e3, 2), "bytes": nbytes, "GBps": round(gbps, 1),
                    "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4), "TFLOPs": round(flops / ms / 1e9, 2),
                    "floor_us": round(nbytes / HBM_PEAK_GBPS / 1e3, 2), "buffer_sets": n_sets})
        print(json.dumps(out[-1]), file=sys.stderr, flush=True)
        del sets
        torch.cuda.empty_cache()
    return out


def unmask_sweep(reps: int, torch) -> list:
    cfg = synth.SWEEP_UNMASK
    b, B, V = cfg["batch"], cfg["block"], cfg["vocab"]
    seq_extra = 5
    seq_len = B + seq_extra
    logit_bytes = b * B * V * 2
    n_sets = max(2, -(-ROTATE_BYTES // logit_bytes))
    gen = torch.Generator(device="cuda")
    out = []
    for scale in cfg["scales"]:
        gen.manual_seed(cfg["seed"] * 1009 + int(scale))
        zs = [(torch.randn(b, B, V, device="cuda", generator=gen) * scale).to(torch.bfloat16)
              for _ in range(n_sets)]
        for frac in cfg["masked_fracs"]:
            flags_blk = synth.sweep_masked(b, B, frac, cfg["seed"])
            flags0 = np.zeros((b, seq_len), np.uint8)
            flags0[:, seq_extra:] = flags_blk
            x0 = np.full((b, seq_len), 7, np.int32)
            x0[:, seq_extra:] = -1
            tx0 = torch.from_numpy(x0).cuda()
            tf0 = torch.from_numpy(flags0).cuda()
            for tau in cfg["taus"]:
                tx, tf = tx0.clone(), tf0.clone()
                conf = torch.zeros(b, B, device="cuda")
                am = torch.zeros(b, B, dtype=torch.int32, device="cuda")
                counts = torch.zeros(b, 2, dtype=torch.int32, device="cuda")
                ws = torch.zeros(F.fdllm_unmask_logits_workspace(b, B, V), dtype=torch.uint8,
                                 device="cuda")

                def reset(i):
                    # every call starts from the same ids and flags, so each
                    # one selects over the same masked pattern
                    tx.copy_(tx0)
                    tf.copy_(tf0)

                def call(i):
                    F.fdllm_confidence_unmask_logits(zs[i], F.BF16, tx, tf, b, seq_len, seq_extra, B, V,
                                                     tau, 0, B, conf, am, counts, ws)

                ms = _time(call, n_sets, reps, torch, pre=reset)
                # only rows still masked are read
                active = int(flags_blk.sum())
                nbytes = active * V * 2 + b * B * (4 + 1) * 2 + b * B * 8 + b * 8
                gbps = nbytes / ms / 1e6
                out.append({"kernel": "unmask_logits", "scale": scale, "masked_frac": frac, "tau": tau,
                            "rows_read": active, "us": round(ms * 1e3, 2), "bytes": nbytes, "GBps": round(gbps, 1),
                            "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4),
                            "floor_us": round(nbytes / HBM_PEAK_GBPS / 1e3, 2), "buffer_sets": n_sets})
                print(json.dumps(out[-1]), file=sys.stderr, flush=True)
        del zs
        torch.cuda.empty_cache()
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--only", choices=("attention", "unmask"))
    ap.add_argument("--out")
    a = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("kernel_sweep needs a GPU")
    F.lib()
    res = {}
    if a.only in (None, "attention"):
        res["attention"] = attention_sweep(a.reps, torch)
    if a.only in (None, "unmask"):
        res["unmask_logits"] = unmask_sweep(a.reps, torch)
    text = json.dumps(res, indent=1)
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text + "\n")
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
