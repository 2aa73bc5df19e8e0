"""Logit-scale calibration of the random-init 8B/7B-shaped workloads (test
infrastructure; calls only the oracle and the seeded input generators).

The workloads ask for logits "scaled so the median top-1 probability is about
0.9". Reading: run the oracle's first forward of the workload (the prompt
followed by gen_length masks), take the LM-head logits of all gen_length
generated rows at scale 1, and bisect the scale alpha until the median over
those rows of max softmax(alpha * z) is 0.90 +- 0.005; alpha is then rounded to
three significant figures. The confidence of a row grows monotonically with
alpha, so bisection applies.

    python -m oracle.calibrate llada8b_prefix_gen256
"""
from __future__ import annotations

import dataclasses
import json
import sys
import time

import numpy as np

from block_wise_kv_amd import synth
from oracle import decode as od
from oracle import model as om


def median_conf(z0: np.ndarray, alpha: float) -> float:
    c, _ = od.confidence(alpha * z0)
    return float(np.median(c))


def calibrate(workload: str, threads: int = 8) -> dict:
    wl = synth.WORKLOADS[workload]
    shape = dataclasses.replace(wl.model, logit_scale=1.0)
    t0 = time.time()
    w = synth.make_weights(shape, wl.seed_w, threads=threads)
    t1 = time.time()
    prompt = synth.make_prompt(shape, wl.decode.prompt_len, wl.seed_p)[0]
    x, _ = synth.initial_sequence(shape, prompt[None], wl.decode.gen_length)
    m = om.Model(shape, w)
    hf, _, _ = m.forward_full(x[0].astype(np.int64))
    P = wl.decode.prompt_len
    z0 = m.logits(hf[P:])  # scale 1
    t2 = time.time()
    lo, hi = 0.0, 1.0
    while median_conf(z0, hi) < 0.9:
        hi *= 2
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if median_conf(z0, mid) < 0.9:
            lo = mid
        else:
            hi = mid
    alpha = float(f"{hi:.3g}")
    med = median_conf(z0, alpha)
    c, _ = od.confidence(alpha * z0)
    return dict(workload=workload, alpha=alpha, median_top1=med,
                frac_above_0_9=float(np.mean(c >= 0.9)),
                quartiles=[float(q) for q in np.quantile(c, [0.25, 0.5, 0.75])],
                seconds_weights=t1 - t0, seconds_forward=t2 - t1)


if __name__ == "__main__":
    for name in sys.argv[1:]:
        print(json.dumps(calibrate(name)), flush=True)
