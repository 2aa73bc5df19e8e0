"""Writes the oracle's decode trajectories of the 8B/7B-shaped workloads
(test infrastructure: calls only ``oracle/`` and the seeded input
generators of ``block_wise_kv_amd.synth``).

For each workload the float64 oracle decodes the seeded prompt with the
workload's settings (block-wise, cache refreshed at every block start,
PrefixCache or DualCache steps in between, threshold selection with the
progress guarantee: [commentary] 3.4.4 "The Integrated Algorithm",
3.4.2 "PrefixCache" / "DualCache", 3.4.3 "Threshold Strategy"). Every step is
recorded compactly in ``traj_<workload>.npz``:

* the step's block, index within the block, kind (0 = refresh, 1 = cached
  forward) and forward rows [r0, r1); the quota;
* c, a, the top-2 probability gap and the maximum logit of every block row;
* the committed positions (the state before each step is the prompt plus
  the commits of all earlier steps, so it is not stored);
* the logits of a few block rows at a seeded subset of vocabulary ids and
  the final-normed hidden state of the same rows at a seeded subset of
  dimensions (estimates of the full rows' relative L2 on the GPU side);
* the oracle's own seconds per step (its measured CPU cost).

The file is rewritten after every block, with ``blocks_done``, so a partial
run is usable. Usage:

    python -m tests.golden.make_trajectories [--resume] llada8b_prefix_gen256 [...]
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

from block_wise_kv_amd import synth
from oracle import decode as od
from oracle import model as om

HERE = os.path.dirname(os.path.abspath(__file__))

# rows of the block whose sampled logits / hidden values are stored, and
# the sample sizes; the Dream-shaped run has ~900 steps, so it keeps fewer
SAMPLING = {
    "tiny_prefix": dict(rows=(0, 5, 10, 15), n_vocab=512, n_dims=128),
    "llada8b_prefix_gen256": dict(rows=(0, 10, 21, 31), n_vocab=512, n_dims=256),
    "llada8b_dual_gen512": dict(rows=(0, 10, 21, 31), n_vocab=512, n_dims=256),
    "dream7b_dual_gen1024": dict(rows=(0, 31), n_vocab=512, n_dims=128),
}
SAMPLE_SEED = 4242


def path(workload: str) -> str:
    return os.path.join(HERE, f"traj_{workload}.npz")


def collect(workload: str, threads: int = 8, log=print, on_block=None, resume=None) -> dict:
    """Runs the oracle's decode of the workload and returns the compact
    trajectory (the arrays stored in the file); on_block(arrays) is called
    after every finished block with the trajectory so far. ``resume`` (the
    arrays of a partial file) continues that run at its first unfinished
    block, from the state its committed steps leave."""
    wl = synth.WORKLOADS[workload]
    shape, st = wl.model, wl.decode
    smp = SAMPLING[workload]
    P, L, B = st.prompt_len, st.gen_length, st.block_size
    K = L // B
    t0 = time.time()
    w = synth.make_weights(shape, wl.seed_w, threads=threads)
    log(f"{workload}: weights in {time.time() - t0:.0f} s")
    model = om.Model(shape, w)
    prompt = synth.make_prompt(shape, P, wl.seed_p)[0].astype(np.int64)
    g = np.random.Generator(np.random.PCG64(SAMPLE_SEED))
    vid = np.sort(g.choice(shape.vocab, smp["n_vocab"], replace=False)).astype(np.int32)
    hdim = np.sort(g.choice(shape.d_model, smp["n_dims"], replace=False)).astype(np.int32)
    rows = np.asarray(smp["rows"], dtype=np.int32)

    recs = []
    start = None
    if resume is not None and int(resume["blocks_done"]) > 0:
        assert str(resume["workload"]) == workload and not st.sampling
        assert np.array_equal(resume["vid"], vid) and np.array_equal(resume["hdim"], hdim)
        x = np.full(P + L, shape.mask_id, dtype=np.int64)
        x[:P] = prompt
        flags = np.zeros(P + L, dtype=np.uint8)
        flags[P:] = 1
        k0 = int(resume["blocks_done"])
        for i in range(len(resume["block"])):
            if int(resume["block"][i]) >= k0:
                break
            sel = resume["sel"][resume["sel_off"][i]:resume["sel_off"][i + 1]].astype(np.int64)
            s0 = P + int(resume["block"][i]) * B
            x[sel] = resume["a"][i][sel - s0]
            flags[sel] = 0
            recs.append(dict(
                block=int(resume["block"][i]), step=int(resume["step"][i]), kind=int(resume["kind"][i]),
                r0=int(resume["r0"][i]), r1=int(resume["r1"][i]), quota=int(resume["quota"][i]),
                c=resume["c"][i], a=resume["a"][i], gap=resume["gap"][i], zmax=resume["zmax"][i],
                zs=resume["zs"][i], hs=resume["hs"][i], sel=sel, seconds=float(resume["seconds"][i])))
        assert not flags[:P + k0 * B].any() and flags[P + k0 * B:].all()
        start = (k0, x, flags)
        log(f"{workload}: resuming at block {k0} after {len(recs)} stored steps")
    tlast = [time.time()]

    def arrays(blocks_done: int) -> dict:
        n = len(recs)
        sel_off = np.zeros(n + 1, dtype=np.int64)
        for i, r in enumerate(recs):
            sel_off[i + 1] = sel_off[i] + len(r["sel"])
        return dict(
            workload=np.array(workload), prompt=prompt.astype(np.int32),
            gen_length=L, block_size=B, steps=st.steps, dual=int(st.dual_cache), tau=st.threshold,
            blocks_total=K, blocks_done=blocks_done, vid=vid, hdim=hdim, rows=rows,
            block=np.array([r["block"] for r in recs], np.int32),
            step=np.array([r["step"] for r in recs], np.int32),
            kind=np.array([r["kind"] for r in recs], np.int32),
            r0=np.array([r["r0"] for r in recs], np.int32),
            r1=np.array([r["r1"] for r in recs], np.int32),
            quota=np.array([r["quota"] for r in recs], np.int32),
            c=np.array([r["c"] for r in recs]).reshape(n, B),
            a=np.array([r["a"] for r in recs], np.int32).reshape(n, B),
            gap=np.array([r["gap"] for r in recs]).reshape(n, B),
            zmax=np.array([r["zmax"] for r in recs]).reshape(n, B),
            zs=np.array([r["zs"] for r in recs], np.float32).reshape(n, len(rows), len(vid)),
            hs=np.array([r["hs"] for r in recs], np.float32).reshape(n, len(rows), len(hdim)),
            sel_off=sel_off,
            sel=np.concatenate([r["sel"] for r in recs]).astype(np.int32) if n else np.zeros(0, np.int32),
            seconds=np.array([r["seconds"] for r in recs]))

    # the decode loop calls model.logits on the block's final hidden state;
    # record that hidden state on the way
    hid = {}
    orig_logits = model.logits

    def logits_hook(hf):
        hid["h"] = np.array(hf)
        return orig_logits(hf)

    model.logits = logits_hook

    def on_step(rec: od.Step):
        now = time.time()
        z = rec.z
        s = P + rec.block * B
        recs.append(dict(
            block=rec.block, step=rec.step, kind=0 if rec.kind == "refresh" else 1,
            r0=rec.rows[0], r1=rec.rows[1], quota=rec.quota, c=rec.c, a=rec.a,
            gap=od.top2_prob_gap(z), zmax=np.max(z, axis=-1), zs=z[rows][:, vid],
            hs=hid["h"][rows][:, hdim], sel=np.asarray(rec.selected), seconds=now - tlast[0]))
        tlast[0] = now
        assert np.all((rec.selected >= s) & (rec.selected < s + B))
        log(f"{workload}: block {rec.block} step {rec.step} {rec.kind} rows {rec.rows} "
            f"committed {len(rec.selected)} in {recs[-1]['seconds']:.1f} s")
        blk_done = not np.any(np.delete(rec.flags_before[s:s + B], rec.selected - s))
        if blk_done and on_block is not None:
            on_block(arrays(rec.block + 1))

    od.decode(model, prompt, st, on_step=on_step, start=start)
    log(f"{workload}: {len(recs)} steps in {time.time() - t0:.0f} s")
    return arrays(K)


def run(workload: str, threads: int = 8, log=print, resume: bool = False) -> str:
    """Writes traj_<workload>.npz, rewritten after every block; with
    resume, an existing partial file is continued."""
    def save(arr):
        tmp = path(workload) + ".partial"  # not matched by traj_*.npz
        with open(tmp, "wb") as f:
            np.savez_compressed(f, **arr)
        os.replace(tmp, path(workload))

    old = None
    if resume and os.path.exists(path(workload)):
        with np.load(path(workload)) as f:
            old = {k: f[k] for k in f.files}
        if int(old["blocks_done"]) >= int(old["blocks_total"]):
            return path(workload)
    collect(workload, threads, log, on_block=save, resume=old)
    return path(workload)


if __name__ == "__main__":
    args = sys.argv[1:]
    resume = "--resume" in args
    for name in [a for a in args if a != "--resume"]:
        run(name, log=lambda m: print(m, flush=True), resume=resume)
