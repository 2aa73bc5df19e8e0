"""The stored trajectory format (tests/golden/make_trajectories.py), on the CPU:
replaying the stored commits from the prompt reproduces the oracle's decode,
every stored step's confidences and ids are the oracle's, and the committed
trajectory files are complete and consistent with their workloads."""
import glob
import os

import numpy as np
import pytest

from block_wise_kv_amd import synth
from oracle import decode as od
from oracle import model as om
from tests.golden import make_trajectories as mt


def replay(tr, shape, settings):
    P, L, B = settings.prompt_len, settings.gen_length, settings.block_size
    x, flags = synth.initial_sequence(shape, tr["prompt"][None], L)
    x, flags = x[0].astype(np.int64), flags[0].copy()
    for i in range(len(tr["block"])):
        s = P + int(tr["block"][i]) * B
        sel = tr["sel"][tr["sel_off"][i]:tr["sel_off"][i + 1]].astype(np.int64)
        assert np.all(flags[sel] == 1) and np.all((sel >= s) & (sel < s + B))
        x[sel] = tr["a"][i][sel - s]
        flags[sel] = 0
    return x, flags


def test_tiny_trajectory_replays_the_oracle_decode():
    wl = synth.WORKLOADS["tiny_prefix"]
    tr = mt.collect("tiny_prefix", threads=2, log=lambda m: None)
    w = synth.make_weights(wl.model, wl.seed_w, threads=2)
    prompt = synth.make_prompt(wl.model, wl.decode.prompt_len, wl.seed_p)[0]
    xo, fo, steps = od.decode(om.Model(wl.model, w), prompt, wl.decode)
    x, flags = replay(tr, wl.model, wl.decode)
    np.testing.assert_array_equal(x, xo)
    assert not flags.any() and not fo.any()
    assert len(steps) == len(tr["block"]) == int(np.sum(tr["kind"] == 0)) + int(np.sum(tr["kind"] == 1))
    for i, rec in enumerate(steps):
        np.testing.assert_array_equal(tr["a"][i], rec.a)
        np.testing.assert_allclose(tr["c"][i], rec.c, rtol=0, atol=0)
        np.testing.assert_allclose(tr["zs"][i], rec.z[tr["rows"]][:, tr["vid"]].astype(np.float32))


def test_resumed_trajectory_equals_an_uninterrupted_one():
    """A run continued from a partial file (the blocks before the cut plus
    the state their commits leave) records the same steps as one run."""
    full = mt.collect("tiny_prefix", threads=2, log=lambda m: None)
    k0 = 2
    n = int(np.sum(full["block"] < k0))
    cut = dict(full)
    for key in ("block", "step", "kind", "r0", "r1", "quota", "c", "a", "gap", "zmax", "zs", "hs", "seconds"):
        cut[key] = full[key][:n]
    cut["sel_off"] = full["sel_off"][:n + 1]
    cut["sel"] = full["sel"][:full["sel_off"][n]]
    cut["blocks_done"] = k0
    resumed = mt.collect("tiny_prefix", threads=2, log=lambda m: None, resume=cut)
    for key, v in full.items():
        if key != "seconds":
            np.testing.assert_array_equal(resumed[key], v, err_msg=key)


@pytest.mark.parametrize("path", sorted(p for p in glob.glob(os.path.join(os.path.dirname(mt.__file__), "traj_*.npz"))
                                         if ".tmp" not in os.path.basename(p)))
def test_stored_trajectories_are_consistent(path):
    tr = dict(np.load(path))
    name = str(tr["workload"])
    wl = synth.WORKLOADS[name]
    st = wl.decode
    P, L, B = st.prompt_len, st.gen_length, st.block_size
    assert int(tr["gen_length"]) == L and int(tr["block_size"]) == B and int(tr["dual"]) == int(st.dual_cache)
    np.testing.assert_array_equal(tr["prompt"], synth.make_prompt(wl.model, P, wl.seed_p)[0])
    done = int(tr["blocks_done"])
    assert 1 <= done <= L // B and set(np.unique(tr["block"])) == set(range(done))
    T = st.steps // (L // B)
    for k in range(done):
        steps = tr["step"][tr["block"] == k]
        assert list(steps) == list(range(len(steps))) and len(steps) <= T
        assert tr["kind"][tr["block"] == k][0] == 0 and np.all(tr["kind"][tr["block"] == k][1:] == 1)
    x, flags = replay(tr, wl.model, st)
    # the finished blocks are fully decoded, the rest untouched
    assert not flags[P:P + done * B].any() and flags[P + done * B:].all()
    # every step commits at least one position, and the confidences are probabilities
    assert np.all(np.diff(tr["sel_off"]) >= 1)
    assert np.all((tr["c"] > 0) & (tr["c"] <= 1))
