"""Parity at the evaluated models' full widths, in the launch configurations
the benchmark times.

* The LLaDA-8B- and Dream-7B-shaped layer stacks at full width (d_model,
  heads, FFN and the whole vocabulary) cut to two layers, so that the float64
  oracle can run the same forward: cache refresh over all N rows, a
  PrefixCache step over [s, N) and a DualCache step over [s, e), with the
  workloads' prompt and generation lengths. Every kernel runs with the row
  counts, key lengths and tile plans of the benchmark's decode.
* The full 32-layer LLaDA-8B-shaped model of the benchmark, through
  properties that hold at any depth: a cached forward run right after a
  refresh with the sequence unchanged reproduces the refresh's block logits,
  PrefixCache and DualCache run the same rows in the last block, and the
  whole decode commits every position within its step budget.
"""
import dataclasses

import numpy as np
import pytest

from block_wise_kv_amd import synth
from oracle import decode as od
from oracle import model as om
from tests.helpers import TOL, StepCheck, host, rel_l2

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TWO_LAYER = {
    "llada8b_2layer": ("llada8b_prefix_gen256", dataclasses.replace(synth.LLADA8B, n_layers=2)),
    # the DualCache gen-512 workload's own sequence length, 1024
    "llada8b_2layer_n1024": ("llada8b_dual_gen512", dataclasses.replace(synth.LLADA8B, n_layers=2)),
    "dream7b_2layer": ("dream7b_dual_gen1024", dataclasses.replace(synth.DREAM7B, n_layers=2)),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_built = {}


def build(name):
    from block_wise_kv_amd.runtime import GPUCache, GPUModel
    if name not in _built:
        _built.clear()  # one full-width model on the device at a time
        wl_name, shape = TWO_LAYER[name]
        wl = synth.WORKLOADS[wl_name]
        st = wl.decode
        N = st.prompt_len + st.gen_length
        w = synth.make_weights(shape, wl.seed_w, threads=16)
        gm = GPUModel(shape, w, max_seq_len=N)
        gc = GPUCache(gm, 1, N)
        prompt = synth.make_prompt(shape, st.prompt_len, wl.seed_p)[0]
        _built[name] = (shape, st, om.Model(shape, w), gm, gc, prompt)
    return _built[name]


def step(gm, gc, shape, x, flags, rows, s, B, tau, t, T, **rule):
    """One forward (refresh if rows is None) and the fused unmask on device
    copies of x / flags (rule: factor / topk / sampling / seed of the
    selection); returns hidden, logits, conf, argmax, committed (and with
    rule given, the ids after the call)."""
    from block_wise_kv_amd import fdllm as F
    N = x.shape[-1]
    tx = torch.from_numpy(x[None].astype(np.int32)).cuda()
    tf = torch.from_numpy(flags[None].astype(np.uint8)).cuda()
    hidden = torch.empty(1, B, shape.d_model, dtype=torch.float32, device="cuda")
    if rows is None:
        F.fdllm_cache_refresh(gm.handle, gc.handle, tx, 1, N, s, B, hidden)
    else:
        F.fdllm_block_forward(gm.handle, gc.handle, tx, 1, N, rows[0], rows[1], s, B, hidden)
    logits = torch.empty(1, B, shape.vocab, device="cuda")
    conf = torch.empty(1, B, device="cuda")
    am = torch.empty(1, B, dtype=torch.int32, device="cuda")
    counts = torch.empty(1, 2, dtype=torch.int32, device="cuda")
    F.fdllm_confidence_unmask(gm.handle, gc.handle, hidden, tx, tf, 1, N, s, B, tau, t, T, conf, am,
                              counts, logits, **rule)
    torch.cuda.synchronize()
    committed = (flags[s:s + B] == 1) & (tf.cpu().numpy()[0, s:s + B] == 0)
    out = (host(hidden)[0], logits.cpu().numpy()[0], conf.cpu().numpy()[0], am.cpu().numpy()[0], committed)
    return out + (tx.cpu().numpy()[0],) if rule else out


def state(shape, st, prompt, s):
    """The sequence at block start s: earlier generated positions decoded
    (seeded ids), the rest masked."""
    P, L = st.prompt_len, st.gen_length
    x, flags = synth.initial_sequence(shape, prompt[None], L)
    x, flags = x[0].copy(), flags[0].copy()
    g = np.random.Generator(np.random.PCG64(99))
    x[P:s] = g.integers(0, shape.vocab - 1, s - P)
    flags[P:s] = 0
    return x, flags


def check(rec_z, x, flags, s, B, tau, out, tol, label):
    hid, logits, conf, am, com = out
    ez = rel_l2(logits, rec_z)
    print(f"{label}: logits rel L2 {ez:.2e}")
    assert ez < tol
    c, a = od.confidence(rec_z)
    rec = od.Step(0, 0, label, (s, s + B), x, flags, rec_z, c, a, 1, s + od.select(c, flags[s:s + B], tau), {})
    chk = StepCheck(tau)
    chk(rec, s, am, conf, com)
    assert chk.compared > 0


@pytest.mark.parametrize("name", list(TWO_LAYER))
def test_full_width_refresh(name):
    shape, st, o, gm, gc, prompt = build(name)
    B, P = st.block_size, st.prompt_len
    N = P + st.gen_length
    s = P + B  # second block: the first is decoded
    x, flags = state(shape, st, prompt, s)
    hf, _, _ = o.forward_full(x.astype(np.int64))
    out = step(gm, gc, shape, x, flags, None, s, B, st.threshold, 0, B)
    eh = rel_l2(out[0], hf[s:s + B])
    print(f"{name} refresh over {N} rows: hidden rel L2 {eh:.2e}")
    assert eh < TOL[shape.dtype]
    check(o.logits(hf[s:s + B]), x, flags, s, B, st.threshold, out, TOL[shape.dtype], f"{name} refresh")


@pytest.mark.parametrize("name", list(TWO_LAYER))
@pytest.mark.parametrize("dual", [False, True])
def test_full_width_cached_step(name, dual):
    shape, st, o, gm, gc, prompt = build(name)
    B, P = st.block_size, st.prompt_len
    N = P + st.gen_length
    s = P + B
    x, flags = state(shape, st, prompt, s)
    _, cache, _ = o.forward_full(x.astype(np.int64))
    step(gm, gc, shape, x, flags, None, s, B, st.threshold, 0, B)  # the device cache of the same x
    x2, f2 = x.copy(), flags.copy()
    x2[s + 2], x2[s + 9], x2[s + 20] = 17, 1234, 98765 % shape.vocab
    f2[s + 2] = f2[s + 9] = f2[s + 20] = 0
    r1 = s + B if dual else N
    hr, _ = o.forward_cached(x2.astype(np.int64), s, r1, cache)
    out = step(gm, gc, shape, x2, f2, (s, r1), s, B, st.threshold, 1, B)
    eh = rel_l2(out[0], hr[:B])
    print(f"{name} {'dual' if dual else 'prefix'} step over {r1 - s} rows: hidden rel L2 {eh:.2e}")
    assert eh < TOL[shape.dtype]
    check(o.logits(hr[:B]), x2, f2, s, B, st.threshold, out, TOL[shape.dtype],
          f"{name} {'dual' if dual else 'prefix'}")


@pytest.mark.parametrize("name", ["llada8b_2layer", "dream7b_2layer"])
def test_full_width_batch_lockstep(name):
    """Two sequences in one cache, in lockstep (the batch > 1 decode): a
    refresh of both and then a DualCache step of both, so every projection
    runs over 2 x 32 block rows, and the fused unmask over both; each
    sequence against its own oracle forward ([commentary] 3.4.4, 3.4.2)."""
    from block_wise_kv_amd import fdllm as F
    from block_wise_kv_amd.runtime import GPUCache
    shape, st, o, gm, gc, prompt = build(name)
    B, P = st.block_size, st.prompt_len
    N = P + st.gen_length
    s = P + B
    xa, fa = state(shape, st, prompt, s)
    xb, fb = xa.copy(), fa.copy()
    g = np.random.Generator(np.random.PCG64(7))
    xb[P:s] = g.integers(0, shape.vocab - 1, s - P)  # another decoded first block
    X, Fl = np.stack([xa, xb]), np.stack([fa, fb])
    gc2 = GPUCache(gm, 2, N)
    d = shape.d_model

    def run(x, flags, rows, t):
        tx = torch.from_numpy(x.astype(np.int32)).cuda()
        tf = torch.from_numpy(flags.astype(np.uint8)).cuda()
        hidden = torch.empty(2, B, d, dtype=torch.float32, device="cuda")
        if rows is None:
            F.fdllm_cache_refresh(gm.handle, gc2.handle, tx, 2, N, s, B, hidden)
        else:
            F.fdllm_block_forward(gm.handle, gc2.handle, tx, 2, N, rows[0], rows[1], s, B, hidden)
        logits = torch.empty(2, B, shape.vocab, device="cuda")
        conf = torch.empty(2, B, device="cuda")
        am = torch.empty(2, B, dtype=torch.int32, device="cuda")
        counts = torch.empty(2, 2, dtype=torch.int32, device="cuda")
        F.fdllm_confidence_unmask(gm.handle, gc2.handle, hidden, tx, tf, 2, N, s, B, st.threshold, t, B,
                                  conf, am, counts, logits)
        torch.cuda.synchronize()
        fl = tf.cpu().numpy()
        return [(host(hidden)[i], logits.cpu().numpy()[i], conf.cpu().numpy()[i], am.cpu().numpy()[i],
                 (flags[i, s:s + B] == 1) & (fl[i, s:s + B] == 0)) for i in range(2)]

    caches = []
    outs = run(X, Fl, None, 0)
    for i in range(2):
        hf, cache_i, _ = o.forward_full(X[i].astype(np.int64))
        caches.append(cache_i)
        eh = rel_l2(outs[i][0], hf[s:s + B])
        print(f"{name} batch-2 refresh, sequence {i}: hidden rel L2 {eh:.2e}")
        assert eh < TOL[shape.dtype]
        check(o.logits(hf[s:s + B]), X[i], Fl[i], s, B, st.threshold, outs[i], TOL[shape.dtype],
              f"{name} batch-2 refresh {i}")
    # the device cache holds the refreshed K/V of X; a DualCache step on
    # changed block tokens of each sequence
    X2, F2 = X.copy(), Fl.copy()
    X2[0, s + 3], X2[1, s + 7], X2[1, s + 30] = 11, 222, 3333
    F2[0, s + 3] = F2[1, s + 7] = F2[1, s + 30] = 0
    outs = run(X2, F2, (s, s + B), 1)
    for i in range(2):
        hr, _ = o.forward_cached(X2[i].astype(np.int64), s, s + B, caches[i])
        eh = rel_l2(outs[i][0], hr[:B])
        print(f"{name} batch-2 dual step, sequence {i}: hidden rel L2 {eh:.2e}")
        assert eh < TOL[shape.dtype]
        check(o.logits(hr[:B]), X2[i], F2[i], s, B, st.threshold, outs[i], TOL[shape.dtype],
              f"{name} batch-2 dual {i}")


@pytest.mark.parametrize("name", ["llada8b_2layer", "dream7b_2layer"])
@pytest.mark.parametrize("rule", ["factor", "topk", "sampling"])
def test_full_width_selection_rules(name, rule):
    """The selection variants at the full vocabulary (126464 / 152064 ids)
    after a full-width refresh: the factor strategy at f = 1 and fixed top-4
    ([commentary] 3.4.3) and tau-leaping sampling ([commentary] 3.4.1)
    against the oracle's choice on its own logits; sampled tokens must equal
    the oracle's draws bar near-ties."""
    from oracle import sampling as smp
    from tests.helpers import sample_fragile
    shape, st, o, gm, gc, prompt = build(name)
    B, P = st.block_size, st.prompt_len
    s = P + B
    x, flags = state(shape, st, prompt, s)
    flags[s + 5] = flags[s + 17] = 0  # two positions of the block already decoded
    x[s + 5], x[s + 17] = 11, 222
    T, t = 8, 2
    kw = {"factor": dict(factor=1.0), "topk": dict(topk=4), "sampling": dict(sampling=True, seed=9)}[rule]
    out = step(gm, gc, shape, x, flags, None, s, B, st.threshold, t, T, **kw)
    hf, _, _ = o.forward_full(x.astype(np.int64))
    z = o.logits(hf[s:s + B])
    assert rel_l2(out[1], z) < TOL[shape.dtype]
    c, a = od.confidence(z)
    masked = flags[s:s + B]
    quota = max(1, -(-int(masked.sum()) // (T - t)))
    tok = None
    if rule == "sampling":
        sel, tok = smp.tau_leap_step(z, masked, s, t, T, 9, 0)
    else:
        sel = od.select_rule(c, masked, st.threshold, quota, kw.get("factor", 0.0), kw.get("topk", 0))
    rec = od.Step(0, t, "refresh", (0, P + st.gen_length), x, flags, z, c, a, quota, sel + s, {}, tok)
    chk = StepCheck(st.threshold, kw.get("factor", 0.0), kw.get("topk", 0), 9 if rule == "sampling" else None,
                    dtype=shape.dtype)
    chk(rec, s, out[3], out[2], out[4])
    assert chk.compared > 0
    if rule == "sampling":
        for j in sel:
            if not sample_fragile(z[j], 9, 0, s + j, t):
                assert out[5][s + j] == tok[j], (j, out[5][s + j], tok[j])
    print(f"{name} {rule}: {len(sel)} committed, {chk.compared} compared, {chk.excluded} excluded, "
          f"{chk.factor_ties} set-rule near-ties")


@pytest.mark.parametrize("name", ["llada8b_2layer", "dream7b_2layer"])
def test_full_width_runs_are_bitwise_deterministic(name):
    """The split-K GEMM merges, the attention split merges and the LM-head
    tile merge run in a fixed order: a refresh and a cached step repeated on
    the same inputs give bitwise identical hidden states, logits and
    confidences."""
    shape, st, o, gm, gc, prompt = build(name)
    B, P = st.block_size, st.prompt_len
    N = P + st.gen_length
    s = P + B
    x, flags = state(shape, st, prompt, s)
    outs = []
    for _ in range(2):
        r = step(gm, gc, shape, x, flags, None, s, B, st.threshold, 0, B)
        c = step(gm, gc, shape, x, flags, (s, s + B), s, B, st.threshold, 1, B)
        outs.append((r, c))
    for a, b in zip(outs[0], outs[1]):
        for u, v in zip(a, b):
            assert np.array_equal(u, v)


# ---- the full 32-layer model of the benchmark ---------------------------------

@pytest.fixture(scope="module")
def full_llada():
    from block_wise_kv_amd.runtime import GPUCache, GPUModel
    _built.clear()
    wl = synth.WORKLOADS["llada8b_prefix_gen256"]
    shape, st = wl.model, wl.decode
    N = st.prompt_len + st.gen_length
    w = synth.make_weights(shape, wl.seed_w, threads=16)
    gm = GPUModel(shape, w, max_seq_len=N)
    del w
    gc = GPUCache(gm, 1, N)
    prompt = synth.make_prompt(shape, st.prompt_len, wl.seed_p)[0]
    yield shape, st, gm, gc, prompt
    del gc, gm


def test_full_model_cached_forward_reproduces_refresh(full_llada):
    shape, st, gm, gc, prompt = full_llada
    B, P = st.block_size, st.prompt_len
    N = P + st.gen_length
    for s in (P, N - 3 * B):
        x, flags = state(shape, st, prompt, s)
        _, z0, c0, a0, _ = step(gm, gc, shape, x, flags, None, s, B, 2.0, 0, B)
        _, z1, c1, a1, _ = step(gm, gc, shape, x, flags, (s, N), s, B, 2.0, 1, B)
        e = rel_l2(z1, z0)
        gap = od.top2_prob_gap(z0.astype(np.float64))
        same = (a0 == a1) | (gap < 1e-3)
        print(f"block at {s}: cached vs refresh logits rel L2 {e:.2e}, argmax equal at {int((a0 == a1).sum())}/{B}")
        assert e < 1e-3 and same.all()


def test_full_model_prefix_equals_dual_in_last_block(full_llada):
    shape, st, gm, gc, prompt = full_llada
    B, P = st.block_size, st.prompt_len
    N = P + st.gen_length
    s = N - B
    x, flags = state(shape, st, prompt, s)
    x2, f2 = x.copy(), flags.copy()
    x2[s + 1] = 77
    f2[s + 1] = 0
    # each cached step runs over the cache a refresh of the original x built
    step(gm, gc, shape, x, flags, None, s, B, 0.9, 0, B)
    hp, zp, _, ap, _ = step(gm, gc, shape, x2, f2, (s, N), s, B, 0.9, 1, B)
    step(gm, gc, shape, x, flags, None, s, B, 0.9, 0, B)
    hd, zd, _, ad, _ = step(gm, gc, shape, x2, f2, (s, s + B), s, B, 0.9, 1, B)
    assert np.array_equal(hp, hd) and np.array_equal(zp, zd) and np.array_equal(ap, ad)


@pytest.mark.parametrize("rule", ["threshold", "factor"])
def test_full_model_decode_commits_every_position(full_llada, rule):
    from block_wise_kv_amd import fdllm as F
    from block_wise_kv_amd.runtime import decode_params
    shape, st, gm, gc, prompt = full_llada
    if rule == "factor":
        st = synth.WORKLOADS["llada8b_prefix_gen256_factor"].decode
    P, L, B = st.prompt_len, st.gen_length, st.block_size
    K, T = L // B, st.steps // (L // B)
    x0, f0 = synth.initial_sequence(shape, prompt[None], L)
    x = torch.from_numpy(x0).cuda()
    fl = torch.from_numpy(f0).cuda()
    stats = F.fdllm_decode(gm.handle, gc.handle, x, fl, 1, P, decode_params(st)).as_dict(K)
    xs, fs = x.cpu().numpy()[0], fl.cpu().numpy()[0]
    print(f"decode: nfe {stats['nfe']}, steps per block {stats['steps_per_block']}")
    assert not fs.any()
    assert np.array_equal(xs[:P], prompt)
    assert ((xs[P:] >= 0) & (xs[P:] < shape.vocab)).all()
    assert stats["committed"] == L
    assert stats["refreshes"] == K
    assert all(1 <= n <= T for n in stats["steps_per_block"])
    assert stats["nfe"] == sum(stats["steps_per_block"])
    assert len(stats["commits_per_step"]) == stats["nfe"] and sum(stats["commits_per_step"]) == L
    assert min(stats["commits_per_step"]) >= 1
