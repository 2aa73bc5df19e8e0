"""GPU parity of the model path -- cache refresh, cached block forward (Prefix
and Dual), fused LM-head confidence unmask and the whole decode -- against
the oracle, through the C ABI, on small models that span several tiles, GQA,
both head sizes and a ragged sequence length."""
import dataclasses

import numpy as np
import pytest

from block_wise_kv_amd import synth
from oracle import decode as od
from oracle import model as om
from tests.helpers import TOL, StepCheck, cache_kv, factor_fragile, host, rel_l2, sample_fragile

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

MODELS = {
    # the tiny fp32 model of the evaluated workloads (2 layers, d 256, 4 x 64, F 768, V 2048)
    "tiny_f32": synth.TINY,
    "tiny_bf16": dataclasses.replace(synth.TINY, dtype="bf16"),
    # grouped-query attention with 128-dim heads (4 query heads per kv head)
    "gqa_bf16": synth.ModelShape(2, 512, 8, 2, 128, 1024, 4096, 4095, "bf16", logit_scale=12.0),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_built = {}


def build(name, max_seq=128, batch=1):
    from block_wise_kv_amd.runtime import GPUCache, GPUModel
    key = (name, max_seq, batch)
    if key not in _built:
        shape = MODELS[name]
        w = synth.make_weights(shape, seed=7, norm_gain_std=0.1, threads=4)
        gm = GPUModel(shape, w, max_seq_len=max_seq)
        gc = GPUCache(gm, batch, max_seq)
        _built[key] = (shape, om.Model(shape, w), gm, gc)
    return _built[key]


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def gpu_step(gm, gc, shape, x, flags, rows, s, B, tau, t, T, factor=0.0, topk=0, sampling=False,
             seed=0):
    """Runs one forward (refresh if rows is None) and the fused unmask on
    copies of x / flags; returns hidden, logits, conf, argmax, committed, counts."""
    from block_wise_kv_amd import fdllm as F
    N = x.shape[-1]
    tx, tf = dev_i32(x[None]), dev_u8(flags[None])
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
                              counts, logits, factor=factor, topk=topk, sampling=sampling, seed=seed)
    torch.cuda.synchronize()
    committed = (flags[s:s + B] == 1) & (tf.cpu().numpy()[0, s:s + B] == 0)
    return (host(hidden)[0], logits.cpu().numpy()[0], conf.cpu().numpy()[0], am.cpu().numpy()[0],
            committed, counts.cpu().numpy()[0], tx.cpu().numpy()[0])


@pytest.mark.parametrize("name", list(MODELS))
@pytest.mark.parametrize("prompt_len", [32, 20])
def test_refresh_matches_oracle(name, prompt_len):
    shape, om_, gm, gc = build(name)
    L, B = 64, 16
    N = prompt_len + L
    prompt = synth.make_prompt(shape, prompt_len, seed=11)[0]
    x, flags = synth.initial_sequence(shape, prompt[None], L)
    x, flags = x[0].copy(), flags[0].copy()
    x[prompt_len + 3] = 5  # some positions already decoded
    flags[prompt_len + 3] = 0
    s = prompt_len
    hf, cache, attn = om_.forward_full(x.astype(np.int64), keep_attn_layers=(0, shape.n_layers - 1))
    hid, logits, conf, am, com, counts, _ = gpu_step(gm, gc, shape, x, flags, None, s, B, 0.9, 0, 16)
    tol = TOL[shape.dtype]
    # K and V of every layer and row
    for l in range(shape.n_layers):
        k, v = cache_kv(gc.mem, shape, 1, 128, l)
        kr = np.transpose(cache[l][0], (1, 0, 2))
        vr = np.transpose(cache[l][1], (1, 0, 2))
        ek, ev = rel_l2(k[0, :, :N], kr), rel_l2(v[0, :, :N], vr)
        print(f"{name} P={prompt_len} layer {l}: K {ek:.2e} V {ev:.2e}")
        assert ek < tol and ev < tol
    eh = rel_l2(hid, hf[s:s + B])
    z = om_.logits(hf[s:s + B])
    ez = rel_l2(logits, z)
    print(f"{name} P={prompt_len}: hidden {eh:.2e} logits {ez:.2e}")
    assert eh < tol and ez < tol
    rec = od.Step(0, 0, "refresh", (0, N), x, flags, z, *od.confidence(z), 1,
                  s + od.select(od.confidence(z)[0], flags[s:s + B], 0.9), {})
    StepCheck(0.9, dtype=shape.dtype)(rec, s, am, conf, com)


@pytest.mark.parametrize("name", list(MODELS))
@pytest.mark.parametrize("dual", [False, True])
def test_cached_forward_matches_oracle(name, dual):
    """After a refresh, the sequence moves on (tokens committed in the block
    and earlier); a cached forward over [s, N) or [s, e) must match the
    oracle's cached forward over the same stale cache."""
    shape, om_, gm, gc = build(name)
    P, L, B = 32, 64, 16
    N = P + L
    prompt = synth.make_prompt(shape, P, seed=12)[0]
    x, flags = synth.initial_sequence(shape, prompt[None], L)
    x, flags = x[0].copy(), flags[0].copy()
    s = P + B  # second block
    x[P:s] = np.arange(B) + 3
    flags[P:s] = 0
    _, cache, _ = om_.forward_full(x.astype(np.int64))
    gpu_step(gm, gc, shape, x, flags, None, s, B, 0.9, 0, 16)   # GPU refresh with the same x
    x2, f2 = x.copy(), flags.copy()
    x2[s + 1], x2[s + 7] = 9, 11
    f2[s + 1] = f2[s + 7] = 0
    r1 = s + B if dual else N
    hr, attn = om_.forward_cached(x2.astype(np.int64), s, r1, cache)
    z = om_.logits(hr[:B])
    hid, logits, conf, am, com, counts, _ = gpu_step(gm, gc, shape, x2, f2, (s, r1), s, B, 0.9, 1, 16)
    tol = TOL[shape.dtype]
    eh, ez = rel_l2(hid, hr[:B]), rel_l2(logits, z)
    print(f"{name} dual={dual}: hidden {eh:.2e} logits {ez:.2e}")
    assert eh < tol and ez < tol
    c, a = od.confidence(z)
    rec = od.Step(1, 1, "cached", (s, r1), x2, f2, z, c, a, 1, s + od.select(c, f2[s:s + B], 0.9), {})
    StepCheck(0.9, dtype=shape.dtype)(rec, s, am, conf, com)


def teacher_forced(name, settings, prompt_len, tau=None):
    """Runs the oracle decode and replays every step on the GPU from the
    oracle's state; compares logits, ids and selections step by step."""
    shape, om_, gm, gc = build(name)
    tau = settings.threshold if tau is None else tau
    prompt = synth.make_prompt(shape, prompt_len, seed=13)[0]
    _, _, steps = od.decode(om_, prompt, settings)
    K = settings.gen_length // settings.block_size
    T = settings.steps // K
    chk = StepCheck(tau, settings.factor, settings.topk, settings.seed if settings.sampling else None,
                    dtype=shape.dtype)
    worst = 0.0
    for rec in steps:
        s = prompt_len + rec.block * settings.block_size
        rows = None if rec.kind in ("refresh", "full") else rec.rows
        hid, logits, conf, am, com, counts, xg = gpu_step(
            gm, gc, shape, rec.x_before.astype(np.int32), rec.flags_before, rows, s,
            settings.block_size, tau, rec.step, T, settings.factor, settings.topk, settings.sampling,
            settings.seed)
        e = rel_l2(logits, rec.z)
        worst = max(worst, e)
        assert e < TOL[shape.dtype], (rec.block, rec.step, e)
        chk(rec, s, am, conf, com)
        if settings.sampling:  # committed tokens are the draws, bar near-ties
            for j in rec.selected - s:
                if not sample_fragile(rec.z[j], settings.seed, 0, s + j, rec.step):
                    assert xg[s + j] == rec.sampled[j], (rec.block, rec.step, j)
                    chk.compared += 1
    print(f"{name}: {chk.steps} steps, {chk.compared} positions compared, {chk.excluded} excluded, "
          f"{chk.fallback_ties} fallback near-ties, {chk.factor_ties} factor near-ties, "
          f"worst logits rel L2 {worst:.2e}")
    assert chk.compared > 0
    return chk


@pytest.mark.parametrize("name", list(MODELS))
@pytest.mark.parametrize("dual", [False, True])
def test_teacher_forced_decode(name, dual):
    st = synth.DecodeSettings(32, 64, 16, 64, True, dual, 0.9)
    teacher_forced(name, st, 32)


@pytest.mark.parametrize("name", list(MODELS))
@pytest.mark.parametrize("dual", [False, True])
def test_teacher_forced_decode_factor_strategy(name, dual):
    """The factor strategy ([commentary] 3.4.3) step by step against the oracle."""
    st = synth.DecodeSettings(32, 64, 16, 64, True, dual, 0.9, factor=1.0)
    chk = teacher_forced(name, st, 32)
    assert chk.factor_ties < chk.steps


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_bf16"])
@pytest.mark.parametrize("dual", [False, True])
def test_teacher_forced_decode_refresh_interval(name, dual):
    """Refresh interval 3 ([commentary] Table 10's policy): the oracle's
    trajectory has cache rebuilds at block steps 0, 3, 6, ...; every step is
    replayed on the GPU (rebuild or cached forward, as the oracle ran it)."""
    st = synth.DecodeSettings(32, 64, 16, 64, True, dual, 1.5, refresh_interval=3)
    chk = teacher_forced(name, st, 32)
    assert chk.steps == 64


def test_decode_end_to_end_tiny_refresh_interval():
    """fdllm_decode with refresh interval 3 and one token per step (tau > 1,
    so every block takes exactly T = 16 steps): 6 rebuilds per block, the
    rest cached forwards, and the oracle's tokens up to the first near-tie."""
    import dataclasses
    from block_wise_kv_amd import fdllm as F
    from block_wise_kv_amd.runtime import decode_params
    wl = synth.WORKLOADS["tiny_prefix"]
    st = dataclasses.replace(wl.decode, threshold=1.5, refresh_interval=3)
    shape, om_, gm, gc = build("tiny_f32")
    prompt = synth.make_prompt(shape, st.prompt_len, seed=wl.seed_p)[0]
    xo, _, steps = od.decode(om_, prompt, st)
    x, flags = synth.initial_sequence(shape, prompt[None], st.gen_length)
    tx, tf = dev_i32(x), dev_u8(flags)
    K = st.gen_length // st.block_size
    stats = F.fdllm_decode(gm.handle, gc.handle, tx, tf, 1, st.prompt_len, decode_params(st)).as_dict(K)
    torch.cuda.synchronize()
    assert not tf.cpu().numpy().any()
    assert stats["steps_per_block"] == [16] * K and stats["nfe"] == 16 * K
    assert stats["refreshes"] == 6 * K and stats["cached_steps"] == 10 * K
    assert stats["refreshes"] == sum(r.kind == "refresh" for r in steps)
    ties = [r for r in steps if np.any(od.top2_prob_gap(r.z) < 1e-3)]
    print("gpu stats", stats, "near-tie steps", len(ties))
    if not ties:
        np.testing.assert_array_equal(tx.cpu().numpy()[0], xo)


@pytest.mark.parametrize("name", list(MODELS))
def test_teacher_forced_decode_topk(name):
    """Fixed top-K = 3 step by step against the oracle (16-position blocks:
    five steps of three, then the last one)."""
    st = synth.DecodeSettings(32, 64, 16, 64, True, False, 0.9, topk=3)
    chk = teacher_forced(name, st, 32)
    assert chk.steps == 4 * 6


@pytest.mark.parametrize("name", list(MODELS))
@pytest.mark.parametrize("dual", [False, True])
def test_teacher_forced_decode_sampling(name, dual):
    """Stochastic tau-leaping ([commentary] 3.4.1) step by step against the
    oracle: identical fill decisions, identical draws bar near-ties."""
    st = synth.DecodeSettings(32, 64, 16, 64, True, dual, 0.9, sampling=True, seed=4242)
    teacher_forced(name, st, 32)


def test_decode_end_to_end_tiny_sampling():
    """fdllm_decode with tau-leaping: the fill decisions depend on the draws
    alone, so the step schedule (forwards, steps per block) equals the
    oracle's exactly; the tokens equal it when no draw is a near-tie."""
    import dataclasses
    from block_wise_kv_amd import fdllm as F
    from block_wise_kv_amd.runtime import decode_params
    wl = synth.WORKLOADS["tiny_prefix"]
    st = dataclasses.replace(wl.decode, sampling=True, seed=2024)
    shape, om_, gm, gc = build("tiny_f32")
    prompt = synth.make_prompt(shape, st.prompt_len, seed=wl.seed_p)[0]
    xo, _, steps = od.decode(om_, prompt, st)
    x, flags = synth.initial_sequence(shape, prompt[None], st.gen_length)
    tx, tf = dev_i32(x), dev_u8(flags)
    K = st.gen_length // st.block_size
    stats = F.fdllm_decode(gm.handle, gc.handle, tx, tf, 1, st.prompt_len, decode_params(st)).as_dict(K)
    torch.cuda.synchronize()
    assert not tf.cpu().numpy().any()
    per_block = [sum(1 for r in steps if r.block == k) for k in range(K)]
    assert stats["steps_per_block"] == per_block and stats["nfe"] == len(steps)
    B = st.block_size
    fragile = [r for r in steps for j in (r.selected - (st.prompt_len + r.block * B))
               if sample_fragile(r.z[j], st.seed, 0, st.prompt_len + r.block * B + j, r.step)]
    print("gpu stats", stats, "fragile draws", len(fragile))
    if not fragile:
        np.testing.assert_array_equal(tx.cpu().numpy()[0], xo)


def test_teacher_forced_vanilla_and_ragged():
    st = synth.DecodeSettings(20, 32, 8, 32, False, False, 0.9)
    teacher_forced("tiny_f32", st, 20)


def test_decode_end_to_end_tiny():
    """fdllm_decode on the tiny fp32 workload (prompt 32, gen 64, block 16,
    steps 64, PrefixCache, tau 0.9) reproduces the oracle's tokens; if a
    near-tie occurs the trajectories may legitimately part, which the
    teacher-forced tests cover, so the comparison stops at the first step
    the oracle flags as a near-tie."""
    from block_wise_kv_amd import fdllm as F
    from block_wise_kv_amd.runtime import decode_params
    wl = synth.WORKLOADS["tiny_prefix"]
    shape, om_, gm, gc = build("tiny_f32")
    prompt = synth.make_prompt(shape, wl.decode.prompt_len, seed=wl.seed_p)[0]
    xo, _, steps = od.decode(om_, prompt, wl.decode)
    x, flags = synth.initial_sequence(shape, prompt[None], wl.decode.gen_length)
    tx, tf = dev_i32(x), dev_u8(flags)
    stats = F.fdllm_decode(gm.handle, gc.handle, tx, tf, 1, wl.decode.prompt_len,
                           decode_params(wl.decode)).as_dict(4)
    torch.cuda.synchronize()
    xg = tx.cpu().numpy()[0]
    assert not tf.cpu().numpy().any()
    assert stats["committed"] == wl.decode.gen_length
    assert stats["nfe"] >= 4 and stats["max_steps_block"] <= 16
    ties = [r for r in steps if np.any((np.abs(r.c - 0.9) < 1e-3) | (od.top2_prob_gap(r.z) < 1e-3))]
    print("oracle steps", len(steps), "gpu stats", stats, "near-tie steps", len(ties))
    assert sum(stats["commits_per_step"]) == wl.decode.gen_length
    assert len(stats["commits_per_step"]) == stats["nfe"] and min(stats["commits_per_step"]) >= 1
    if not ties:
        np.testing.assert_array_equal(xg, xo)
        assert stats["nfe"] == len(steps)
        # the oracle's commit count of every step, in decode order
        assert stats["commits_per_step"] == [len(r.selected) for r in steps]


def gpu_batch_step(gm, gc, shape, x, flags, rows, s, B, tau, t, T, factor=0.0):
    """gpu_step for a batch: x, flags [b][N]. Returns logits [b][B][V],
    conf, argmax [b][B], committed [b][B] and counts [b][2]."""
    from block_wise_kv_amd import fdllm as F
    b, N = x.shape
    tx, tf = dev_i32(x), dev_u8(flags)
    hidden = torch.empty(b, B, shape.d_model, dtype=torch.float32, device="cuda")
    if rows is None:
        F.fdllm_cache_refresh(gm.handle, gc.handle, tx, b, N, s, B, hidden)
    else:
        F.fdllm_block_forward(gm.handle, gc.handle, tx, b, N, rows[0], rows[1], s, B, hidden)
    logits = torch.empty(b, B, shape.vocab, device="cuda")
    conf = torch.empty(b, B, device="cuda")
    am = torch.empty(b, B, dtype=torch.int32, device="cuda")
    counts = torch.empty(b, 2, dtype=torch.int32, device="cuda")
    F.fdllm_confidence_unmask(gm.handle, gc.handle, hidden, tx, tf, b, N, s, B, tau, t, T, conf, am,
                              counts, logits, factor=factor)
    torch.cuda.synchronize()
    committed = (flags[:, s:s + B] == 1) & (tf.cpu().numpy()[:, s:s + B] == 0)
    return logits.cpu().numpy(), conf.cpu().numpy(), am.cpu().numpy(), committed, counts.cpu().numpy()


@pytest.mark.parametrize("dual", [False, True])
def test_teacher_forced_batch_lockstep(dual):
    """Three sequences stepped together the way fdllm_decode runs a batch
    (block by block, every sequence forwarded at every step until the
    slowest has finished the block). Each step feeds every sequence its own
    oracle state; sequences with oracle steps left are compared with the
    oracle step by step, sequences already done with the block must commit
    nothing."""
    import dataclasses
    b, P = 3, 32
    st = dataclasses.replace(synth.WORKLOADS["tiny_prefix"].decode, dual_cache=dual, batch=b)
    shape, om_, gm, gc = build("tiny_f32", batch=b)
    prompts = synth.make_prompt(shape, P, seed=29, batch=b)
    B, L = st.block_size, st.gen_length
    K, T = L // B, st.steps // (L // B)
    N = P + L
    traj = [od.decode(om_, prompts[i], st)[2] for i in range(b)]
    by = [{(r.block, r.step): r for r in tr} for tr in traj]
    chk = StepCheck(st.threshold, dtype=shape.dtype)
    state_x = [None] * b
    state_f = [None] * b
    for k in range(K):
        s = P + k * B
        t_max = max(sum(1 for r in tr if r.block == k) for tr in traj)
        for t in range(t_max):
            x = np.zeros((b, N), np.int32)
            fl = np.zeros((b, N), np.uint8)
            for i in range(b):
                rec = by[i].get((k, t))
                if rec is not None:
                    state_x[i], state_f[i] = rec.x_before.astype(np.int32), rec.flags_before.copy()
                else:  # done with this block: its state after its last step
                    last = by[i][(k, t - 1)] if (k, t - 1) in by[i] else None
                    if last is not None:
                        xi, fi = last.x_before.astype(np.int32).copy(), last.flags_before.copy()
                        xi[last.selected] = last.a[last.selected - s]
                        fi[last.selected] = 0
                        state_x[i], state_f[i] = xi, fi
                x[i], fl[i] = state_x[i], state_f[i]
            rows = None if t == 0 else ((s, s + B) if dual else (s, N))
            logits, conf, am, com, counts = gpu_batch_step(gm, gc, shape, x, fl, rows, s, B,
                                                            st.threshold, t, T)
            for i in range(b):
                rec = by[i].get((k, t))
                if rec is None:
                    assert not com[i].any() and counts[i, 0] == 0, (k, t, i)
                    continue
                assert rel_l2(logits[i], rec.z) < TOL[shape.dtype], (k, t, i)
                chk(rec, s, am[i], conf[i], com[i])
    print(f"batch lockstep: {chk.steps} sequence-steps, {chk.compared} positions compared, "
          f"{chk.excluded} excluded, {chk.fallback_ties} fallback near-ties")
    assert chk.compared > 0


def test_decode_end_to_end_tiny_batch():
    """One fdllm_decode call over a batch of four where sequences 0 and 2
    share a prompt: every position is committed, the counters add up, and
    the two equal prompts decode to the same tokens (rows of a batch are
    computed independently of their place in it)."""
    import dataclasses
    from block_wise_kv_amd import fdllm as F
    from block_wise_kv_amd.runtime import decode_params
    b = 4
    st = dataclasses.replace(synth.WORKLOADS["tiny_prefix"].decode, batch=b)
    shape, om_, gm, gc = build("tiny_f32", batch=b)
    prompts = synth.make_prompt(shape, st.prompt_len, seed=29, batch=b)
    prompts[2] = prompts[0]
    x, flags = synth.initial_sequence(shape, prompts, st.gen_length)
    tx, tf = dev_i32(x), dev_u8(flags)
    K = st.gen_length // st.block_size
    T = st.steps // K
    stats = F.fdllm_decode(gm.handle, gc.handle, tx, tf, b, st.prompt_len, decode_params(st)).as_dict(K)
    torch.cuda.synchronize()
    xg = tx.cpu().numpy()
    assert not tf.cpu().numpy().any()
    assert stats["committed"] == b * st.gen_length
    assert stats["nfe"] == sum(stats["steps_per_block"]) and all(1 <= n <= T for n in stats["steps_per_block"])
    np.testing.assert_array_equal(xg[:, :st.prompt_len], prompts)
    np.testing.assert_array_equal(xg[0], xg[2])
    assert ((xg >= 0) & (xg < shape.vocab)).all()
    print("gpu stats", stats)


def test_decode_end_to_end_tiny_factor_strategy():
    """fdllm_decode with the factor strategy (f = 1) on the tiny fp32 workload
    reproduces the oracle's tokens up to the first near-tie step."""
    from block_wise_kv_amd import fdllm as F
    from block_wise_kv_amd.runtime import decode_params
    wl = synth.WORKLOADS["tiny_prefix"]
    st = dataclasses.replace(wl.decode, factor=1.0)
    shape, om_, gm, gc = build("tiny_f32")
    prompt = synth.make_prompt(shape, st.prompt_len, seed=wl.seed_p)[0]
    xo, _, steps = od.decode(om_, prompt, st)
    x, flags = synth.initial_sequence(shape, prompt[None], st.gen_length)
    tx, tf = dev_i32(x), dev_u8(flags)
    stats = F.fdllm_decode(gm.handle, gc.handle, tx, tf, 1, st.prompt_len, decode_params(st)).as_dict(4)
    torch.cuda.synchronize()
    assert not tf.cpu().numpy().any()
    assert stats["committed"] == st.gen_length
    B = st.block_size
    fragile = [r for r in steps
               if np.any(od.top2_prob_gap(r.z) < 1e-3)
               or factor_fragile(r.c[r.flags_before[st.prompt_len + r.block * B:][:B] != 0], 1.0,
                                 r.selected.size)]
    print("oracle steps", len(steps), "gpu stats", stats, "fragile steps", len(fragile))
    if not fragile:
        np.testing.assert_array_equal(tx.cpu().numpy()[0], xo)
        assert stats["nfe"] == len(steps)


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_bf16"])
def test_refresh_long_sequence(name):
    """A 320-row refresh and a 288-row PrefixCache forward: the tall GEMM
    tiles (up to 256 rows, with a ragged last tile) against the oracle."""
    shape, om_, gm, gc = build(name, max_seq=320)
    P, L, B = 256, 64, 16
    N = P + L
    prompt = synth.make_prompt(shape, P, seed=17)[0]
    x, flags = synth.initial_sequence(shape, prompt[None], L)
    x, flags = x[0].copy(), flags[0].copy()
    hf, cache, _ = om_.forward_full(x.astype(np.int64))
    hid, logits, conf, am, com, counts, _ = gpu_step(gm, gc, shape, x, flags, None, P, B, 0.9, 0, 16)
    tol = TOL[shape.dtype]
    z = om_.logits(hf[P:P + B])
    for l in range(shape.n_layers):
        k, v = cache_kv(gc.mem, shape, 1, 320, l)
        assert rel_l2(k[0, :, :N], np.transpose(cache[l][0], (1, 0, 2))) < tol
        assert rel_l2(v[0, :, :N], np.transpose(cache[l][1], (1, 0, 2))) < tol
    ez = rel_l2(logits, z)
    assert ez < tol, ez
    x2, f2 = x.copy(), flags.copy()
    x2[P + 2] = 4
    f2[P + 2] = 0
    s = P - 32  # rows [224, 320): a 96-row cached forward
    hr, _ = om_.forward_cached(x2.astype(np.int64), P, N, cache)
    hid2, logits2, *_ = gpu_step(gm, gc, shape, x2, f2, (P, N), P, B, 0.9, 1, 16)
    e2 = rel_l2(logits2, om_.logits(hr[:B]))
    print(f"{name} long: refresh logits {ez:.2e}, cached logits {e2:.2e}")
    assert e2 < tol


def test_hidden_alignment_is_checked():
    """d_hidden_blk must be 16-byte aligned (the final norm writes and the LM
    head reads it in 16-byte pieces): a pointer 4 bytes in is rejected with
    EINVAL by every call that takes it, before any kernel runs."""
    from block_wise_kv_amd import fdllm as F
    shape, _, gm, gc = build("tiny_bf16")
    P, L, B = 32, 64, 16
    N = P + L
    prompt = synth.make_prompt(shape, P, seed=3)[0]
    x, flags = synth.initial_sequence(shape, prompt[None], L)
    tx, tf = dev_i32(x), dev_u8(flags)
    buf = torch.zeros(B * shape.d_model + 4, dtype=torch.float32, device="cuda")
    off = buf[1:]  # 4 bytes past a 256-byte-aligned allocation
    assert off.data_ptr() % 16 == 4
    calls = [
        lambda: F.fdllm_cache_refresh(gm.handle, gc.handle, tx, 1, N, P, B, off),
        lambda: F.fdllm_block_forward(gm.handle, gc.handle, tx, 1, N, P, N, P, B, off),
        lambda: F.fdllm_confidence_unmask(gm.handle, gc.handle, off, tx, tf, 1, N, P, B, 0.9, 0, 16),
    ]
    for call in calls:
        with pytest.raises(F.FdllmError) as err:
            call()
        assert err.value.status == F.EINVAL and "16-byte aligned" in str(err.value)
    torch.cuda.synchronize()
    # the aligned buffer is accepted
    F.fdllm_cache_refresh(gm.handle, gc.handle, tx, 1, N, P, B, buf[:B * shape.d_model])
    torch.cuda.synchronize()


def test_workspace_bytes_is_the_arena_past_the_kv_blocks():
    """fdllm_workspace_bytes = fdllm_cache_bytes minus the K/V blocks (every
    layer's K and V, 256-byte aligned, first in the arena)."""
    from block_wise_kv_amd import fdllm as F
    from tests.helpers import cache_layout
    for name, max_seq, batch in (("tiny_f32", 96, 1), ("gqa_bf16", 128, 3)):
        shape, _, gm, _ = build(name, max_seq=max_seq, batch=batch)
        total = F.fdllm_cache_bytes(gm.handle, batch, max_seq)
        ws = F.fdllm_workspace_bytes(gm.handle, batch, max_seq)
        _, offs = cache_layout(shape, batch, max_seq)
        kb_al = -(-offs[0][2] // 256) * 256
        assert total - ws == 2 * shape.n_layers * kb_al
        assert 0 < ws < total
