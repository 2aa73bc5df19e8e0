"""Pins of the oracle's forward and block-wise decoding loop: invariants the
pages fix, special cases that reduce to simpler decoders, and cache no-op
cases (CPU only)."""
import dataclasses

import numpy as np
import pytest

from block_wise_kv_amd import synth
from oracle import decode as od
from oracle import model as om

SMALL = synth.ModelShape(n_layers=2, d_model=64, n_heads=4, n_kv_heads=2, head_dim=16, ffn_dim=128,
                         vocab=97, mask_id=96, dtype="f32", logit_scale=40.0)


def small_model(shape=SMALL, seed=5, gain_std=0.1):
    return om.Model(shape, synth.make_weights(shape, seed, norm_gain_std=gain_std, threads=2))


def settings(**kw):
    base = dict(prompt_len=8, gen_length=16, block_size=4, steps=16, use_cache=True,
                dual_cache=False, threshold=0.9)
    base.update(kw)
    p = base.pop("prompt_len")
    return p, synth.DecodeSettings(prompt_len=p, **base)


@pytest.fixture(scope="module")
def model():
    return small_model()


@pytest.fixture(scope="module")
def prompt():
    return synth.make_prompt(SMALL, 8, seed=3)[0]


def check_invariants(x, flags, steps, prompt, st, vocab):
    P, L, B = prompt.size, st.gen_length, st.block_size
    K, T = L // B, st.steps // (L // B)
    assert not flags.any()
    np.testing.assert_array_equal(x[:P], prompt)
    assert np.all((x >= 0) & (x < vocab))
    committed = {}
    per_block = {}
    for rec in steps:
        assert rec.selected.size >= 1                      # progress: >= 1 per step
        s = P + rec.block * B
        assert np.all((rec.selected >= s) & (rec.selected < s + B))
        assert np.all(rec.flags_before[rec.selected] == 1)  # only masked positions commit
        for pos in rec.selected:
            assert pos not in committed                     # never re-masked / re-decided
            committed[int(pos)] = int(rec.a[pos - s])
        per_block[rec.block] = per_block.get(rec.block, 0) + 1
    assert len(committed) == L                              # sum of commits = L
    for pos, tok in committed.items():
        assert x[pos] == tok
    assert all(1 <= n <= T for n in per_block.values())    # each block within its budget
    assert sorted(per_block) == list(range(K))


@pytest.mark.parametrize("dual", [False, True])
def test_decode_invariants(model, prompt, dual):
    _, st = settings(dual_cache=dual)
    x, flags, steps = od.decode(model, prompt, st)
    check_invariants(x, flags, steps, prompt, st, SMALL.vocab)
    # both branches of the selection rule occur at this logit scale
    sizes = [r.selected.size for r in steps]
    assert max(sizes) > 1 and min(sizes) == 1
    # committed ids never change between steps
    for r1, r2 in zip(steps, steps[1:]):
        done = r1.flags_before == 0
        np.testing.assert_array_equal(r2.x_before[done], r1.x_before[done])


def test_tau_above_one_commits_one_per_step(model, prompt):
    _, st = settings(threshold=1.5)
    x, flags, steps = od.decode(model, prompt, st)
    assert all(r.selected.size == 1 for r in steps)
    assert len(steps) == st.gen_length
    check_invariants(x, flags, steps, prompt, st, SMALL.vocab)


def test_tau_zero_finishes_each_block_in_one_step(model, prompt):
    _, st = settings(threshold=0.0)
    _, _, steps = od.decode(model, prompt, st)
    assert len(steps) == st.gen_length // st.block_size
    assert all(r.kind == "refresh" for r in steps)


def test_vanilla_reduction(model, prompt):
    """No cache and tau > 1: identical to a separately written decoder that
    recomputes everything and commits the single most confident masked token
    of the current block per step (LLaDA-style semi-autoregressive decoding)."""
    _, st = settings(use_cache=False, threshold=2.0)
    x, _, steps = od.decode(model, prompt, st)
    assert all(r.kind == "full" for r in steps)

    P, L, B = prompt.size, st.gen_length, st.block_size
    seq = np.concatenate([prompt, np.full(L, SMALL.mask_id)])
    known = np.zeros(P + L, bool)
    known[:P] = True
    for blk in range(L // B):
        lo, hi = P + blk * B, P + (blk + 1) * B
        while not known[lo:hi].all():
            hf, _, _ = model.forward_full(seq)
            z = model.logits(hf[lo:hi])
            p = np.exp(z - z.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            best, best_conf = None, -1.0
            for j in range(B):
                if not known[lo + j] and p[j].max() > best_conf:
                    best, best_conf = j, p[j].max()
            seq[lo + best] = int(np.argmax(p[best]))
            known[lo + best] = True
    np.testing.assert_array_equal(x, seq)


def test_block_size_one_makes_cache_a_no_op(model, prompt):
    runs = []
    for use_cache, dual in [(False, False), (True, False), (True, True)]:
        _, st = settings(block_size=1, steps=16, use_cache=use_cache, dual_cache=dual)
        runs.append(od.decode(model, prompt, st)[0])
    np.testing.assert_array_equal(runs[0], runs[1])
    np.testing.assert_array_equal(runs[0], runs[2])


def test_cached_forward_after_refresh_reproduces_refresh(prompt):
    """With x unchanged since the refresh, a cached forward (Prefix rows [s,N)
    or Dual rows [s,e)) gives the refresh's block logits (float64 storage, so
    only summation order differs). Pins row ranges, positions and cache
    assembly of the cached path."""
    shape = dataclasses.replace(SMALL, dtype="f64")
    m = small_model(shape)
    P, L = 8, 16
    x = np.concatenate([prompt, np.full(L, SMALL.mask_id)])
    x[P + 2] = 5
    hf, cache, _ = m.forward_full(x)
    for s in (P, P + 4, P + 12):
        e = s + 4
        for r0, r1 in ((s, P + L), (s, e)):
            hc, _ = m.forward_cached(x, r0, r1, cache)
            np.testing.assert_allclose(m.logits(hc[: e - s]), m.logits(hf[s:e]), rtol=1e-10, atol=1e-10)


def test_prefix_equals_dual_in_last_block(model, prompt):
    P, L, B = 8, 16, 4
    x = np.concatenate([prompt, np.random.default_rng(1).integers(0, 96, L)])
    _, cache, _ = model.forward_full(x)
    x2 = x.copy()
    x2[P + 1] = 7  # state moved on since the refresh
    s = P + L - B
    h1, _ = model.forward_cached(x2, s, P + L, cache)
    h2, _ = model.forward_cached(x2, s, s + B, cache)
    np.testing.assert_array_equal(h1, h2)


def test_cache_is_used_outside_the_fresh_rows(prompt):
    """A cached step must read prefix K/V from the cache, not recompute them:
    perturbing the cache of a prefix row changes the block output, while
    perturbing the cache of a fresh row does not."""
    shape = dataclasses.replace(SMALL, dtype="f64")
    m = small_model(shape)
    x = np.concatenate([prompt, np.full(16, SMALL.mask_id)])
    _, cache, _ = m.forward_full(x)
    s, e = 12, 16
    base, _ = m.forward_cached(x, s, e, cache)
    c1 = [(k.copy(), v.copy()) for k, v in cache]
    c1[0][1][3] += 1.0        # prefix row 3, layer 0 values
    out1, _ = m.forward_cached(x, s, e, c1)
    assert np.abs(out1 - base).max() > 1e-6
    c2 = [(k.copy(), v.copy()) for k, v in cache]
    c2[0][1][13] += 1.0       # a fresh row: overwritten by the fresh values
    out2, _ = m.forward_cached(x, s, e, c2)
    np.testing.assert_array_equal(out2, base)
    c3 = [(k.copy(), v.copy()) for k, v in cache]
    c3[1][0][20] += 1.0       # a suffix row: read from cache in DualCache only
    out3, _ = m.forward_cached(x, s, e, c3)
    out4, _ = m.forward_cached(x, s, 24, c3)
    assert np.abs(out3 - base).max() > 1e-6
    np.testing.assert_allclose(out4[:4], m.forward_cached(x, s, 24, cache)[0][:4], rtol=0, atol=0)


def test_forward_is_bidirectional(model, prompt):
    x = np.concatenate([prompt, np.full(16, SMALL.mask_id)])
    h1, _, _ = model.forward_full(x)
    x2 = x.copy()
    x2[-1] = 3
    h2, _, _ = model.forward_full(x2)
    assert np.abs(h1[0] - h2[0]).max() > 1e-6   # the first row sees the last


def test_forward_translation_invariance(prompt):
    """RoPE makes attention depend on relative positions only, so shifting
    every position by the same offset leaves the forward unchanged."""
    shape = dataclasses.replace(SMALL, dtype="f64")
    m = small_model(shape)
    x = np.concatenate([prompt, np.full(16, SMALL.mask_id)])
    h0, _, _ = m.forward_full(x)
    h1, _, _ = m.forward_full(x, pos0=37)
    np.testing.assert_allclose(h1, h0, rtol=1e-9, atol=1e-9)


def test_forward_without_blocks_is_embedding_norm_head(prompt):
    """Zero output and down projections: the residual stream stays the
    embedding, so logits = scale * rmsnorm(E[x]) W_lm^T."""
    w = synth.make_weights(SMALL, 5, norm_gain_std=0.1, threads=2)
    for l in range(SMALL.n_layers):
        w[f"l{l}.wo"][:] = 0
        w[f"l{l}.w_down"][:] = 0
    m = om.Model(SMALL, w)
    x = np.concatenate([prompt, np.full(16, SMALL.mask_id)])
    hf, _, _ = m.forward_full(x)
    e = w["embed"][x].astype(np.float64)
    g = w["final_norm"].astype(np.float64)
    ref = e * g / np.sqrt((e * e).mean(1, keepdims=True) + SMALL.norm_eps)
    np.testing.assert_allclose(hf, ref, rtol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_weights(prompt):
    gqa = dataclasses.replace(SMALL, dtype="f64")
    mha = dataclasses.replace(gqa, n_kv_heads=gqa.n_heads)
    w = synth.make_weights(gqa, 8, threads=2)
    w2 = dict(w)
    grp = gqa.n_heads // gqa.n_kv_heads
    for l in range(gqa.n_layers):
        for t in ("wk", "wv"):
            m_ = w[f"l{l}.{t}"].reshape(gqa.n_kv_heads, gqa.head_dim, gqa.d_model)
            w2[f"l{l}.{t}"] = np.repeat(m_, grp, axis=0).reshape(-1, gqa.d_model)
    x = np.concatenate([prompt, np.full(16, SMALL.mask_id)])
    a, _, _ = om.Model(gqa, w).forward_full(x)
    b, _, _ = om.Model(mha, w2).forward_full(x)
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("dual", [False, True])
def test_decode_invariants_factor_strategy(model, prompt, dual):
    """The factor strategy ([commentary] 3.4.3) keeps every decoding invariant,
    and each step commits exactly the positions select_factor picks from
    that step's confidences."""
    _, st = settings(dual_cache=dual, factor=1.0)
    x, flags, steps = od.decode(model, prompt, st)
    check_invariants(x, flags, steps, prompt, st, SMALL.vocab)
    B = st.block_size
    for r in steps:
        s = prompt.size + r.block * B
        want = od.select_factor(r.c, r.flags_before[s:s + B], 1.0, r.quota) + s
        np.testing.assert_array_equal(r.selected, want)
    assert max(r.selected.size for r in steps) > 1


def test_factor_strategy_large_f_finishes_each_block_in_one_step(model, prompt):
    _, st = settings(factor=1e6)
    _, _, steps = od.decode(model, prompt, st)
    assert len(steps) == st.gen_length // st.block_size


def test_refresh_every_step_is_vanilla_decoding(model, prompt):
    """Refresh interval 1 ([commentary] Table 10's refresh policy at its
    finest): the cache is rebuilt from the current tokens at every step, so
    every step's logits come from a full forward and the trajectory equals
    uncached decoding exactly (both run the same float64 forward)."""
    _, cached = settings(refresh_interval=1)
    _, vanilla = settings(use_cache=False)
    xa, _, sa = od.decode(model, prompt, cached)
    xb, _, sb = od.decode(model, prompt, vanilla)
    np.testing.assert_array_equal(xa, xb)
    assert [r.selected.tolist() for r in sa] == [r.selected.tolist() for r in sb]
    assert all(r.kind == "refresh" for r in sa)
    for ra, rb in zip(sa, sb):
        np.testing.assert_array_equal(ra.z, rb.z)


@pytest.mark.parametrize("dual", [False, True])
def test_refresh_interval_at_least_T_is_the_per_block_scheme(model, prompt, dual):
    _, per_block = settings(dual_cache=dual)
    T = per_block.steps // (per_block.gen_length // per_block.block_size)
    _, every_T = settings(dual_cache=dual, refresh_interval=T)
    xa, _, sa = od.decode(model, prompt, per_block)
    xb, _, sb = od.decode(model, prompt, every_T)
    np.testing.assert_array_equal(xa, xb)
    for ra, rb in zip(sa, sb):
        assert ra.kind == rb.kind
        np.testing.assert_array_equal(ra.z, rb.z)


@pytest.mark.parametrize("r", [2, 3])
def test_refresh_interval_rebuilds_at_multiples_of_r(model, prompt, r):
    _, st = settings(threshold=1.5, refresh_interval=r)   # one token per step: 4 steps per block
    x, flags, steps = od.decode(model, prompt, st)
    check_invariants(x, flags, steps, prompt, st, SMALL.vocab)
    for rec in steps:
        assert rec.kind == ("refresh" if rec.step % r == 0 else "cached"), (rec.block, rec.step)


def test_topk_decode(model, prompt):
    """Fixed top-K = 2: every step commits two tokens (a 4-position block in
    two steps) and the invariants hold."""
    _, st = settings(topk=2)
    x, flags, steps = od.decode(model, prompt, st)
    check_invariants(x, flags, steps, prompt, st, SMALL.vocab)
    assert all(r.selected.size == 2 for r in steps) and len(steps) == 2 * 4


@pytest.mark.parametrize("bad", [
    dict(gen_length=15), dict(steps=6), dict(use_cache=False, dual_cache=True), dict(topk=-2),
    dict(threshold=float("nan")), dict(factor=-1.0), dict(factor=float("inf")),
    dict(refresh_interval=-1),
])
def test_validation(model, prompt, bad):
    _, st = settings(**bad)
    with pytest.raises(ValueError):
        od.decode(model, prompt, st)


def test_validation_prompt_ids(model):
    _, st = settings()
    with pytest.raises(ValueError):
        od.decode(model, np.array([1, 2, SMALL.mask_id, 3, 4, 5, 6, 7]), st)
    with pytest.raises(ValueError):
        od.decode(model, np.array([1, 2, 97, 3, 4, 5, 6, 7]), st)


def test_quota_finishes_block_when_budget_is_short(model, prompt):
    _, st = settings(steps=8, threshold=1.5)   # T = 2 steps for B = 4 positions
    x, flags, steps = od.decode(model, prompt, st)
    check_invariants(x, flags, steps, prompt, st, SMALL.vocab)
    assert all(r.selected.size == 2 for r in steps)
