"""Confidence-aware parallel unmasking and block-wise decoding, float64.

Follows [commentary] §3.2 "Big-Picture Architecture" (information flow),
§3.4.2 "Block-Wise Generation Scheme", "PrefixCache", "DualCache",
§3.4.3 "From Theorem to Practice: Threshold Strategy" and "Factor
Strategy", and §3.4.4 "The Integrated Algorithm", and the decode parameters of [README] "Parameter
descriptions" (gen_length, steps, block_size, use_cache, dual cache,
threshold).

Readings where the pages are silent or disagree:

* ">= tau": §3.4.3 states the rule as c_i >= tau and its code snippet uses
  >=; other sentences say "exceeds". This uses >=.
* Blocks are numbered from 0; block k covers [P + kB, P + (k+1)B).
* The cache is refreshed by a full forward at the start of every block
  (block 0 included), whose block logits drive that block's first step;
  no forward runs after the last block. §3.4.4 places the update "fused with
  the last decoding step" of a block and the initialisation "fused with the
  first decoding step"; a full forward at block start is both.
* T = steps / K denoising steps per block (steps counts the whole answer).
  Every step commits at least one token; when fewer than T - t steps would
  be left for the |U| still-masked positions, the step commits at least
  ceil(|U| / (T - t)) so the block always finishes within T steps. With
  T >= B (all evaluated settings) this is the plain "at least one" rule.
* Softmax and argmax run over the whole vocabulary (the [MASK] id included);
  whether a position is still masked is its flag, not its token id.
* Ties: the vocabulary argmax takes the lowest id; when positions are picked
  by confidence, equal confidences go to the lower position.
* Refresh interval ([commentary] Table 10, "updating the cache every r
  steps rather than per-block"): with r > 0 the cache is also rebuilt by a
  full forward at every step t of a block with t % r == 0; step 0 of a block
  always rebuilds it. r = 0 (or r >= T) is the per-block scheme.
* Stochastic sampling (``sampling``): the tau-leaping step of
  ``oracle.sampling`` replaces the confidence rule (its readings are listed
  there); the committed ids are the sampled tokens, not the argmax.
* Fixed top-K (the LLaDA baseline of [commentary] §2 "Related Work" /
  §3.4.3 "Why factor-based over threshold-based"): the K most confident
  masked positions each step (all of them when fewer are masked), at least
  the quota.
* Factor strategy: the condition is the strict (n+1)(1 - c_(n)) < f of the
  strategy's step 2 (the theorem's own bound is non-strict at f = 1). The
  left side grows with n, so the n meeting it form a prefix 1..n*. Like the
  threshold rule it commits at least the quota (at least one token).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from . import sampling as smp


def confidence(z: np.ndarray):
    """c_i = max_v softmax(z_i)_v = 1 / sum_v exp(z_iv - max_v z_iv); a_i = argmax.

    [commentary] §3.4.3 "The Core Idea": the confidence of a masked
    position is the largest probability the model gives any vocabulary
    token. z is [rows][V]; returns (c float64 [rows], a int64 [rows]).
    """
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=-1)
    a = np.argmax(z, axis=-1)  # first occurrence = lowest id
    c = 1.0 / np.sum(np.exp(z - m[:, None]), axis=-1)
    return c, a


def top2_prob_gap(z: np.ndarray) -> np.ndarray:
    """p_(1) - p_(2) of softmax(z_i), per row (used to flag near-ties)."""
    z = np.asarray(z, dtype=np.float64)
    zs = np.sort(z, axis=-1)
    m = zs[:, -1]
    s = np.sum(np.exp(z - m[:, None]), axis=-1)
    return (1.0 - np.exp(zs[:, -2] - m)) / s


def select(c: np.ndarray, masked: np.ndarray, tau: float, quota: int = 1) -> np.ndarray:
    """Positions to commit at one step (indices into the block).

    [commentary] §3.4.3 "Threshold Strategy": every masked position with
    c_i >= tau is unmasked; if none is, the single most confident one is
    (progress guarantee). ``quota`` generalises the guarantee to "at least
    quota" (see the module docstring); quota = 1 is the pages' rule.
    """
    masked_idx = np.flatnonzero(np.asarray(masked) != 0)
    if masked_idx.size == 0:
        return masked_idx
    chosen = masked_idx[c[masked_idx] >= tau]
    if chosen.size >= quota:
        return chosen
    # highest confidence first, lower position first among equal confidences
    order = sorted(masked_idx.tolist(), key=lambda i: (-c[i], i))
    return np.array(sorted(order[:quota]), dtype=np.int64)


def select_factor(c: np.ndarray, masked: np.ndarray, f: float, quota: int = 1) -> np.ndarray:
    """Positions to commit under [commentary] §3.4.3 "From Theorem to
    Practice: Factor Strategy": order the masked positions by confidence,
    c_(1) >= c_(2) >= ... (equal confidences: lower position first), take
    the largest n with (n + 1) * (1 - c_(n)) < f and commit the n most
    confident; if no n qualifies, the most confident one. ``quota`` raises
    the minimum as in ``select``.
    """
    masked_idx = np.flatnonzero(np.asarray(masked) != 0)
    if masked_idx.size == 0:
        return masked_idx
    order = sorted(masked_idx.tolist(), key=lambda i: (-c[i], i))
    n_star = 0
    for n in range(1, len(order) + 1):
        if (n + 1) * (1.0 - c[order[n - 1]]) < f:
            n_star = n
    return np.array(sorted(order[:max(n_star, quota)]), dtype=np.int64)


def select_topk(c: np.ndarray, masked: np.ndarray, k: int, quota: int = 1) -> np.ndarray:
    """Fixed top-K: the max(K, quota) most confident masked positions
    (all of them when fewer are masked); equal confidences go to the lower
    position."""
    masked_idx = np.flatnonzero(np.asarray(masked) != 0)
    order = sorted(masked_idx.tolist(), key=lambda i: (-c[i], i))
    return np.array(sorted(order[:max(k, quota)]), dtype=np.int64)


def select_rule(c: np.ndarray, masked: np.ndarray, tau: float, quota: int = 1,
                factor: float = 0.0, topk: int = 0) -> np.ndarray:
    """Fixed top-K when topk > 0, else the factor rule when factor > 0,
    else the threshold rule."""
    if topk > 0:
        return select_topk(c, masked, topk, quota)
    if factor > 0:
        return select_factor(c, masked, factor, quota)
    return select(c, masked, tau, quota)


@dataclasses.dataclass
class Step:
    block: int
    step: int           # 0-based step within the block
    kind: str           # "refresh" (cache rebuilt), "cached" or "full" (no cache)
    rows: tuple         # rows [r0, r1) whose hidden states were computed
    x_before: np.ndarray
    flags_before: np.ndarray
    z: np.ndarray       # logits of the block rows [B][V]
    c: np.ndarray
    a: np.ndarray
    quota: int
    selected: np.ndarray  # absolute positions committed at this step
    attn: dict          # layer -> attention output of the block rows [B][Hq][D]
    sampled: np.ndarray = None  # with sampling: the drawn token per block position (-1 if not masked)


def validate(shape, settings, prompt: np.ndarray):
    """Parameter checks of the decode call (raises ValueError)."""
    L, B, steps = settings.gen_length, settings.block_size, settings.steps
    if L <= 0 or B <= 0 or L % B:
        raise ValueError("gen_length must be a positive multiple of block_size")
    K = L // B
    if steps <= 0 or steps % K:
        raise ValueError("steps must be a positive multiple of gen_length / block_size")
    if settings.dual_cache and not settings.use_cache:
        raise ValueError("dual cache requires use_cache")
    if not math.isfinite(settings.threshold):
        raise ValueError("threshold must be finite")
    if not (math.isfinite(settings.factor) and settings.factor >= 0):
        raise ValueError("factor must be finite and >= 0")
    if settings.refresh_interval < 0:
        raise ValueError("refresh_interval must be >= 0")
    if settings.topk < 0:
        raise ValueError("topk must be >= 0")
    p = np.asarray(prompt)
    if p.ndim != 1 or np.any(p < 0) or np.any(p >= shape.vocab) or np.any(p == shape.mask_id):
        raise ValueError("prompt ids must lie in [0, vocab) and differ from the mask id")
    return K, steps // K


def decode(model, prompt: np.ndarray, settings, keep_attn_layers=(), on_step=None,
           teacher=None, start=None):
    """Block-wise decoding of one sequence (Algorithm 1 as described in
    [commentary] §3.4.4).

    x = [prompt; MASK * L] with flags marking the L generated positions
    ([commentary] §3.2, "Initialization"). Each block k runs up to T steps:
    step 0 is a full forward (with use_cache it also rebuilds the cache),
    later steps are cached forwards over rows [s, N) (PrefixCache) or
    [s, e) (DualCache), or full forwards when use_cache is off (vanilla
    decoding). Each step scores the block's masked positions, selects and
    commits; the block ends early once it has no masked position.

    ``on_step(Step)`` sees every step (default: steps are collected and
    returned). ``teacher``, if given, is a callable (block, step, x, flags)
    -> (x, flags) that replaces the state before each step (teacher forcing
    of another trajectory). ``start`` = (k0, x, flags) begins at block k0
    from that state: every block starts with a full forward, so no other
    state crosses a block boundary and this continues an interrupted decode
    exactly.

    Returns (x [N] int64, flags [N], list of Step or None).
    """
    s_ = model.s
    prompt = np.asarray(prompt).reshape(-1)
    K, T = validate(s_, settings, prompt)
    P, L, B = prompt.size, settings.gen_length, settings.block_size
    N = P + L
    x = np.full(N, s_.mask_id, dtype=np.int64)
    x[:P] = prompt
    flags = np.zeros(N, dtype=np.uint8)
    flags[P:] = 1
    k0 = 0
    if start is not None:
        k0 = int(start[0])
        x = np.array(start[1], dtype=np.int64, copy=True)
        flags = np.array(start[2], dtype=np.uint8, copy=True)
    steps_out = [] if on_step is None else None
    cache = None
    for k in range(k0, K):
        s, e = P + k * B, P + (k + 1) * B
        t = 0
        while True:
            if teacher is not None:
                x, flags = teacher(k, t, x.copy(), flags.copy())
            r = settings.refresh_interval
            if t == 0 or not settings.use_cache or (r > 0 and t % r == 0):
                hf, new_cache, attn = model.forward_full(x, keep_attn_layers)
                if settings.use_cache:
                    cache = new_cache
                h_blk = hf[s:e]
                attn_blk = {l: a[s:e] for l, a in attn.items()}
                kind = "refresh" if settings.use_cache else "full"
                rows = (0, N)
            else:
                r0, r1 = (s, e) if settings.dual_cache else (s, N)
                h_rows, attn = model.forward_cached(x, r0, r1, cache, keep_attn_layers)
                h_blk = h_rows[: e - s]
                attn_blk = {l: a[: e - s] for l, a in attn.items()}
                kind = "cached"
                rows = (r0, r1)
            z = model.logits(h_blk)
            c, a = confidence(z)
            masked = flags[s:e]
            quota = max(1, -(-int(masked.sum()) // (T - t)))
            tok = None
            if settings.sampling:
                sel, tok = smp.tau_leap_step(z, masked, s, t, T, settings.seed, 0)
                quota = 0
            else:
                sel = select_rule(c, masked, settings.threshold, quota, settings.factor, settings.topk)
            rec = Step(k, t, kind, rows, x.copy(), flags.copy(), z, c, a, quota, sel + s, attn_blk, tok)
            x[sel + s] = (a if tok is None else tok)[sel]
            flags[sel + s] = 0
            t += 1
            if on_step is None:
                steps_out.append(rec)
            else:
                on_step(rec)
            if not flags[s:e].any():
                break
            if t >= T:  # cannot happen: the quota finishes the block by step T
                raise RuntimeError("block still masked after its step budget")
    return x, flags, steps_out


def unmask_step(z: np.ndarray, ids: np.ndarray, flags: np.ndarray, tau: float, quota=1,
                factor: float = 0.0, topk: int = 0, sampling: bool = False, seed: int = 0,
                blk_start: int = 0, step: int = 0, T: int = 1):
    """One scoring + selection + commit step for a batch of blocks.

    z [b][B][V] logits of the block rows, ids [b][B] token ids, flags [b][B]
    (1 = masked). Returns (new ids, new flags, c [b][B], a [b][B],
    committed [b][B] bool, still-masked count [b]). ``quota`` is an int or
    one int per sequence. [commentary] §3.4.3 "Threshold Strategy" and the
    three-line selection snippet under "Why This Approach Is Training-Free";
    with factor > 0 the "Factor Strategy" of the same section instead; with
    sampling, the tau-leaping step of ``oracle.sampling`` for sequence i
    (key (seed, i)), block at ``blk_start``, step ``step`` of ``T``, and the
    committed ids are the sampled tokens.
    """
    z = np.asarray(z, dtype=np.float64)
    b, B, _ = z.shape
    ids = np.array(ids, dtype=np.int64, copy=True)
    flags = np.array(flags, dtype=np.uint8, copy=True)
    quotas = np.broadcast_to(np.asarray(quota, dtype=np.int64), (b,))
    c = np.empty((b, B))
    a = np.empty((b, B), dtype=np.int64)
    committed = np.zeros((b, B), dtype=bool)
    for i in range(b):
        c[i], a[i] = confidence(z[i])
        if sampling:
            sel, tok = smp.tau_leap_step(z[i], flags[i], blk_start, step, T, seed, i)
            a[i] = np.where(tok >= 0, tok, a[i])
        else:
            sel = select_rule(c[i], flags[i], tau, int(quotas[i]), factor, topk)
        ids[i, sel] = a[i, sel]
        flags[i, sel] = 0
        committed[i, sel] = True
    return ids, flags, c, a, committed, flags.sum(axis=1).astype(np.int64)
