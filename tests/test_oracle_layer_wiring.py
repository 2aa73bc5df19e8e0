"""Pins the oracle's layer wiring against an independently written forward in
torch's functional ops (CPU, float64): RMSNorm via F.rms_norm, rotate-half
RoPE written as a complex rotation, attention via scaled_dot_product_attention
with repeat_interleave for grouped-query heads, SwiGLU as
F.silu(u W_gate^T) * (u W_up^T), and the two residual adds of a pre-norm layer.
A swapped gate/up pair, a misplaced norm, a dropped residual or a RoPE on the
wrong operand changes these outputs far beyond the tolerance.

The layer follows the model shapes the method is evaluated on (pre-norm
RMSNorm, RoPE, SwiGLU FFN, untied LM head); [commentary] 3.4.2 "Why Standard
KV Caching Fails" fixes the bidirectional attention over every position."""
import dataclasses

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from block_wise_kv_amd import synth
from oracle import model as om

SHAPE = synth.ModelShape(2, 64, 4, 2, 16, 96, 53, 52, "f64", logit_scale=3.0)


def weights(shape, seed=3):
    return synth.make_weights(shape, seed, std=0.2, norm_gain_std=0.2, threads=2)


def T(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def rope(x, pos, theta):
    """x [rows][heads][D]: entries (i, i + D/2) as the complex number
    x_i + j x_{i+D/2}, turned by the angle pos * theta^(-2i/D)."""
    d = x.shape[-1]
    z = torch.complex(x[..., : d // 2], x[..., d // 2:])
    freq = theta ** (-torch.arange(d // 2, dtype=torch.float64) * 2.0 / d)
    turn = torch.polar(torch.ones(len(pos), d // 2, dtype=torch.float64),
                       torch.as_tensor(pos, dtype=torch.float64)[:, None] * freq[None, :])
    z = z * turn[:, None, :]
    return torch.cat([z.real, z.imag], dim=-1)


def layer_kv(w, s, l, h, pos):
    u = F.rms_norm(h, (s.d_model,), weight=T(w[f"l{l}.attn_norm"]), eps=s.norm_eps)
    q = F.linear(u, T(w[f"l{l}.wq"])).view(len(pos), s.n_heads, s.head_dim)
    k = F.linear(u, T(w[f"l{l}.wk"])).view(len(pos), s.n_kv_heads, s.head_dim)
    v = F.linear(u, T(w[f"l{l}.wv"])).view(len(pos), s.n_kv_heads, s.head_dim)
    return rope(q, pos, s.rope_theta), rope(k, pos, s.rope_theta), v


def layer_rest(w, s, l, h, q, k, v):
    g = s.n_heads // s.n_kv_heads
    a = F.scaled_dot_product_attention(
        q.transpose(0, 1), k.transpose(0, 1).repeat_interleave(g, dim=0),
        v.transpose(0, 1).repeat_interleave(g, dim=0), is_causal=False).transpose(0, 1)
    h = h + F.linear(a.reshape(h.shape[0], -1), T(w[f"l{l}.wo"]))
    u = F.rms_norm(h, (s.d_model,), weight=T(w[f"l{l}.ffn_norm"]), eps=s.norm_eps)
    ffn = F.silu(F.linear(u, T(w[f"l{l}.w_gate"]))) * F.linear(u, T(w[f"l{l}.w_up"]))
    return h + F.linear(ffn, T(w[f"l{l}.w_down"])), a


def torch_forward(w, s, x, rows=None, stale_x=None):
    """Final-normed hidden states and logits of `rows` (default: all) of x.
    With stale_x, keys and values of the rows outside `rows` come from a
    forward over stale_x (the approximate cache), those inside from x."""
    n = len(x)
    pos = np.arange(n)
    r = np.arange(n) if rows is None else np.arange(*rows)
    h_all = T(w["embed"])[torch.as_tensor(x)]
    h_stale = None if stale_x is None else T(w["embed"])[torch.as_tensor(stale_x)]
    h = h_all[r]
    for l in range(s.n_layers):
        q, k, v = layer_kv(w, s, l, h, r)
        if stale_x is not None:
            qs, ks, vs = layer_kv(w, s, l, h_stale, pos)
            k_all, v_all = ks.clone(), vs.clone()
            k_all[r], v_all[r] = k, v
            h_stale, _ = layer_rest(w, s, l, h_stale, qs, ks, vs)
        else:
            k_all, v_all = k, v
        h, _ = layer_rest(w, s, l, h, q, k_all, v_all)
    hf = F.rms_norm(h, (s.d_model,), weight=T(w["final_norm"]), eps=s.norm_eps)
    return hf.numpy(), (s.logit_scale * F.linear(hf, T(w["lm_head"]))).numpy()


@pytest.mark.parametrize("n_layers", [1, 2])
def test_full_forward_matches_torch_functional(n_layers):
    s = dataclasses.replace(SHAPE, n_layers=n_layers)
    w = weights(s)
    x = np.random.default_rng(1).integers(0, s.vocab, 21)
    hf, _, _ = om.Model(s, w).forward_full(x)
    ref_h, ref_z = torch_forward(w, s, x)
    np.testing.assert_allclose(hf, ref_h, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(om.Model(s, w).logits(hf), ref_z, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("rows", [(8, 21), (8, 12)])
def test_cached_forward_matches_torch_functional(rows):
    """PrefixCache rows [s, N) and DualCache rows [s, e) over a cache built
    from an older sequence."""
    w = weights(SHAPE)
    g = np.random.default_rng(2)
    stale = g.integers(0, SHAPE.vocab, 21)
    x = stale.copy()
    x[[2, 9, 10, 17]] = g.integers(0, SHAPE.vocab, 4)  # the sequence moved on
    m = om.Model(SHAPE, w)
    _, cache, _ = m.forward_full(stale)
    hf, _ = m.forward_cached(x, rows[0], rows[1], cache)
    ref_h, _ = torch_forward(w, SHAPE, x, rows=rows, stale_x=stale)
    np.testing.assert_allclose(hf, ref_h, rtol=1e-10, atol=1e-10)


def test_wiring_mistakes_are_caught():
    """The comparison above separates the right wiring from a plausible wrong
    one: the same torch forward with gate and up swapped misses the oracle by
    far more than the tolerance."""
    w = weights(SHAPE)
    x = np.random.default_rng(1).integers(0, SHAPE.vocab, 21)
    hf, _, _ = om.Model(SHAPE, w).forward_full(x)
    swapped = dict(w)
    for l in range(SHAPE.n_layers):
        swapped[f"l{l}.w_gate"], swapped[f"l{l}.w_up"] = w[f"l{l}.w_up"], w[f"l{l}.w_gate"]
    assert np.max(np.abs(torch_forward(swapped, SHAPE, x)[0] - hf)) > 1e-3
