"""Pins of the oracle's layer primitives against library routines, closed forms
and invariants (CPU only)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import model as om


def rng(seed=0):
    return np.random.default_rng(seed)


def test_rms_norm_matches_torch():
    x = rng(1).standard_normal((7, 96))
    g = 1.0 + 0.1 * rng(2).standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(x), (96,), weight=torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(om.rms_norm(x, g, 1e-5), ref, rtol=1e-12, atol=1e-12)


def test_silu_matches_torch():
    x = rng(3).standard_normal(1000) * 6
    np.testing.assert_allclose(om.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (7, 1)])
def test_attention_matches_torch_sdpa(hq, hkv):
    r = rng(4)
    m, n, d = 5, 19, 16
    q = r.standard_normal((m, hq, d))
    k = r.standard_normal((n, hkv, d))
    v = r.standard_normal((n, hkv, d))
    out = om.attention(q, k, v, 1.0 / np.sqrt(d))
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=False).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_attention_has_no_causal_mask():
    """Zero queries give uniform weights over all keys, later ones included."""
    r = rng(5)
    q = np.zeros((3, 2, 8))
    k = r.standard_normal((11, 2, 8))
    v = r.standard_normal((11, 2, 8))
    out = om.attention(q, k, v, 0.3)
    for i in range(3):
        np.testing.assert_allclose(out[i], v.mean(axis=0), rtol=1e-12)


def test_rope_closed_form_and_invariants():
    d, theta = 8, 10000.0
    r = rng(6)
    x = r.standard_normal((5, 3, d))
    pos = np.array([0, 1, 7, 100, 1279])
    y = om.apply_rope(x, pos, theta)
    # position 0 is the identity
    np.testing.assert_allclose(y[0], x[0], rtol=0, atol=0)
    # each pair (j, j + d/2) is the complex number x_j + i x_{j+d/2} times e^{i p w_j}
    w = theta ** (-2.0 * np.arange(d // 2) / d)
    for ri, p in enumerate(pos):
        zc = (x[ri, :, : d // 2] + 1j * x[ri, :, d // 2:]) * np.exp(1j * p * w)
        np.testing.assert_allclose(y[ri, :, : d // 2], zc.real, atol=1e-12)
        np.testing.assert_allclose(y[ri, :, d // 2:], zc.imag, atol=1e-12)
    # norm preserving
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    # scores depend only on relative position
    q, k = r.standard_normal((1, 1, d)), r.standard_normal((1, 1, d))
    s1 = np.sum(om.apply_rope(q, [13], theta) * om.apply_rope(k, [5], theta))
    s2 = np.sum(om.apply_rope(q, [1013], theta) * om.apply_rope(k, [1005], theta))
    assert abs(s1 - s2) < 1e-9


def test_store_rounds_to_nearest_even():
    one = 1.0
    vals = np.array([one + 2 ** -8, one + 3 * 2 ** -8, one + 2 ** -8 + 2 ** -20, -2.0, 3.0e38 * 2])
    out = om.store(vals, "bf16")
    assert out[0] == 1.0                      # tie -> even mantissa
    assert out[1] == 1.0 + 2 ** -6            # tie -> even mantissa (upwards)
    assert out[2] == 1.0 + 2 ** -7            # above the tie -> up
    assert out[3] == -2.0
    assert np.isinf(out[4])
    assert om.store(np.array([1.0 + 2 ** -30]), "f32")[0] == 1.0
    assert om.store(np.array([1.0 + 2 ** -30]), "f64")[0] == 1.0 + 2 ** -30


def test_bf16_bits_decode():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000], dtype=np.uint16)
    np.testing.assert_array_equal(om.as_f64(bits), [1.0, -2.0, 1.0 + 2 ** -7, 0.0, -0.0])


def test_block_attention_head_major_layout():
    r = rng(7)
    b, m, hq, hkv, n, d = 2, 3, 4, 2, 9, 8
    q = r.standard_normal((b, m, hq, d))
    k = r.standard_normal((b, hkv, n, d))
    v = r.standard_normal((b, hkv, n, d))
    out = om.block_attention(q, k, v, 0.25)
    for i in range(b):
        for h in range(hq):
            s = q[i, :, h] @ k[i, h // 2].T * 0.25
            p = np.exp(s - s.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            np.testing.assert_allclose(out[i, :, h], p @ v[i, h // 2], rtol=1e-12)


def test_attention_lse_matches_scipy_and_normalises_softmax():
    """block_attention_lse is scipy's logsumexp of the scaled scores, and
    exp(scores - lse) sums to one over the keys (GQA heads share kv heads)."""
    from scipy.special import logsumexp
    r = rng(11)
    b, m, hq, hkv, n, d = 2, 5, 6, 3, 40, 16
    q = r.standard_normal((b, m, hq, d)) * 3
    k = r.standard_normal((b, hkv, n, d))
    lse = om.block_attention_lse(q, k, 0.25)
    for i in range(b):
        for h in range(hq):
            s = 0.25 * q[i, :, h] @ k[i, h // 2].T
            np.testing.assert_allclose(lse[i, :, h], logsumexp(s, axis=-1), rtol=1e-13)
            np.testing.assert_allclose(np.exp(s - lse[i, :, h, None]).sum(-1), 1.0, rtol=1e-12)
