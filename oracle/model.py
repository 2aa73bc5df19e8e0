"""Bidirectional masked-diffusion transformer forward, float64.

The pages fix the attention pattern of the model, not its layer internals:
[commentary] §3.4.2 "Why Standard KV Caching Fails" says every position
attends to every other position (no causal mask) and that K_i = W_K h_i,
V_i = W_V h_i. The layer itself (pre-norm RMSNorm, rotate-half RoPE at
absolute positions, grouped-query attention, SwiGLU feed-forward, final
RMSNorm and an untied LM head scaled by a logit scale) is the standard
LLaDA / Dream layout the evaluated model shapes name.

Precision. Arithmetic is float64. The pages fix no precision; the evaluated
model shapes name a storage dtype (bf16 or f32), read here as the dtype of
what the model keeps in memory across denoising steps: its weights and its
KV cache. So the oracle rounds k and v (after RoPE) to that dtype, the values
a cache in that dtype holds, and nothing else (``store``); the residual
stream, the normed activations, q, the attention output, the FFN activation,
every reduction and the logits stay float64. The rounding is a library
primitive (torch's round-to-nearest-even cast).
"""
from __future__ import annotations

import numpy as np
import torch


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Value a tensor of storage dtype ``dtype`` holds (RNE), back as float64."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    if dtype == "bf16":
        return t.to(torch.bfloat16).to(torch.float64).numpy()
    if dtype == "f32":
        return t.to(torch.float32).to(torch.float64).numpy()
    if dtype == "f64":
        return t.numpy()
    raise ValueError(dtype)


def as_f64(w: np.ndarray) -> np.ndarray:
    """Weights as float64. uint16 arrays are bf16 bit patterns (the upper half
    of an IEEE float32), float arrays are taken as they are. Both widenings
    are exact; the bf16 one is torch's bfloat16 -> float64 cast (a library
    primitive, multi-threaded, so an 8B-shaped model's per-forward
    conversion of its weights does not dominate the oracle's time)."""
    w = np.ascontiguousarray(w)
    if w.dtype == np.uint16:
        return torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return w.astype(np.float64)


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x * gain / sqrt(mean(x^2) + eps), per row."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gain


def rope_angles(positions: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """angle[p][i] = p * theta^(-2i/D), i < D/2 (rotate-half RoPE)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / head_dim)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]


def apply_rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """x [rows][heads][D]; pairs (j, j + D/2) rotate by the angle of row's position."""
    d = x.shape[-1]
    ang = rope_angles(positions, d, theta)
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = x[..., : d // 2]
    x2 = x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Bidirectional attention, no mask.

    q [M][Hq][D]; k, v [N][Hkv][D]; query head h reads kv head h // (Hq/Hkv).
    Returns [M][Hq][D] = softmax(q k^T * scale) v over all N keys.
    [commentary] §3.4.2: at a denoising step every position attends to all
    other positions, including later ones.
    """
    m, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    out = np.empty((m, hq, d), dtype=np.float64)
    for h in range(hq):
        g = h // group
        s = (q[:, h, :] @ k[:, g, :].T) * scale
        out[:, h, :] = softmax_rows(s) @ v[:, g, :]
    return out


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


class Model:
    """Random-init transformer: ``shape`` is a synth.ModelShape-like object,
    ``weights`` a dict of [out][in] matrices (bf16 bits or float arrays).

    Weights are converted to float64 on use, so an 8B-shaped bf16 model stays
    in its 16 GB bit form in host memory.
    """

    def __init__(self, shape, weights: dict):
        self.s = shape
        self.w = weights
        self.dt = shape.dtype

    def W(self, name: str) -> np.ndarray:
        return as_f64(self.w[name])

    # -- one layer ---------------------------------------------------------
    def _qkv(self, l: int, h: np.ndarray, positions: np.ndarray):
        s = self.s
        u = rms_norm(h, self.W(f"l{l}.attn_norm"), s.norm_eps)
        rows = h.shape[0]
        q = (u @ self.W(f"l{l}.wq").T).reshape(rows, s.n_heads, s.head_dim)
        k = (u @ self.W(f"l{l}.wk").T).reshape(rows, s.n_kv_heads, s.head_dim)
        v = (u @ self.W(f"l{l}.wv").T).reshape(rows, s.n_kv_heads, s.head_dim)
        q = apply_rope(q, positions, s.rope_theta)
        k = store(apply_rope(k, positions, s.rope_theta), self.dt)  # as the KV cache holds it
        v = store(v, self.dt)
        return q, k, v

    def _post_attention(self, l: int, h: np.ndarray, a: np.ndarray) -> np.ndarray:
        s = self.s
        a = a.reshape(h.shape[0], s.q_dim)
        h = h + a @ self.W(f"l{l}.wo").T
        u = rms_norm(h, self.W(f"l{l}.ffn_norm"), s.norm_eps)
        gate = u @ self.W(f"l{l}.w_gate").T
        up = u @ self.W(f"l{l}.w_up").T
        act = silu(gate) * up
        return h + act @ self.W(f"l{l}.w_down").T

    def embed(self, ids: np.ndarray) -> np.ndarray:
        return as_f64(self.w["embed"][np.asarray(ids)])

    def final_hidden(self, h: np.ndarray) -> np.ndarray:
        return rms_norm(h, self.W("final_norm"), self.s.norm_eps)

    def logits(self, hf: np.ndarray) -> np.ndarray:
        """z = logit_scale * (final hidden) W_lm^T, float64 [rows][V].

        The vocabulary is taken in slices of 16384 rows of W_lm, so that the
        float64 copy of a large LM head is never materialised whole; each
        logit is the same single dot product either way."""
        w = self.w["lm_head"]
        hf = np.asarray(hf, dtype=np.float64)
        out = np.empty((hf.shape[0], w.shape[0]), dtype=np.float64)
        for v0 in range(0, w.shape[0], 16384):
            out[:, v0:v0 + 16384] = hf @ as_f64(w[v0:v0 + 16384]).T
        return self.s.logit_scale * out

    # -- full forward (no cache, or a cache refresh) -------------------------
    def forward_full(self, x: np.ndarray, keep_attn_layers=(), pos0: int = 0):
        """Forward over every row of one sequence x [N] (no mask).

        Returns (final normed hidden [N][d], cache, attn) where cache[l] =
        (k, v) of all N rows of layer l (post-RoPE, as stored) and attn maps
        each layer in ``keep_attn_layers`` to its attention output [N][Hq][D].
        Row i sits at position pos0 + i (pos0 = 0 in decoding).
        [commentary] §3.4.4 "Cache Initialization": the first forward both
        decodes and fills the cache; the cache update at a block boundary
        recomputes the K/V of every position.
        """
        s = self.s
        n = x.shape[0]
        pos = pos0 + np.arange(n)
        h = self.embed(x)
        cache, attn = [], {}
        scale = 1.0 / np.sqrt(s.head_dim)
        for l in range(s.n_layers):
            q, k, v = self._qkv(l, h, pos)
            a = attention(q, k, v, scale)
            if l in keep_attn_layers:
                attn[l] = a
            cache.append((k, v))
            h = self._post_attention(l, h, a)
        return self.final_hidden(h), cache, attn

    # -- forward of a row range over an approximate KV cache ----------------
    def forward_cached(self, x: np.ndarray, r0: int, r1: int, cache, keep_attn_layers=()):
        """Forward of rows [r0, r1) of x [N] over the cache from the last refresh.

        Fresh q, k, v are computed for rows [r0, r1) at their absolute
        positions; every query attends to all N keys, taking k, v of rows
        outside [r0, r1) from ``cache`` and of rows inside from the fresh
        computation. The cache itself is not modified.
        [commentary] §3.4.2 "PrefixCache" (rows = current block + suffix,
        prefix from cache) and "DualCache" (rows = current block only, prefix
        and suffix from cache).

        Returns (final normed hidden of rows [r0, r1), attn dict as in
        forward_full but over the rows [r0, r1)).
        """
        s = self.s
        pos = np.arange(r0, r1)
        h = self.embed(x[r0:r1])
        attn = {}
        scale = 1.0 / np.sqrt(s.head_dim)
        for l in range(s.n_layers):
            q, k_new, v_new = self._qkv(l, h, pos)
            k_all = cache[l][0].copy()
            v_all = cache[l][1].copy()
            k_all[r0:r1] = k_new
            v_all[r0:r1] = v_new
            a = attention(q, k_all, v_all, scale)
            if l in keep_attn_layers:
                attn[l] = a
            h = self._post_attention(l, h, a)
        return self.final_hidden(h), attn


def block_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Batched block attention: q [b][M][Hq][D], k and v [b][Hkv][N][D]
    (head-major cache layout) -> [b][M][Hq][D]; no mask, GQA by head groups.
    [commentary] §3.4.2: the block's queries attend to the whole cached
    sequence."""
    q = np.asarray(q, dtype=np.float64)
    out = np.empty_like(q)
    for i in range(q.shape[0]):
        out[i] = attention(q[i], np.transpose(np.asarray(k[i], np.float64), (1, 0, 2)),
                           np.transpose(np.asarray(v[i], np.float64), (1, 0, 2)), scale)
    return out


def block_attention_lse(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """Log-sum-exp of the scaled scores of batched block attention:
    lse[b][m][h] = log sum_n exp(scale q[b][m][h] . k[b][h // group][n]), the
    log of the softmax normaliser (softmax = exp(scores - lse)). q
    [b][M][Hq][D], k [b][Hkv][N][D] -> [b][M][Hq]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    b, m, hq, _ = q.shape
    group = hq // k.shape[1]
    out = np.empty((b, m, hq))
    for i in range(b):
        for h in range(hq):
            s = (q[i, :, h, :] @ k[i, h // group].T) * scale
            mx = np.max(s, axis=-1)
            out[i, :, h] = mx + np.log(np.sum(np.exp(s - mx[:, None]), axis=-1))
    return out
