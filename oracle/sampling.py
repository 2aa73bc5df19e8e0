"""Stochastic tau-leaping sampling, float64 / exact integer. Test
infrastructure, like the rest of ``oracle/``.

[commentary] §3.4.1 "The Reverse Generation Process (with tau-leaping)": in a
step from noise level t to s < t every still-masked position independently
stays masked with probability s / t, and otherwise takes a token drawn from
the model's distribution q_{0|t}(. | x_t). Readings:

* Within a block of T steps the schedule runs linearly from t = 1 to 0, so
  step j (0-based) goes from t = (T - j) / T to s = (T - j - 1) / T and a
  masked position is filled with probability (t - s) / t = 1 / (T - j); the
  last step fills every remaining position, so a block ends within T steps.
* The token is a draw from softmax(z) with z the scaled logits, made with
  the Gumbel-max construction: argmax_v (z_v + G_v), G_v = -log(-log u_v),
  u_v uniform on (0, 1) (Gumbel 1954; an exact sample of the softmax).
* Random numbers come from Philox-4x64-10 (Salmon, Moraes, Dror, Shaw,
  "Parallel random numbers: as easy as 1, 2, 3", SC 2011), a counter-based
  generator, so both implementations draw the same numbers: key = (seed,
  sequence index); counter = (v // 4, position, step within the block, 1)
  gives the uniforms of vocabulary ids v .. v + 3 (output word v % 4), and
  counter = (0, position, step, 2) the fill decision (output word 0).
* Uniforms: the fill decision compares u = (w >> 11) * 2^-53 with
  1 / (T - j) in float64 (exact on both sides); the Gumbel noise uses
  u = ((w >> 41) + 0.5) * 2^-23, exactly representable and strictly inside
  (0, 1) (23 bits plus one half: with 24 bits the largest value would round
  to 1 in float32 and give an infinite noise term), and G = -log(-log u) in
  float64 like the rest of the oracle; z + G is compared in float64.
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157   # Philox-4x64 multipliers
W0, W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B   # key increments (Weyl)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a: np.ndarray, m: int):
    """(high, low) 64-bit words of the 128-bit product a * m, a uint64 array."""
    a = np.asarray(a, dtype=np.uint64)
    m0, m1 = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
    a0, a1 = a & _LO32, a >> _S32
    p00, p01, p10, p11 = a0 * m0, a0 * m1, a1 * m0, a1 * m1
    carry = ((p00 >> _S32) + (p01 & _LO32) + (p10 & _LO32)) >> _S32
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + carry
    with np.errstate(over="ignore"):
        lo = a * np.uint64(m)
    return hi, lo


def philox4x64(counter, key, rounds: int = 10) -> np.ndarray:
    """Philox-4x64-R of counters [..., 4] under key (k0, k1): [..., 4] uint64."""
    c = np.array(counter, dtype=np.uint64, copy=True)
    k0, k1 = np.uint64(key[0]), np.uint64(key[1])
    with np.errstate(over="ignore"):
        for _ in range(rounds):
            hi0, lo0 = _mulhilo(c[..., 0], M0)
            hi1, lo1 = _mulhilo(c[..., 2], M1)
            c = np.stack([hi1 ^ c[..., 1] ^ k0, lo1, hi0 ^ c[..., 3] ^ k1, lo0], axis=-1)
            k0 = k0 + np.uint64(W0)
            k1 = k1 + np.uint64(W1)
    return c


def gumbel_noise(seed: int, seq: int, pos: int, step: int, vocab: int) -> np.ndarray:
    """G_v = -log(-log u_v), v in [0, vocab), float64."""
    n4 = (vocab + 3) // 4
    ctr = np.zeros((n4, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(n4, dtype=np.uint64)
    ctr[:, 1], ctr[:, 2], ctr[:, 3] = pos, step, 1
    w = philox4x64(ctr, (seed, seq)).reshape(-1)[:vocab]
    u = ((w >> np.uint64(41)).astype(np.float64) + 0.5) * 2.0 ** -23
    return -np.log(-np.log(u))


def fill_uniform(seed: int, seq: int, pos: int, step: int) -> float:
    w = philox4x64(np.array([[0, pos, step, 2]], dtype=np.uint64), (seed, seq))[0, 0]
    return float(int(w) >> 11) * 2.0 ** -53


def sample_token(z: np.ndarray, seed: int, seq: int, pos: int, step: int) -> int:
    """Gumbel-max draw from softmax(z) for block position ``pos`` at ``step``
    (lowest id on an exact tie of z + G)."""
    s = np.asarray(z, dtype=np.float64) + gumbel_noise(seed, seq, pos, step, len(z))
    return int(np.argmax(s))


def tau_leap_step(z: np.ndarray, masked: np.ndarray, blk_start: int, step: int, T: int,
                  seed: int, seq: int = 0):
    """One tau-leaping step of one sequence's block: z [B][V] scaled logits,
    masked [B]. Returns (selected block positions, sampled token per block
    position (-1 where not masked))."""
    B = len(masked)
    p = 1.0 / (T - step)
    tok = np.full(B, -1, dtype=np.int64)
    sel = []
    for i in range(B):
        if not masked[i]:
            continue
        tok[i] = sample_token(z[i], seed, seq, blk_start + i, step)
        if fill_uniform(seed, seq, blk_start + i, step) < p:
            sel.append(i)
    return np.array(sel, dtype=np.int64), tok
