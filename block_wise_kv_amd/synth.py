"""Seeded synthetic inputs: workload shapes, random-init weights, prompts,
attention operands and logits.

This module only *draws* inputs. It holds none of the decoding method's
arithmetic, so both the HIP path and the CPU oracle can be fed from it
without sharing any computation.

Workloads (model shapes and decode settings) follow the configurations the
method is evaluated on: a tiny fp32 model, an LLaDA-8B-shaped model and a
Dream-7B-shaped model (random init), plus an isolated kernel sweep. Weights
are N(0, 0.02^2), drawn per tensor and per fixed-size chunk from PCG64 streams
keyed by (seed, tensor index, chunk index), so the result does not depend on
the number of threads used. bf16 weights are the round-to-nearest-even bf16
of the float32 draw, returned as raw uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22  # elements per independent random stream


@dataclasses.dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    mask_id: int
    dtype: str  # "f32" or "bf16"
    rope_theta: float = 10000.0
    norm_eps: float = 1e-5
    logit_scale: float = 1.0

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def n_params(self) -> int:
        d, f, v = self.d_model, self.ffn_dim, self.vocab
        per_layer = d * (self.q_dim + 2 * self.kv_dim) + self.q_dim * d + 3 * d * f + 2 * d
        return self.n_layers * per_layer + 2 * v * d + d


@dataclasses.dataclass(frozen=True)
class DecodeSettings:
    prompt_len: int
    gen_length: int
    block_size: int
    steps: int
    use_cache: bool
    dual_cache: bool
    threshold: float
    batch: int = 1
    factor: float = 0.0  # > 0: the factor strategy with this f (threshold unused)
    refresh_interval: int = 0  # > 0: also rebuild the cache at steps t % r == 0 of a block
    topk: int = 0  # > 0: fixed top-K selection (the LLaDA baseline) instead of tau / factor
    sampling: bool = False  # stochastic tau-leaping instead of a confidence rule
    seed: int = 0  # key of the counter-based generator the sampling draws from


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    decode: DecodeSettings
    seed_w: int
    seed_p: int


# The five evaluated workloads. The logit scale of the 8B/7B-shaped models is
# calibrated once on the oracle so that the median top-1 probability of the
# first (all-masked) forward is about 0.9; see oracle/calibrate.py.
TINY = ModelShape(2, 256, 4, 4, 64, 768, 2048, 2047, "f32", logit_scale=20.0)
LLADA8B = ModelShape(32, 4096, 32, 32, 128, 12288, 126464, 126463, "bf16", logit_scale=13.5)
DREAM7B = ModelShape(28, 3584, 28, 4, 128, 18944, 152064, 152063, "bf16", logit_scale=4.78)

WORKLOADS = {
    "tiny_prefix": Workload("tiny_prefix", TINY, DecodeSettings(32, 64, 16, 64, True, False, 0.9), 1, 11),
    "llada8b_prefix_gen256": Workload(
        "llada8b_prefix_gen256", LLADA8B, DecodeSettings(512, 256, 32, 256, True, False, 0.9), 2, 12),
    "llada8b_dual_gen512": Workload(
        "llada8b_dual_gen512", LLADA8B, DecodeSettings(512, 512, 32, 512, True, True, 0.9), 2, 13),
    "dream7b_dual_gen1024": Workload(
        "dream7b_dual_gen1024", DREAM7B, DecodeSettings(256, 1024, 32, 1024, True, True, 0.9), 3, 14),
    # eight sequences decoded in lockstep (a block advances once every
    # sequence has finished it): the cached steps run 8 x 32 rows per weight pass
    "llada8b_dual_gen512_b8": Workload(
        "llada8b_dual_gen512_b8", LLADA8B,
        DecodeSettings(512, 512, 32, 512, True, True, 0.9, batch=8), 2, 13),
    # the cache also rebuilt every 4 steps within a block ([commentary]
    # Table 10's refresh policy) on the LLaDA Prefix setup
    "llada8b_prefix_gen256_r4": Workload(
        "llada8b_prefix_gen256_r4", LLADA8B,
        DecodeSettings(512, 256, 32, 256, True, False, 0.9, refresh_interval=4), 2, 12),
    # the fixed top-K baseline the pages compare against, 4 tokens per step
    "llada8b_prefix_gen256_top4": Workload(
        "llada8b_prefix_gen256_top4", LLADA8B,
        DecodeSettings(512, 256, 32, 256, True, False, 0.9, topk=4), 2, 12),
    # stochastic tau-leaping (the LLaDA sampling baseline, [commentary] 3.4.1)
    "llada8b_prefix_gen256_sample": Workload(
        "llada8b_prefix_gen256_sample", LLADA8B,
        DecodeSettings(512, 256, 32, 256, True, False, 0.9, sampling=True, seed=1), 2, 12),
    # the factor strategy ([commentary] 3.4.3) at f = 1, the theorem's own
    # bound and the pages' chosen operating point, on the LLaDA Prefix setup
    "llada8b_prefix_gen256_factor": Workload(
        "llada8b_prefix_gen256_factor", LLADA8B,
        DecodeSettings(512, 256, 32, 256, True, False, 0.9, factor=1.0), 2, 12),
}

# Isolated kernel sweep (bf16): block attention and logits-in confidence unmask.
SWEEP_ATTN = dict(batch=8, q_rows=32, n_heads=32, head_dim=128, kv_lens=(1024, 2048, 4096, 8192), seed=21)
SWEEP_UNMASK = dict(batch=8, block=32, vocab=126464, scales=(5.0, 10.0, 20.0),
                    masked_fracs=(1.0, 0.5, 0.1), taus=(0.7, 0.9, 0.95), seed=31)


def scaled(shape: ModelShape, **kw) -> ModelShape:
    return dataclasses.replace(shape, **kw)


# ----------------------------------------------------------------------------
# bf16 bit helpers (storage format only)

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 (ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).copy()
    nan = np.isnan(a)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = (u >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# random tensors

def _draw_chunk(seed: int, tensor_idx: int, chunk_idx: int, n: int, std: float, mean: float,
                bf16: bool) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_idx, chunk_idx])))
    a = g.standard_normal(n, dtype=np.float32)
    a *= np.float32(std)
    if mean:
        a += np.float32(mean)
    return f32_to_bf16_bits(a) if bf16 else a


def normal_tensor(shape, seed: int, tensor_idx: int, std: float, bf16: bool, mean: float = 0.0,
                  pool: ThreadPoolExecutor | None = None) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    starts = list(range(0, n, CHUNK))

    def job(ci):
        s = starts[ci]
        m = min(CHUNK, n - s)
        out[s:s + m] = _draw_chunk(seed, tensor_idx, ci, m, std, mean, bf16)

    if pool is None or len(starts) == 1:
        for ci in range(len(starts)):
            job(ci)
    else:
        list(pool.map(job, range(len(starts))))
    return out.reshape(shape)


def tensor_names(m: ModelShape):
    """Fixed tensor order; the index of a name keys its random stream."""
    names = ["embed"]
    for l in range(m.n_layers):
        names += [f"l{l}.{t}" for t in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm",
                                         "w_gate", "w_up", "w_down")]
    names += ["final_norm", "lm_head"]
    return names


def tensor_shape(m: ModelShape, name: str):
    base = name.split(".")[-1]
    d, f = m.d_model, m.ffn_dim
    return {
        "embed": (m.vocab, d), "lm_head": (m.vocab, d),
        "attn_norm": (d,), "ffn_norm": (d,), "final_norm": (d,),
        "wq": (m.q_dim, d), "wk": (m.kv_dim, d), "wv": (m.kv_dim, d), "wo": (d, m.q_dim),
        "w_gate": (f, d), "w_up": (f, d), "w_down": (d, f),
    }[base]


def make_weights(m: ModelShape, seed: int, std: float = 0.02, norm_gain_std: float = 0.0,
                 threads: int | None = None) -> dict:
    """All weights of a random-init model.

    Matrices are [out][in] row-major. bf16 models return uint16 bf16 bits,
    fp32 models float32. Norm gains are 1 unless ``norm_gain_std`` > 0, in
    which case they are 1 + N(0, norm_gain_std^2) (used by tests so the gain
    path is exercised).
    """
    bf16 = m.dtype == "bf16"
    threads = threads or min(16, os.cpu_count() or 1)
    out = {}
    with ThreadPoolExecutor(threads) as pool:
        for idx, name in enumerate(tensor_names(m)):
            shape = tensor_shape(m, name)
            if name.endswith("norm"):
                out[name] = normal_tensor(shape, seed, idx, norm_gain_std, bf16, mean=1.0) \
                    if norm_gain_std > 0 else (
                        np.full(shape, 0x3F80, np.uint16) if bf16 else np.ones(shape, np.float32))
            else:
                out[name] = normal_tensor(shape, seed, idx, std, bf16, pool=pool)
    return out


def make_prompt(m: ModelShape, prompt_len: int, seed: int, batch: int = 1) -> np.ndarray:
    """Uniform prompt ids in [0, vocab) excluding the [MASK] id; int32 [batch][prompt_len]."""
    g = np.random.Generator(np.random.PCG64(seed))
    ids = g.integers(0, m.vocab - 1, size=(batch, prompt_len), dtype=np.int64)
    ids = np.where(ids >= m.mask_id, ids + 1, ids)  # skip mask_id wherever it sits
    return ids.astype(np.int32)


def initial_sequence(m: ModelShape, prompt: np.ndarray, gen_length: int):
    """x = [prompt; MASK * gen_length] and the masked flags (1 = masked)."""
    b, p = prompt.shape
    x = np.full((b, p + gen_length), m.mask_id, dtype=np.int32)
    x[:, :p] = prompt
    flags = np.zeros((b, p + gen_length), dtype=np.uint8)
    flags[:, p:] = 1
    return x, flags


def attention_operands(batch, q_rows, n_heads, n_kv_heads, head_dim, kv_len, seed, bf16=True):
    """Q [b][q_rows][Hq][D], K and V [b][Hkv][kv_len][D], N(0,1)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, kv_len, q_rows, n_heads])))
    q = g.standard_normal((batch, q_rows, n_heads, head_dim), dtype=np.float32)
    k = g.standard_normal((batch, n_kv_heads, kv_len, head_dim), dtype=np.float32)
    v = g.standard_normal((batch, n_kv_heads, kv_len, head_dim), dtype=np.float32)
    if bf16:
        return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    return q, k, v


def sweep_logits(batch, block, vocab, scale, seed, bf16=True):
    """Logits scale * N(0,1), [batch][block][vocab]."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, int(scale * 100), vocab])))
    z = g.standard_normal((batch, block, vocab), dtype=np.float32)
    z *= np.float32(scale)
    return f32_to_bf16_bits(z) if bf16 else z


def sweep_masked(batch, block, frac, seed) -> np.ndarray:
    """uint8 [batch][block]: exactly round(frac*block) masked positions per row, seeded."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, int(frac * 1000), block])))
    k = int(round(frac * block))
    flags = np.zeros((batch, block), dtype=np.uint8)
    for b in range(batch):
        flags[b, g.permutation(block)[:k]] = 1
    return flags
