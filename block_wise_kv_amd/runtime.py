"""Device-memory plumbing around the C ABI: uploads host weights with torch,
creates the model and cache handles, and keeps the torch tensors that back
them alive. No computation happens here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import fdllm as F
from .synth import tensor_names


def model_config(shape, max_seq_len: int) -> F.ModelConfig:
    return F.ModelConfig(
        n_layers=shape.n_layers, d_model=shape.d_model, n_heads=shape.n_heads,
        n_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim, ffn_dim=shape.ffn_dim,
        vocab=shape.vocab, mask_id=shape.mask_id, dtype=F.BF16 if shape.dtype == "bf16" else F.F32,
        max_seq_len=max_seq_len, rope_theta=shape.rope_theta, norm_eps=shape.norm_eps,
        logit_scale=shape.logit_scale)


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Host array -> device tensor with the same bytes (bf16 bits stay uint16 bits)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(a).to(device)


def elem_dtype(shape):
    return torch.int16 if shape.dtype == "bf16" else torch.float32


class GPUModel:
    """Packed model on the current device. ``weights`` maps tensor names (the
    fixed order of synth.tensor_names) to host arrays or device tensors."""

    def __init__(self, shape, weights: dict, max_seq_len: int, device="cuda"):
        self.shape = shape
        self.cfg = model_config(shape, max_seq_len)
        nbytes = F.fdllm_model_packed_bytes(self.cfg)
        self.packed = torch.empty(nbytes, dtype=torch.uint8, device=device)
        raw = []
        for name in tensor_names(shape):
            w = weights[name]
            raw.append(w if isinstance(w, torch.Tensor) else to_device(w, device))
        self.handle = F.fdllm_model_create(self.cfg, raw, self.packed)
        torch.cuda.synchronize()
        del raw

    def __del__(self):
        h = getattr(self, "handle", None)
        # at interpreter exit the binding's module may already be torn down
        if h is not None and getattr(F, "fdllm_model_destroy", None) is not None:
            F.fdllm_model_destroy(h)
            self.handle = None


class GPUCache:
    def __init__(self, model: GPUModel, batch: int, max_seq: int, device="cuda"):
        self.model = model
        nbytes = F.fdllm_cache_bytes(model.handle, batch, max_seq)
        self.mem = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.handle = F.fdllm_cache_create(model.handle, batch, max_seq, self.mem)
        torch.cuda.synchronize()

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and getattr(F, "fdllm_cache_destroy", None) is not None:
            F.fdllm_cache_destroy(h)
            self.handle = None


def decode_params(settings) -> F.DecodeParams:
    return F.DecodeParams(gen_length=settings.gen_length, steps=settings.steps,
                          block_size=settings.block_size, use_cache=int(settings.use_cache),
                          dual_cache=int(settings.dual_cache), threshold=settings.threshold,
                          factor=settings.factor, refresh_interval=settings.refresh_interval,
                          topk=settings.topk, sampling=int(settings.sampling), seed=settings.seed)
