"""Python binding of libfdllm.so: one function per C-ABI entry point, same
names, argument marshalling only (torch tensors -> device pointers, the
current torch stream -> hipStream_t). Every computation runs in the library's
HIP kernels; if the library is missing this module raises instead of falling
back to anything else.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfdllm.so")

F32, BF16 = 0, 1

OK, EINVAL, ESHAPE, EDTYPE, ENOTSUP, EHIP, EBUDGET, ENUMERIC = 0, -1, -2, -3, -4, -5, -6, -7


class FdllmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"fdllm status {status}: {msg}")
        self.status = status


class ModelConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "d_model", "n_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab", "mask_id",
        "dtype", "max_seq_len")] + [(n, ctypes.c_float) for n in ("rope_theta", "norm_eps", "logit_scale")]


class DecodeParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "gen_length", "steps", "block_size", "use_cache", "dual_cache")] + [
        ("threshold", ctypes.c_float), ("factor", ctypes.c_float), ("refresh_interval", ctypes.c_int32),
        ("topk", ctypes.c_int32), ("sampling", ctypes.c_int32), ("seed", ctypes.c_uint32)]


class SelectParams(ctypes.Structure):
    _fields_ = [("tau", ctypes.c_float), ("factor", ctypes.c_float), ("topk", ctypes.c_int32),
                ("sampling", ctypes.c_int32), ("seed", ctypes.c_uint32)]


STATS_BLOCKS, STATS_STEPS = 1024, 4096


class DecodeStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "nfe", "refreshes", "cached_steps", "full_steps", "max_steps_block", "committed")] + [
        ("steps_per_block", ctypes.c_int32 * STATS_BLOCKS),
        ("commits_per_step", ctypes.c_int32 * STATS_STEPS)]

    def as_dict(self, n_blocks: int | None = None) -> dict:
        d = {n: getattr(self, n) for n, _ in self._fields_
             if n not in ("steps_per_block", "commits_per_step")}
        k = min(n_blocks or STATS_BLOCKS, STATS_BLOCKS)
        d["steps_per_block"] = list(self.steps_per_block[:k])
        d["commits_per_step"] = list(self.commits_per_step[:min(self.nfe, STATS_STEPS)])
        return d


_lib = None
_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "fdllm_version": ([], ctypes.c_char_p),
    "fdllm_last_error": ([], ctypes.c_char_p),
    "fdllm_model_packed_bytes": ([ctypes.POINTER(ModelConfig), ctypes.POINTER(_sz)], _i32),
    "fdllm_model_create": ([ctypes.POINTER(ModelConfig), ctypes.POINTER(_vp), _vp, _sz, _vp,
                            ctypes.POINTER(_vp)], _i32),
    "fdllm_model_destroy": ([_vp], _i32),
    "fdllm_cache_bytes": ([_vp, _i32, _i32, ctypes.POINTER(_sz)], _i32),
    "fdllm_cache_create": ([_vp, _i32, _i32, _vp, _sz, _vp, ctypes.POINTER(_vp)], _i32),
    "fdllm_cache_destroy": ([_vp], _i32),
    "fdllm_cache_refresh": ([_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp], _i32),
    "fdllm_block_forward": ([_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp], _i32),
    "fdllm_block_attention_workspace": ([_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)], _i32),
    "fdllm_block_attention": ([_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                               _f32, _vp, _sz, _vp], _i32),
    "fdllm_tile_values": ([_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp], _i32),
    "fdllm_workspace_bytes": ([_vp, _i32, _i32, ctypes.POINTER(_sz)], _i32),
    "fdllm_stream_read_blocks": ([_sz, ctypes.POINTER(_i32)], _i32),
    "fdllm_stream_read": ([_vp, _sz, _vp, _vp], _i32),
    "fdllm_confidence_unmask": ([_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                 ctypes.POINTER(SelectParams), _i32, _i32, _vp, _vp, _vp, _vp, _vp], _i32),
    "fdllm_unmask_logits_workspace": ([_i32, _i32, _i32, ctypes.POINTER(_sz)], _i32),
    "fdllm_confidence_unmask_logits": ([_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                        ctypes.POINTER(SelectParams), _i32, _i32, _vp, _vp, _vp, _vp, _sz,
                                        _vp], _i32),
    "fdllm_confidence_unmask_logits_noalloc": ([_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                                ctypes.POINTER(SelectParams), _i32, _i32, _vp, _vp, _vp,
                                                _vp], _i32),
    "fdllm_decode": ([_vp, _vp, _vp, _vp, _i32, _i32, ctypes.POINTER(DecodeParams),
                      ctypes.POINTER(DecodeStats), _vp], _i32),
    "fdllm_cache_kv": ([_vp, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_i32)], _i32),
    "fdllm_kv_cosine": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp], _i32),
    "fdllm_cache_profile_enable": ([_vp, _i32], _i32),
    "fdllm_cache_profile_select": ([_vp, ctypes.c_char_p, _i32], _i32),
    "fdllm_cache_profile_peaks": ([_vp, ctypes.c_double, ctypes.c_double], _i32),
    "fdllm_cache_profile_read": ([_vp, ctypes.c_char_p, _sz, _i32], _i32),
}
EXPORTS = tuple(_SIGS)


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_wise_kv_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(h, name)
            f.argtypes = args
            f.restype = res
        _lib = h
    return _lib


def _check(status: int):
    if status != OK:
        raise FdllmError(status, lib().fdllm_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def fdllm_version() -> str:
    return lib().fdllm_version().decode()


def fdllm_model_packed_bytes(cfg: ModelConfig) -> int:
    n = _sz()
    _check(lib().fdllm_model_packed_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def fdllm_model_create(cfg: ModelConfig, weights, packed, stream=None):
    arr = (_vp * len(weights))(*[w.data_ptr() for w in weights])
    out = _vp()
    _check(lib().fdllm_model_create(ctypes.byref(cfg), arr, _p(packed), packed.numel() * packed.element_size(),
                                    _stream(stream), ctypes.byref(out)))
    return out


def fdllm_model_destroy(model):
    _check(lib().fdllm_model_destroy(model))


def fdllm_cache_bytes(model, batch: int, max_seq: int) -> int:
    n = _sz()
    _check(lib().fdllm_cache_bytes(model, batch, max_seq, ctypes.byref(n)))
    return n.value


def fdllm_cache_create(model, batch: int, max_seq: int, mem, stream=None):
    out = _vp()
    _check(lib().fdllm_cache_create(model, batch, max_seq, _p(mem), mem.numel() * mem.element_size(),
                                    _stream(stream), ctypes.byref(out)))
    return out


def fdllm_cache_destroy(cache):
    _check(lib().fdllm_cache_destroy(cache))


def fdllm_cache_refresh(model, cache, x, batch, seq_len, blk_start, blk_len, hidden, stream=None):
    _check(lib().fdllm_cache_refresh(model, cache, _p(x), batch, seq_len, blk_start, blk_len,
                                     _p(hidden), _stream(stream)))


def fdllm_block_forward(model, cache, x, batch, seq_len, row_start, row_end, blk_start, blk_len,
                        hidden, stream=None):
    _check(lib().fdllm_block_forward(model, cache, _p(x), batch, seq_len, row_start, row_end,
                                     blk_start, blk_len, _p(hidden), _stream(stream)))


def fdllm_block_attention_workspace(batch, q_rows, hq, head_dim, kv_len) -> int:
    n = _sz()
    _check(lib().fdllm_block_attention_workspace(batch, q_rows, hq, head_dim, kv_len, ctypes.byref(n)))
    return n.value


def fdllm_block_attention(q, k, v, o, batch, q_rows, hq, hkv, head_dim, kv_len, dtype, scale,
                          workspace=None, stream=None, lse=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fdllm_block_attention(_p(q), _p(k), _p(v), _p(o), _p(lse), batch, q_rows, hq, hkv,
                                       head_dim, kv_len, dtype, scale, _p(workspace), ws_bytes,
                                       _stream(stream)))


def fdllm_tile_values(v, vt, batch, hkv, kv_len, head_dim, dtype, stream=None):
    _check(lib().fdllm_tile_values(_p(v), _p(vt), batch, hkv, kv_len, head_dim, dtype, _stream(stream)))


def fdllm_workspace_bytes(model, batch: int, max_seq: int) -> int:
    n = _sz()
    _check(lib().fdllm_workspace_bytes(model, batch, max_seq, ctypes.byref(n)))
    return n.value


def fdllm_stream_read_blocks(nbytes: int) -> int:
    n = _i32()
    _check(lib().fdllm_stream_read_blocks(nbytes, ctypes.byref(n)))
    return n.value


def fdllm_stream_read(buf, nbytes: int, out, stream=None):
    _check(lib().fdllm_stream_read(_p(buf), nbytes, _p(out), _stream(stream)))


def fdllm_confidence_unmask(model, cache, hidden, x, masked, batch, seq_len, blk_start, blk_len,
                            tau, step_in_block, steps_per_block, conf=None, argmax=None,
                            counts=None, logits=None, stream=None, factor=0.0, topk=0, sampling=False,
                            seed=0):
    rule = SelectParams(tau=tau, factor=factor, topk=topk, sampling=int(sampling), seed=seed)
    _check(lib().fdllm_confidence_unmask(model, cache, _p(hidden), _p(x), _p(masked), batch, seq_len,
                                         blk_start, blk_len, ctypes.byref(rule), step_in_block,
                                         steps_per_block, _p(conf), _p(argmax), _p(counts),
                                         _p(logits), _stream(stream)))


def fdllm_unmask_logits_workspace(batch, blk_len, vocab) -> int:
    n = _sz()
    _check(lib().fdllm_unmask_logits_workspace(batch, blk_len, vocab, ctypes.byref(n)))
    return n.value


def fdllm_confidence_unmask_logits(logits, dtype, x, masked, batch, seq_len, blk_start, blk_len,
                                   vocab, tau, step_in_block, steps_per_block, conf, argmax, counts,
                                   workspace, stream=None, factor=0.0, topk=0, sampling=False, seed=0):
    rule = SelectParams(tau=tau, factor=factor, topk=topk, sampling=int(sampling), seed=seed)
    _check(lib().fdllm_confidence_unmask_logits(
        _p(logits), dtype, _p(x), _p(masked), batch, seq_len, blk_start, blk_len, vocab, ctypes.byref(rule),
        step_in_block, steps_per_block, _p(conf), _p(argmax), _p(counts), _p(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


NOALLOC_UNMASK_ENTRIES = 16384


def fdllm_confidence_unmask_logits_noalloc(logits, dtype, x, masked, batch, seq_len, blk_start, blk_len,
                                           vocab, tau, step_in_block, steps_per_block, conf, argmax, counts,
                                           stream=None, factor=0.0, topk=0, sampling=False, seed=0):
    rule = SelectParams(tau=tau, factor=factor, topk=topk, sampling=int(sampling), seed=seed)
    _check(lib().fdllm_confidence_unmask_logits_noalloc(
        _p(logits), dtype, _p(x), _p(masked), batch, seq_len, blk_start, blk_len, vocab, ctypes.byref(rule),
        step_in_block, steps_per_block, _p(conf), _p(argmax), _p(counts), _stream(stream)))


def fdllm_decode(model, cache, x, masked, batch, prompt_len, params: DecodeParams, stream=None) -> DecodeStats:
    st = DecodeStats()
    _check(lib().fdllm_decode(model, cache, _p(x), _p(masked), batch, prompt_len, ctypes.byref(params),
                              ctypes.byref(st), _stream(stream)))
    return st


def fdllm_cache_kv(cache, layer: int):
    """(K pointer, V pointer, ncap) of one layer of the cache."""
    k, v, n = _vp(), _vp(), _i32()
    _check(lib().fdllm_cache_kv(cache, layer, ctypes.byref(k), ctypes.byref(v), ctypes.byref(n)))
    return k.value, v.value, n.value


def fdllm_kv_cosine(k_a, v_a, k_b, v_b, batch, n_kv_heads, cap, head_dim, row0, row1, dtype, out,
                    stream=None):
    """K/V arguments are tensors or raw device addresses (ints)."""
    ptr = lambda t: ctypes.c_void_p(t) if isinstance(t, int) else _p(t)
    _check(lib().fdllm_kv_cosine(ptr(k_a), ptr(v_a), ptr(k_b), ptr(v_b), batch, n_kv_heads, cap,
                                 head_dim, row0, row1, dtype, _p(out), _stream(stream)))


def fdllm_cache_profile_enable(cache, enable: bool):
    _check(lib().fdllm_cache_profile_enable(cache, int(enable)))


def fdllm_cache_profile_select(cache, variant: str | None = None, stride: int = 1):
    _check(lib().fdllm_cache_profile_select(cache, variant.encode() if variant else None, stride))


def fdllm_cache_profile_peaks(cache, hbm_bytes_per_s: float, flops_per_s: float):
    _check(lib().fdllm_cache_profile_peaks(cache, hbm_bytes_per_s, flops_per_s))


def fdllm_cache_profile_read(cache, reset: bool = False) -> dict:
    """{variant: (launches, total_ms, total_bytes, total_flops, floor_ms)} of the timed launches."""
    buf = ctypes.create_string_buffer(1 << 16)
    _check(lib().fdllm_cache_profile_read(cache, buf, len(buf), int(reset)))
    out = {}
    for line in buf.value.decode().splitlines():
        name, n, ms, b, f, fl = line.split()
        out[name] = (int(n), float(ms), float(b), float(f), float(fl))
    return out
