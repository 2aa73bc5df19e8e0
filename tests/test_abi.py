"""The C-ABI library loads and exports every function include/fdllm.h declares
(CPU only: no compute call is made)."""
import ctypes
import os
import re

import pytest

from block_wise_kv_amd import fdllm as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fdllm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fdllm_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("fdllm_cache_refresh", "fdllm_block_attention", "fdllm_block_forward",
                     "fdllm_confidence_unmask", "fdllm_decode"):
        assert required in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(F.LIB_PATH):
        pytest.fail("libfdllm.so is not built (python -m block_wise_kv_amd.build)")
    lib = ctypes.CDLL(F.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(F.EXPORTS)


def test_version_and_host_side_validation():
    lib = F.lib()
    assert b"gfx950" in lib.fdllm_version()
    cfg = F.ModelConfig(n_layers=1, d_model=100, n_heads=2, n_kv_heads=1, head_dim=64, ffn_dim=128,
                        vocab=64, mask_id=63, dtype=F.F32, max_seq_len=8, rope_theta=1e4,
                        norm_eps=1e-5, logit_scale=1.0)
    with pytest.raises(F.FdllmError) as e:
        F.fdllm_model_packed_bytes(cfg)
    assert e.value.status == F.ESHAPE and "d_model" in str(e.value)
    cfg.d_model = 256
    assert F.fdllm_model_packed_bytes(cfg) > 0
    cfg.head_dim = 96
    with pytest.raises(F.FdllmError):
        F.fdllm_model_packed_bytes(cfg)
    n = ctypes.c_size_t()
    assert lib.fdllm_block_attention_workspace(0, 1, 1, 64, 8, ctypes.byref(n)) == F.EINVAL
    assert lib.fdllm_unmask_logits_workspace(2, 8, 512, ctypes.byref(n)) == F.OK and n.value > 0


def test_struct_layouts_and_host_only_calls():
    """The ctypes mirrors have the header's sizes, and the host-only sizing
    calls validate their arguments."""
    lib = F.lib()
    assert ctypes.sizeof(F.DecodeStats) == 4 * (6 + F.STATS_BLOCKS + F.STATS_STEPS)
    assert ctypes.sizeof(F.DecodeParams) == 11 * 4 and ctypes.sizeof(F.SelectParams) == 5 * 4
    n = ctypes.c_int32()
    assert lib.fdllm_stream_read_blocks(1 << 30, ctypes.byref(n)) == F.OK and n.value == 2048
    assert lib.fdllm_stream_read_blocks(1 << 16, ctypes.byref(n)) == F.OK and n.value == 2
    assert lib.fdllm_stream_read_blocks(100, ctypes.byref(n)) == F.EINVAL
    assert lib.fdllm_tile_values(None, None, 1, 1, 32, 64, F.BF16, None) == F.EINVAL
