"""Host-side checks of the benchmark's byte accounting (no GPU)."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402
from block_wise_kv_amd import synth  # noqa: E402


@pytest.mark.parametrize("shape,kv_rows", [(synth.LLADA8B, 768), (synth.LLADA8B, 1024), (synth.DREAM7B, 1280),
                                           (synth.TINY, 96)])
def test_step_bytes_from_parameter_count(shape, kv_rows):
    """The cached step's bytes equal the model's parameters minus the
    embedding table and the norm gains, at the storage width, plus K and V
    of every cache row read and of the block rows written, per layer."""
    es = 2 if shape.dtype == "bf16" else 4
    d = shape.d_model
    gains = shape.n_layers * 2 * d + d
    weights = (shape.n_params() - shape.vocab * d - gains) * es
    kv = shape.n_layers * 2 * shape.n_kv_heads * shape.head_dim * es * (kv_rows + 32)
    assert bench.step_bytes(shape, 1, 32, kv_rows) == weights + kv


def test_step_bytes_llada_prefix_figure():
    """LLaDA-8B-shaped PrefixCache step at the last block (32 rows over a
    768-row cache): 15.41 GB, the figure the hot-path scope table quotes."""
    assert round(bench.step_bytes(synth.LLADA8B, 1, 32, 768) / 1e9, 2) == 15.41


def test_step_bytes_scales_with_batch_only_in_kv():
    """Weights are read once per step whatever the batch; each further
    sequence adds its own K/V (1024 rows read, 32 written, per layer)."""
    one = bench.step_bytes(synth.LLADA8B, 1, 32, 1024)
    eight = bench.step_bytes(synth.LLADA8B, 8, 32, 1024)
    kvd = synth.LLADA8B.n_kv_heads * synth.LLADA8B.head_dim
    assert eight - one == 7 * synth.LLADA8B.n_layers * kvd * 2 * 2 * (1024 + 32)
