"""The allocation-free logits-in unmask (fdllm_confidence_unmask_logits_noalloc)
against the workspace entry point it varies (fdllm_confidence_unmask_logits):
identical ids, flags, confidences, argmaxes and counts, on two calls in a
row, the second with a smaller input, so the fixed scratch's contents left
by the first call are shown not to leak into the second."""
import numpy as np
import pytest

from block_wise_kv_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def inputs(b, B, V, dt, frac, seed):
    z = synth.sweep_logits(b, B, V, 10.0, seed, bf16=(dt == "bf16"))
    flags_blk = synth.sweep_masked(b, B, frac, seed)
    extra = 3
    x = np.full((b, B + extra), 5, np.int32)
    x[:, extra:] = -1
    flags = np.zeros((b, B + extra), np.uint8)
    flags[:, extra:] = flags_blk
    return z, x, flags, extra


def run(entry, z, x, flags, extra, dt, tau, sampling):
    from block_wise_kv_amd import fdllm as F
    b, B, V = z.shape
    tz = torch.from_numpy(z.view(np.int16) if z.dtype == np.uint16 else z).cuda()
    tx, tf = torch.from_numpy(x).cuda(), torch.from_numpy(flags).cuda()
    conf = torch.full((b, B), -1.0, device="cuda")
    am = torch.full((b, B), -7, dtype=torch.int32, device="cuda")
    counts = torch.full((b, 2), -7, dtype=torch.int32, device="cuda")
    dtc = F.BF16 if dt == "bf16" else F.F32
    kw = dict(sampling=sampling, seed=11)
    if entry == "workspace":
        ws = torch.zeros(F.fdllm_unmask_logits_workspace(b, B, V), dtype=torch.uint8, device="cuda")
        F.fdllm_confidence_unmask_logits(tz, dtc, tx, tf, b, x.shape[1], extra, B, V, tau, 1, 4, conf, am,
                                         counts, ws, **kw)
    else:
        F.fdllm_confidence_unmask_logits_noalloc(tz, dtc, tx, tf, b, x.shape[1], extra, B, V, tau, 1, 4,
                                                 conf, am, counts, **kw)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (tx, tf, conf, am, counts)]


@pytest.mark.parametrize("sampling", [False, True])
def test_noalloc_unmask_matches_workspace_entry_point(sampling):
    cases = [  # the sweep shape, then a smaller, ragged one
        (8, 32, 126464, "bf16", 0.5, 31, 0.9),
        (2, 13, 40000, "f32", 1.0, 32, 0.7),
    ]
    for b, B, V, dt, frac, seed, tau in cases:
        z, x, flags, extra = inputs(b, B, V, dt, frac, seed)
        ref = run("workspace", z, x, flags, extra, dt, tau, sampling)
        got = run("noalloc", z, x, flags, extra, dt, tau, sampling)
        for r, g in zip(ref, got):
            np.testing.assert_array_equal(g, r)
        assert ref[4][:, 0].sum() > 0  # something was committed


def test_noalloc_unmask_rejects_sizes_beyond_its_scratch():
    from block_wise_kv_amd import fdllm as F
    b, B, V = 64, 64, 126464  # 64 * 64 * 8 (row, chunk) entries > 16384
    assert b * B * -(-V // 16384) > F.NOALLOC_UNMASK_ENTRIES
    z = torch.zeros(b, B, V, dtype=torch.int16, device="cuda")
    x = torch.zeros(b, B, dtype=torch.int32, device="cuda")
    fl = torch.ones(b, B, dtype=torch.uint8, device="cuda")
    c = torch.zeros(b, B, device="cuda")
    a = torch.zeros(b, B, dtype=torch.int32, device="cuda")
    n = torch.zeros(b, 2, dtype=torch.int32, device="cuda")
    with pytest.raises(F.FdllmError) as e:
        F.fdllm_confidence_unmask_logits_noalloc(z, F.BF16, x, fl, b, B, 0, B, V, 0.9, 0, 4, c, a, n)
    assert e.value.status == F.EINVAL and "fixed scratch" in str(e.value)
    torch.cuda.synchronize()
    assert fl.all()  # nothing was enqueued
