"""GPU parity of the K/V drift diagnostic (fdllm_kv_cosine) against the
oracle's float64 cosine, on random snapshots in the cache layout and on the
caches two refreshes of a tiny model leave behind."""
import numpy as np
import pytest

from block_wise_kv_amd import synth
from oracle import diagnostics as dg
from oracle import model as om
from tests.helpers import host, tile_v, untile_v

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_wise_kv_amd import fdllm
    fdllm.lib()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_kv_cosine_random_snapshots(dt):
    from block_wise_kv_amd import fdllm as F
    rng = np.random.default_rng(11)
    b, h, cap, d = 2, 3, 70, 64          # a capacity that is not a multiple of 32
    row0, row1 = 5, 66
    ka = rng.standard_normal((b, h, cap, d)).astype(np.float32)
    va = rng.standard_normal((b, h, cap, d)).astype(np.float32)
    kb = (ka + rng.uniform(0, 1.5) * rng.standard_normal(ka.shape)).astype(np.float32)
    vb = (0.7 * va + 0.5 * rng.standard_normal(va.shape)).astype(np.float32)
    kb[1, :, 9] = 0.0                     # an all-zero token: cosine 0
    if dt == "bf16":
        ka, va, kb, vb = (synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a)) for a in (ka, va, kb, vb))
    dev = lambda a: torch.from_numpy(synth.f32_to_bf16_bits(a).view(np.int16) if dt == "bf16" else a).cuda()
    out = torch.zeros(b * (row1 - row0) * 2, device="cuda")
    F.fdllm_kv_cosine(dev(ka), dev(tile_v(va)), dev(kb), dev(tile_v(vb)), b, h, cap, d, row0, row1,
                      F.BF16 if dt == "bf16" else F.F32, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(b, row1 - row0, 2)
    for s in range(b):
        tok = lambda a: np.swapaxes(a[s], 0, 1)[row0:row1]   # [rows][h][d]
        np.testing.assert_allclose(got[s, :, 0], dg.cosine_rows(tok(ka), tok(kb)), atol=2e-6)
        np.testing.assert_allclose(got[s, :, 1], dg.cosine_rows(tok(va), tok(vb)), atol=2e-6)
    assert got[1, 9 - row0, 0] == 0.0


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_bf16"])
def test_kv_drift_between_two_refreshes(name):
    """Cache snapshot after a refresh of x, then a refresh of x with part of
    the block filled in: the per-token K/V cosine over the prompt and the
    suffix rows, GPU against the oracle's two forwards."""
    import dataclasses
    from block_wise_kv_amd import fdllm as F
    from block_wise_kv_amd.runtime import GPUCache, GPUModel
    shape = synth.TINY if name == "tiny_f32" else dataclasses.replace(synth.TINY, dtype="bf16")
    w = synth.make_weights(shape, seed=7, norm_gain_std=0.1, threads=4)
    gm = GPUModel(shape, w, max_seq_len=128)
    gc = GPUCache(gm, 1, 128)
    P, L, B = 32, 64, 16
    N = P + L
    prompt = synth.make_prompt(shape, P, seed=13)[0]
    x, _ = synth.initial_sequence(shape, prompt[None], L)
    x1 = x[0].copy()
    x2 = x1.copy()
    x2[P:P + 9] = np.arange(100, 109)     # nine tokens of the first block decided
    o = om.Model(shape, w)
    _, c1, _ = o.forward_full(x1.astype(np.int64))
    _, c2, _ = o.forward_full(x2.astype(np.int64))
    hid = torch.empty(1, B, shape.d_model, device="cuda")
    snaps = []
    for xx in (x1, x2):
        F.fdllm_cache_refresh(gm.handle, gc.handle, torch.from_numpy(xx[None].astype(np.int32)).cuda(),
                              1, N, P, B, hid)
        torch.cuda.synchronize()
        snaps.append([kv_snapshot(gc, l, shape) for l in range(shape.n_layers)])
    dtc = F.BF16 if shape.dtype == "bf16" else F.F32
    tol = 1e-5 if shape.dtype == "f32" else 2e-3
    for l in range(shape.n_layers):
        (ka, va, ncap), (kb, vb, _) = snaps[0][l], snaps[1][l]
        out = torch.zeros(N * 2, device="cuda")
        F.fdllm_kv_cosine(ka, va, kb, vb, 1, shape.n_kv_heads, ncap, shape.head_dim, 0, N, dtc, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().reshape(N, 2)
        ck, cv = dg.kv_cosine(c1[l], c2[l])
        for rows, label in ((slice(0, P), "prompt"), (slice(P + B, N), "suffix")):
            err = max(np.abs(got[rows, 0] - ck[rows]).max(), np.abs(got[rows, 1] - cv[rows]).max())
            print(f"{name} layer {l} {label}: mean cos K {ck[rows].mean():.4f} V {cv[rows].mean():.4f}, "
                  f"max |gpu - oracle| {err:.1e}")
            assert err < tol
        assert np.all(np.abs(got) <= 1.0 + 1e-6)
        if l == 0:
            # layer 0's keys and values depend only on a row's token and
            # position: unchanged rows give exactly 1
            same = x1 == x2
            np.testing.assert_allclose(got[same], 1.0, atol=1e-6)
            assert np.all(got[~same, 0] < 0.5)


def kv_snapshot(gc, layer, shape):
    """Copies of one layer's K and V out of the cache arena (located with
    fdllm_cache_kv) and the cache's ncap."""
    from block_wise_kv_amd import fdllm as F
    kp, vp, ncap = F.fdllm_cache_kv(gc.handle, layer)
    nbytes = shape.n_kv_heads * ncap * shape.head_dim * (2 if shape.dtype == "bf16" else 4)
    base = gc.mem.data_ptr()
    assert base <= kp and kp + nbytes <= base + gc.mem.numel()
    assert base <= vp and vp + nbytes <= base + gc.mem.numel()
    return (gc.mem[kp - base:kp - base + nbytes].clone(), gc.mem[vp - base:vp - base + nbytes].clone(), ncap)
