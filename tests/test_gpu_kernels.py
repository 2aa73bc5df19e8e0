"""GPU parity of the standalone kernels (block attention, logits-in confidence
unmask) against the oracle, through the C ABI."""
import numpy as np
import pytest

from block_wise_kv_amd import synth
from oracle import decode as od
from oracle import model as om
from tests.helpers import TOL, NEAR, rel_l2, host, tile_v, factor_fragile, cut_fragile

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_wise_kv_amd import fdllm
    fdllm.lib()


def dev(a):
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def run_attention(q, k, vt, b, rows, hq, hkv, d, kv, dt, scale, workspace=True, with_lse=False,
                  raw=False):
    """vt: V in the value cache's tile layout (tile_v), host array or device
    tensor. Returns o (and the log-sum-exp [b][rows][hq] with with_lse) as
    float64, or the device tensors with raw."""
    from block_wise_kv_amd import fdllm as F
    tq, tk = dev(q), dev(k)
    tv = vt if isinstance(vt, torch.Tensor) else dev(vt)
    o = torch.empty_like(tq)
    lse = torch.full((b, rows, hq), float("nan"), device="cuda") if with_lse else None
    ws = None
    if workspace:
        nb = F.fdllm_block_attention_workspace(b, rows, hq, d, kv)
        ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    F.fdllm_block_attention(tq, tk, tv, o, b, rows, hq, hkv, d, kv, F.BF16 if dt == "bf16" else F.F32,
                            scale, ws, lse=lse)
    torch.cuda.synchronize()
    if raw:
        return o, lse
    if with_lse:
        return host(o), lse.cpu().numpy().astype(np.float64)
    return host(o)


ATTN_CASES = [
    # batch, q_rows, hq, hkv, D, kv_len, dtype
    (2, 32, 4, 4, 64, 64, "f32"),
    (2, 40, 8, 2, 128, 100, "bf16"),
    (1, 7, 28, 4, 128, 1028, "bf16"),
    (1, 32, 32, 32, 128, 1024, "bf16"),
    (3, 70, 4, 1, 64, 36, "f32"),
    (1, 256, 4, 4, 128, 768, "bf16"),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "b{}q{}h{}x{}d{}n{}{}".format(*c))
@pytest.mark.parametrize("workspace", [True, False])
def test_block_attention_matches_oracle(case, workspace):
    b, rows, hq, hkv, d, kv, dt = case
    q, k, v = synth.attention_operands(b, rows, hq, hkv, d, kv, seed=21, bf16=(dt == "bf16"))
    vt = tile_v(v)
    scale = 1.0 / np.sqrt(d)
    out, lse = run_attention(q, k, vt, b, rows, hq, hkv, d, kv, dt, scale, workspace, with_lse=True)
    f = om.as_f64
    ref = om.block_attention(f(q), f(k), f(v), scale)
    err = rel_l2(out, ref)
    lse_err = float(np.max(np.abs(lse - om.block_attention_lse(f(q), f(k), scale))))
    print(f"attention {case} ws={workspace}: rel L2 {err:.2e}, lse max abs err {lse_err:.2e}")
    assert err < (3e-3 if dt == "bf16" else 1e-5), err
    assert err < TOL[dt]
    assert lse_err < 1e-4, lse_err


@pytest.mark.parametrize("kv", [1024, 2048, 4096, 8192])
def test_block_attention_sweep_shapes(kv):
    """The sweep shape (batch 8, 32 queries, 32 heads x 128) in the launch
    configuration the sweep times: every output of all 256 (sequence, head)
    pairs, and every row's log-sum-exp, against the oracle."""
    cfg = synth.SWEEP_ATTN
    b, rows, h, d = cfg["batch"], cfg["q_rows"], cfg["n_heads"], cfg["head_dim"]
    q, k, v = synth.attention_operands(b, rows, h, h, d, kv, seed=cfg["seed"])
    scale = 1.0 / np.sqrt(d)
    out, lse = run_attention(q, k, tile_v(v), b, rows, h, h, d, kv, "bf16", scale, with_lse=True)
    f = om.as_f64
    ref = om.block_attention(f(q), f(k), f(v), scale)
    worst = max(rel_l2(out[bi, :, hi], ref[bi, :, hi]) for bi in range(b) for hi in range(h))
    lse_err = float(np.max(np.abs(lse - om.block_attention_lse(f(q), f(k), scale))))
    print(f"attention sweep kv {kv}: worst (sequence, head) rel L2 {worst:.2e}, whole {rel_l2(out, ref):.2e}, "
          f"lse max abs err {lse_err:.2e}")
    assert worst < 3e-3
    assert lse_err < 1e-4


@pytest.mark.parametrize("dt,d,kv", [("bf16", 128, 1000), ("f32", 64, 72), ("bf16", 64, 33)])
def test_tile_values_matches_layout_and_feeds_attention(dt, d, kv):
    """fdllm_tile_values writes exactly the tile layout (bit-exact against
    the layout's definition, zeros past kv_len), and attention over its
    output matches the oracle on plain values."""
    from block_wise_kv_amd import fdllm as F
    b, hkv, hq = 2, 3, 6
    rows = 17
    q, k, v = synth.attention_operands(b, rows, hq, hkv, d, kv, seed=5, bf16=(dt == "bf16"))
    n_t = -(-kv // 32)
    vt = torch.full((b, hkv, n_t, d, 32), 77, dtype=torch.int16 if dt == "bf16" else torch.float32,
                    device="cuda")
    F.fdllm_tile_values(dev(v), vt, b, hkv, kv, d, F.BF16 if dt == "bf16" else F.F32)
    torch.cuda.synchronize()
    got = vt.cpu().numpy()
    want = tile_v(v)
    assert np.array_equal(got.view(want.dtype), want)
    if kv % 4 == 0:
        scale = 0.125
        out = run_attention(q, k, vt, b, rows, hq, hkv, d, kv, dt, scale)
        f = om.as_f64
        assert rel_l2(out, om.block_attention(f(q), f(k), f(v), scale)) < TOL[dt]


def test_block_attention_is_deterministic():
    """Two runs with split partials merged through the workspace give
    bitwise the same outputs and log-sum-exps (fixed merge order)."""
    cfg = synth.SWEEP_ATTN
    b, rows, h, d, kv = 2, 32, 32, 128, 1024
    q, k, v = synth.attention_operands(b, rows, h, h, d, kv, seed=cfg["seed"])
    vt = dev(tile_v(v))
    from block_wise_kv_amd import fdllm as F
    assert F.fdllm_block_attention_workspace(b, rows, h, d, kv) > 4096  # split partials in use
    o1, l1 = run_attention(q, k, vt, b, rows, h, h, d, kv, "bf16", 0.088, with_lse=True, raw=True)
    o2, l2 = run_attention(q, k, vt, b, rows, h, h, d, kv, "bf16", 0.088, with_lse=True, raw=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def run_unmask(z, dt, flags_blk, tau, step=0, T=None, seq_extra=5, factor=0.0, topk=0):
    from block_wise_kv_amd import fdllm as F
    b, B, V = z.shape
    T = T or B
    seq_len = B + seq_extra
    x = np.full((b, seq_len), 7, np.int32)
    x[:, seq_extra:] = -1
    flags = np.zeros((b, seq_len), np.uint8)
    flags[:, seq_extra:] = flags_blk
    tz = torch.from_numpy(z.view(np.int16) if z.dtype == np.uint16 else z).cuda()
    tx = torch.from_numpy(x).cuda()
    tf = torch.from_numpy(flags).cuda()
    conf = torch.zeros(b, B, device="cuda")
    am = torch.zeros(b, B, dtype=torch.int32, device="cuda")
    counts = torch.zeros(b, 2, dtype=torch.int32, device="cuda")
    ws = torch.zeros(F.fdllm_unmask_logits_workspace(b, B, V), dtype=torch.uint8, device="cuda")
    F.fdllm_confidence_unmask_logits(tz, F.BF16 if dt == "bf16" else F.F32, tx, tf, b, seq_len,
                                     seq_extra, B, V, tau, step, T, conf, am, counts, ws,
                                     factor=factor, topk=topk)
    torch.cuda.synchronize()
    return (tx.cpu().numpy()[:, seq_extra:], tf.cpu().numpy()[:, seq_extra:], conf.cpu().numpy(),
            am.cpu().numpy(), counts.cpu().numpy())


def check_unmask(z, dt, flags_blk, tau, step=0, T=None, factor=0.0, topk=0):
    zf = om.as_f64(z)
    b, B, V = z.shape
    T = T or B
    ids0 = np.full((b, B), -1)
    quota = [max(1, -(-int(f.sum()) // (T - step))) if f.any() else 0 for f in flags_blk]
    r_ids, r_flags, r_c, r_a, r_com, r_left = od.unmask_step(zf, ids0, flags_blk, tau, quota, factor, topk)
    g_ids, g_flags, g_c, g_a, g_counts = run_unmask(z, dt, flags_blk, tau, step, T, factor=factor,
                                                    topk=topk)
    excluded = 0
    for i in range(b):
        m = flags_blk[i] != 0
        # identical logits on both sides: argmax (lowest id on ties) must agree exactly
        np.testing.assert_array_equal(g_a[i][m], r_a[i][m])
        np.testing.assert_allclose(g_c[i][m], r_c[i][m], rtol=2e-5, atol=1e-7)
        if factor > 0 or topk > 0:  # the whole set at once, unless the choice is a near-tie
            fragile = (cut_fragile(r_c[i][m], int(r_com[i].sum())) if topk > 0 else
                       factor_fragile(r_c[i][m], factor, int(r_com[i].sum())))
            if fragile:
                excluded += 1
                continue
            np.testing.assert_array_equal(g_flags[i], r_flags[i])
            np.testing.assert_array_equal(g_ids[i][r_com[i]], r_a[i][r_com[i]])
            assert g_counts[i, 0] == r_com[i].sum() and g_counts[i, 1] == r_left[i]
            continue
        near = m & (np.abs(r_c[i] - tau) < NEAR)
        fallback = (m & (r_c[i] >= tau)).sum() < quota[i]
        if fallback:
            mc = np.sort(r_c[i][m])[::-1]
            if len(mc) > quota[i] and mc[quota[i] - 1] - mc[quota[i]] < NEAR:
                excluded += 1
                continue
        ok = ~near
        np.testing.assert_array_equal(g_flags[i][ok], r_flags[i][ok])
        np.testing.assert_array_equal(g_ids[i][ok & r_com[i]], r_a[i][ok & r_com[i]])
        if not near.any():
            assert g_counts[i, 0] == r_com[i].sum() and g_counts[i, 1] == r_left[i]
        excluded += int(near.sum())
    return excluded


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("tau", [0.5, 0.9, 1.5])
def test_unmask_logits_small(dt, tau):
    rng = np.random.default_rng(4)
    b, B, V = 3, 8, 512
    z = (rng.standard_normal((b, B, V)) * 6).astype(np.float32)
    z[0, 2, 100] = z[0, 2, 101] = 40.0  # an exact tie: the lower id wins
    if dt == "bf16":
        z = synth.f32_to_bf16_bits(z)
    flags = np.ones((b, B), np.uint8)
    flags[1, ::2] = 0
    flags[2] = 0
    flags[2, 5] = 1
    check_unmask(z, dt, flags, tau)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_unmask_logits_nonfinite_and_cross_chunk_tie(dt):
    """The documented handling of special logits, over a vocabulary of several
    16384-logit chunks with a ragged last one: NaN counts as -inf; a row whose
    maximum is +inf gets confidence 1/(number of +inf) and the first of them;
    an exact tie split across chunks goes to the lower id."""
    rng = np.random.default_rng(9)
    b, B, V = 2, 4, 40000
    z = (rng.standard_normal((b, B, V)) * 6).astype(np.float32)
    z[0, 1, 100] = z[0, 1, 30000] = 50.0
    z[0, 2, 17] = np.nan
    z[0, 2, 39999] = np.nan
    z[1, 0, 5] = z[1, 0, V - 1] = np.inf
    z[1, 0, 20000] = np.nan
    if dt == "bf16":
        z = synth.f32_to_bf16_bits(z)
    zf = om.as_f64(z)
    flags = np.ones((b, B), np.uint8)
    _, _, g_c, g_a, _ = run_unmask(z, dt, flags, 2.0)
    zs = np.where(np.isnan(zf), -np.inf, zf)
    for i in range(b):
        for j in range(B):
            row = zs[i, j]
            m = row.max()
            if m == np.inf:
                c_ref, a_ref = 1.0 / (row == m).sum(), int(np.argmax(row == m))
            else:
                c_ref, a_ref = 1.0 / np.exp(row - m).sum(), int(np.argmax(row))
            assert g_a[i, j] == a_ref, (i, j)
            np.testing.assert_allclose(g_c[i, j], c_ref, rtol=2e-5, atol=1e-7)
    assert g_a[0, 1] == 100 and g_a[1, 0] == 5 and g_c[1, 0] == 0.5


@pytest.mark.gpu
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("b", [11, 22])
def test_unmask_logits_many_rows_ragged(dt, b):
    """Hundreds of rows (352 and 704) over a 40000-id vocabulary: three
    16384-logit chunks, the last one partial. Ties across chunks go to the
    lower id, a maximum in the partial chunk is found, and rows no longer
    masked are skipped."""
    rng = np.random.default_rng(11 + b)
    B, V = 32, 40000
    z = (rng.standard_normal((b, B, V)) * 6).astype(np.float32)
    z[0, 1, 100] = z[0, 1, 35000] = 50.0    # chunks 0 and 2
    z[0, 3, 20] = z[0, 3, 16400] = 50.0     # chunks 0 and 1
    z[0, 2, 39999] = 50.0                   # the partial chunk
    if dt == "bf16":
        z = synth.f32_to_bf16_bits(z)
    flags = (rng.random((b, B)) < 0.7).astype(np.uint8)
    flags[0, 1:4] = 1
    check_unmask(z, dt, flags, 0.9)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("factor", [0.7, 1.0, 1.9])
def test_unmask_logits_factor_small(dt, factor):
    """Factor strategy ([commentary] 3.4.3) on confidences spread from low to
    near 1: several sequences, some positions already committed, one
    sequence with a single masked position."""
    rng = np.random.default_rng(int(factor * 10))
    b, B, V = 4, 16, 512
    z = (rng.standard_normal((b, B, V)) * rng.uniform(1, 14, (b, B, 1))).astype(np.float32)
    if dt == "bf16":
        z = synth.f32_to_bf16_bits(z)
    flags = np.ones((b, B), np.uint8)
    flags[1, ::3] = 0
    flags[3] = 0
    flags[3, 7] = 1
    n_ex = check_unmask(z, dt, flags, 0.9, factor=factor)
    print(f"factor {factor} {dt}: {n_ex} sequences excluded")
    assert n_ex < b


@pytest.mark.parametrize("scale", synth.SWEEP_UNMASK["scales"])
@pytest.mark.parametrize("frac", synth.SWEEP_UNMASK["masked_fracs"])
@pytest.mark.parametrize("factor", [0.7, 1.0, 1.9])
def test_unmask_logits_factor_sweep(scale, frac, factor):
    cfg = synth.SWEEP_UNMASK
    z = synth.sweep_logits(cfg["batch"], cfg["block"], cfg["vocab"], scale, cfg["seed"])
    flags = synth.sweep_masked(cfg["batch"], cfg["block"], frac, cfg["seed"])
    n_ex = check_unmask(z, "bf16", flags, 0.9, factor=factor)
    print(f"factor sweep scale={scale} frac={frac} f={factor}: {n_ex} sequences excluded")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("k", [1, 3, 40])
def test_unmask_logits_topk(dt, k):
    """Fixed top-K: the k most confident masked positions (all when fewer)."""
    rng = np.random.default_rng(k)
    b, B, V = 3, 16, 512
    z = (rng.standard_normal((b, B, V)) * rng.uniform(1, 14, (b, B, 1))).astype(np.float32)
    if dt == "bf16":
        z = synth.f32_to_bf16_bits(z)
    flags = np.ones((b, B), np.uint8)
    flags[1, ::2] = 0
    n_ex = check_unmask(z, dt, flags, 0.9, topk=k)
    assert n_ex < b


@pytest.mark.parametrize("scale", synth.SWEEP_UNMASK["scales"])
@pytest.mark.parametrize("frac", synth.SWEEP_UNMASK["masked_fracs"])
def test_unmask_logits_topk_sweep(scale, frac):
    cfg = synth.SWEEP_UNMASK
    z = synth.sweep_logits(cfg["batch"], cfg["block"], cfg["vocab"], scale, cfg["seed"])
    flags = synth.sweep_masked(cfg["batch"], cfg["block"], frac, cfg["seed"])
    check_unmask(z, "bf16", flags, 0.9, topk=4)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("step", [0, 3, 5])
def test_unmask_logits_sampling(dt, step):
    """Stochastic tau-leaping ([commentary] 3.4.1): the fill decisions equal
    the oracle's exactly (they depend on the draws alone), and every filled
    position holds the oracle's Gumbel-max draw unless that draw is a near-tie."""
    from block_wise_kv_amd import fdllm as F
    from tests.helpers import sample_fragile
    rng = np.random.default_rng(100 + step)
    b, B, V, T, blk, seed = 3, 16, 2000, 6, 40, 12345
    z = (rng.standard_normal((b, B, V)) * rng.uniform(0.5, 4, (b, B, 1))).astype(np.float32)
    if dt == "bf16":
        z = synth.f32_to_bf16_bits(z)
    zf = om.as_f64(z)
    flags = (rng.random((b, B)) < 0.8).astype(np.uint8)
    r_ids, r_flags, _, _, r_com, _ = od.unmask_step(zf, np.full((b, B), -1), flags, 0.9, 1, sampling=True,
                                                    seed=seed, blk_start=blk, step=step, T=T)
    x = np.full((b, blk + B), 7, np.int32)
    x[:, blk:] = -1
    fl = np.zeros((b, blk + B), np.uint8)
    fl[:, blk:] = flags
    tx, tf = torch.from_numpy(x).cuda(), torch.from_numpy(fl).cuda()
    conf = torch.zeros(b, B, device="cuda")
    am = torch.zeros(b, B, dtype=torch.int32, device="cuda")
    counts = torch.zeros(b, 2, dtype=torch.int32, device="cuda")
    ws = torch.zeros(F.fdllm_unmask_logits_workspace(b, B, V), dtype=torch.uint8, device="cuda")
    tz = torch.from_numpy(z.view(np.int16) if z.dtype == np.uint16 else z).cuda()
    F.fdllm_confidence_unmask_logits(tz, F.BF16 if dt == "bf16" else F.F32, tx, tf, b, blk + B, blk, B, V,
                                     0.9, step, T, conf, am, counts, ws, sampling=True, seed=seed)
    torch.cuda.synchronize()
    gx, gf = tx.cpu().numpy()[:, blk:], tf.cpu().numpy()[:, blk:]
    np.testing.assert_array_equal(gf, r_flags)
    compared = 0
    for i in range(b):
        for j in np.flatnonzero(r_com[i]):
            if sample_fragile(zf[i, j], seed, i, blk + j, step):
                continue
            assert gx[i, j] == r_ids[i, j], (i, j)
            compared += 1
    assert compared > 0


def test_unmask_logits_quota_when_budget_is_short():
    rng = np.random.default_rng(5)
    z = (rng.standard_normal((2, 16, 256)) * 2).astype(np.float32)
    flags = np.ones((2, 16), np.uint8)
    check_unmask(z, "f32", flags, 1.5, step=2, T=4)   # quota ceil(16 / 2) = 8


@pytest.mark.parametrize("scale", synth.SWEEP_UNMASK["scales"])
@pytest.mark.parametrize("frac", synth.SWEEP_UNMASK["masked_fracs"])
@pytest.mark.parametrize("tau", synth.SWEEP_UNMASK["taus"])
def test_unmask_logits_sweep(scale, frac, tau):
    cfg = synth.SWEEP_UNMASK
    z = synth.sweep_logits(cfg["batch"], cfg["block"], cfg["vocab"], scale, cfg["seed"])
    flags = synth.sweep_masked(cfg["batch"], cfg["block"], frac, cfg["seed"])
    n_ex = check_unmask(z, "bf16", flags, tau)
    print(f"unmask sweep scale={scale} frac={frac} tau={tau}: {n_ex} positions excluded")
