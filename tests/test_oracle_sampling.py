"""Pins of the tau-leaping sampler (oracle/sampling.py): the generator
against numpy's Philox-4x64-10, the Gumbel-max draw against the softmax it
must sample, the fill rate against its probability, and the decode loop."""
import numpy as np
import pytest
from scipy.special import softmax

from block_wise_kv_amd import synth
from oracle import decode as od
from oracle import model as om
from oracle import sampling as smp


def test_philox_matches_numpy():
    # numpy's Philox advances its counter before each block of four words,
    # so its n-th block is the generator at counter n + 1
    for key in ([0, 0], [0x1234, 0xABCD], [2**64 - 1, 7]):
        g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.zeros(4, dtype=np.uint64))
        raw = g.random_raw(4 * 6).reshape(6, 4)
        ctr = np.zeros((6, 4), dtype=np.uint64)
        ctr[:, 0] = np.arange(1, 7, dtype=np.uint64)
        np.testing.assert_array_equal(smp.philox4x64(ctr, key), raw)
    # a counter with every word in use (numpy's 256-bit counter carries upward)
    g = np.random.Philox(key=np.array([5, 9], dtype=np.uint64),
                         counter=np.array([2**64 - 1, 3, 0, 11], dtype=np.uint64))
    np.testing.assert_array_equal(smp.philox4x64(np.array([[0, 4, 0, 11]], dtype=np.uint64), (5, 9))[0],
                                  g.random_raw(4))


def test_gumbel_max_samples_the_softmax():
    z = np.array([2.0, 0.5, -1.0, 1.5, 0.0])
    p = softmax(z)
    n = 20000
    draws = np.array([smp.sample_token(z, seed=3, seq=0, pos=i % 997, step=i // 997) for i in range(n)])
    freq = np.bincount(draws, minlength=len(z)) / n
    sigma = np.sqrt(p * (1 - p) / n)
    assert np.all(np.abs(freq - p) < 4 * sigma), (freq, p)


def test_fill_rate_and_last_step():
    for T, j in ((8, 0), (8, 5), (32, 30)):
        p = 1.0 / (T - j)
        fills = np.mean([smp.fill_uniform(11, 0, pos, j) < p for pos in range(4000)])
        assert abs(fills - p) < 4 * np.sqrt(p * (1 - p) / 4000)
    z = np.zeros((6, 9))
    masked = np.array([1, 1, 0, 1, 1, 1], np.uint8)
    sel, tok = smp.tau_leap_step(z, masked, 40, 7, 8, seed=1)   # step T - 1: probability 1
    assert sel.tolist() == [0, 1, 3, 4, 5] and tok[2] == -1 and (tok[masked == 1] >= 0).all()


def test_sampling_is_a_function_of_the_seed():
    z = np.random.default_rng(0).standard_normal((4, 50))
    masked = np.ones(4, np.uint8)
    a = smp.tau_leap_step(z, masked, 100, 1, 4, seed=5)
    b = smp.tau_leap_step(z, masked, 100, 1, 4, seed=5)
    c = smp.tau_leap_step(z, masked, 100, 1, 4, seed=6)
    assert a[0].tolist() == b[0].tolist() and a[1].tolist() == b[1].tolist()
    assert a[1].tolist() != c[1].tolist() or a[0].tolist() != c[0].tolist()


def test_sampling_decode_invariants():
    shape = synth.ModelShape(2, 64, 2, 2, 32, 128, 97, 96, "f32")
    m = om.Model(shape, synth.make_weights(shape, 5, norm_gain_std=0.1, threads=2))
    prompt = synth.make_prompt(shape, 8, seed=3)[0]
    st = synth.DecodeSettings(8, 16, 4, 16, True, False, 0.9, sampling=True, seed=9)
    x, flags, steps = od.decode(m, prompt, st)
    assert not flags.any() and np.all((x >= 0) & (x < shape.vocab))
    per_block = {}
    for r in steps:
        per_block[r.block] = per_block.get(r.block, 0) + 1
        s = 8 + r.block * 4
        np.testing.assert_array_equal(x[r.selected], r.sampled[r.selected - s])
    assert all(n <= 4 for n in per_block.values())
    x2, _, _ = od.decode(m, prompt, st)
    np.testing.assert_array_equal(x, x2)


def test_gumbel_noise_follows_the_gumbel_law():
    """G = -log(-log u) with u uniform on (0, 1) is standard Gumbel: its CDF is
    exp(-exp(-g)) (Kolmogorov-Smirnov against scipy's gumbel_r), its mean the
    Euler-Mascheroni constant, and every value is finite."""
    from scipy import stats
    g = np.concatenate([smp.gumbel_noise(7, 0, pos, 0, 4096) for pos in range(25)])
    assert np.all(np.isfinite(g))
    assert stats.kstest(g, stats.gumbel_r.cdf).pvalue > 1e-3
    assert abs(g.mean() - np.euler_gamma) < 4 * (np.pi / np.sqrt(6)) / np.sqrt(g.size)
