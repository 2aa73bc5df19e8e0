"""Pins of confidence scoring and threshold selection (CPU only)."""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import decode as od


def test_confidence_matches_scipy_softmax():
    z = np.random.default_rng(0).standard_normal((6, 500)) * 7
    c, a = od.confidence(z)
    p = softmax(z, axis=-1)
    np.testing.assert_allclose(c, p.max(axis=-1), rtol=1e-12)
    np.testing.assert_array_equal(a, np.argmax(p, axis=-1))


def test_confidence_worked_examples_from_the_pages():
    # a token at 0.97 with the rest spread -> confidence 0.97;
    # an uncertain split 0.3 / 0.3 / 0.4 -> confidence 0.4 (commentary §3.4.3)
    p1 = np.array([0.97, 0.01, 0.01, 0.01])
    p2 = np.array([0.3, 0.3, 0.4])
    c1, a1 = od.confidence(np.log(p1)[None])
    c2, a2 = od.confidence(np.log(p2)[None])
    assert abs(c1[0] - 0.97) < 1e-12 and a1[0] == 0
    assert abs(c2[0] - 0.4) < 1e-12 and a2[0] == 2


def test_argmax_ties_take_lowest_id():
    z = np.array([[0.0, 5.0, 1.0, 5.0]])
    c, a = od.confidence(z)
    assert a[0] == 1


def test_top2_gap_closed_form():
    p = np.array([[0.5, 0.3, 0.2]])
    np.testing.assert_allclose(od.top2_prob_gap(np.log(p)), [0.2], rtol=1e-12)


def test_select_threshold_rule():
    # tau = 0.9: the 0.97 position commits, the 0.4 one does not
    c = np.array([0.97, 0.4])
    np.testing.assert_array_equal(od.select(c, np.array([1, 1]), 0.9), [0])
    # several above tau: all of them
    c = np.array([0.95, 0.2, 0.91, 0.9, 0.5])
    np.testing.assert_array_equal(od.select(c, np.ones(5), 0.9), [0, 2, 3])  # >= tau


def test_select_progress_guarantee():
    c = np.array([0.3, 0.6, 0.5, 0.6])
    # none reaches tau -> exactly one, the most confident, lower position on ties
    np.testing.assert_array_equal(od.select(c, np.ones(4), 0.9), [1])
    # tau > 1 is never met -> exactly one per step
    np.testing.assert_array_equal(od.select(np.ones(4) * 0.999, np.ones(4), 1.5), [0])


def test_select_ignores_unmasked_positions():
    c = np.array([0.99, 0.95, 0.2])
    np.testing.assert_array_equal(od.select(c, np.array([0, 1, 1]), 0.9), [1])
    np.testing.assert_array_equal(od.select(c, np.array([1, 0, 0]), 0.999), [0])
    assert od.select(c, np.zeros(3), 0.5).size == 0


def test_select_quota():
    c = np.array([0.1, 0.8, 0.95, 0.7])
    np.testing.assert_array_equal(od.select(c, np.ones(4), 0.9, quota=3), [1, 2, 3])
    np.testing.assert_array_equal(od.select(c, np.ones(4), 0.5, quota=2), [1, 2, 3])


def test_unmask_step_batch():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((3, 8, 50)) * 6
    ids = np.full((3, 8), 49)
    flags = np.array([[1] * 8, [0, 1] * 4, [0] * 8], dtype=np.uint8)
    new_ids, new_flags, c, a, com, left = od.unmask_step(z, ids, flags, 0.9)
    for i in range(3):
        ci, ai = od.confidence(z[i])
        sel = od.select(ci, flags[i], 0.9)
        assert set(np.flatnonzero(com[i])) == set(sel.tolist())
        np.testing.assert_array_equal(new_ids[i, sel], ai[sel])
        assert left[i] == flags[i].sum() - len(sel)
    assert com[0].sum() >= 1 and com[1].sum() >= 1 and com[2].sum() == 0


# ---- factor strategy ([commentary] 3.4.3 "From Theorem to Practice: Factor
# Strategy"): largest n with (n+1)(1 - c_(n)) < f, at least one ----

def _factor_brute(c, masked, f):
    """Every prefix size n of the confidence order tested on its own; the
    answer is the largest passing n (at least 1). Also asserts that the
    passing sizes form a prefix 1..n*, which the rule relies on."""
    idx = [i for i in range(len(c)) if masked[i]]
    order = sorted(idx, key=lambda i: (-c[i], i))
    passing = [n for n in range(1, len(order) + 1) if (n + 1) * (1 - c[order[n - 1]]) < f]
    assert passing == list(range(1, len(passing) + 1))
    n = max(passing) if passing else 1
    return sorted(order[:n])


def test_factor_rule_brute_force_over_n():
    rng = np.random.default_rng(17)
    for _ in range(400):
        m = int(rng.integers(1, 9))
        c = rng.uniform(0.3, 1.0, m) ** rng.uniform(0.2, 3.0)
        if rng.random() < 0.3:
            c[rng.integers(0, m, 2)] = c[0]  # equal confidences
        masked = (rng.random(m) < 0.8).astype(np.uint8)
        f = float(rng.choice([0.3, 0.7, 1.0, 1.3, 1.9, 4.0]))
        got = od.select_factor(c, masked, f).tolist()
        if not masked.any():
            assert got == []
            continue
        assert got == _factor_brute(c, masked, f)


def test_factor_rule_worked_shapes_from_the_pages():
    # uniformly high confidences (0.99, 0.98, ...): the bound stays small for
    # many tokens; (6)(1 - 0.5) = 3 stops the set at 4 tokens
    c = np.array([0.99, 0.98, 0.97, 0.96, 0.5])
    assert od.select_factor(c, np.ones(5), 1.0).tolist() == [0, 1, 2, 3]
    # a sharp drop after the top token: (2)(0.05) = 0.1 < 1, (3)(0.4) = 1.2 >= 1
    c = np.array([0.6, 0.95, 0.59])
    assert od.select_factor(c, np.ones(3), 1.0).tolist() == [1]
    # even n = 1 fails ((2)(0.7) = 1.4): the single most confident position
    c = np.array([0.2, 0.3, 0.1])
    assert od.select_factor(c, np.ones(3), 1.0).tolist() == [1]


def test_factor_rule_equal_confidences_closed_form():
    # all m masked confidences equal c0: (n+1)(1-c0) < f  <=>  n < f/(1-c0) - 1,
    # so n* = ceil(f / (1 - c0)) - 2, clamped to [1, m]
    for c0 in (0.5, 0.8, 0.9, 0.93, 0.99):
        for f in (0.7, 1.0, 1.3, 1.9):
            for m in (1, 4, 16):
                eps = 1 - c0
                if abs(f / eps - round(f / eps)) < 1e-9:
                    continue  # on the boundary the strict test is decided by rounding
                n_star = min(m, max(1, int(np.ceil(f / eps)) - 2))
                got = od.select_factor(np.full(m, c0), np.ones(m), f)
                assert got.tolist() == list(range(n_star)), (c0, f, m)


def test_factor_rule_limits_and_quota():
    rng = np.random.default_rng(3)
    c = rng.uniform(0.0, 1.0, 12)
    masked = np.ones(12, np.uint8)
    masked[[2, 5]] = 0
    # a huge factor commits every masked position; a tiny one only the best
    assert od.select_factor(c, masked, 1e9).tolist() == np.flatnonzero(masked).tolist()
    best = max(np.flatnonzero(masked), key=lambda i: (c[i], -i))
    assert od.select_factor(c, masked, 1e-9).tolist() == [best]
    # the quota raises the minimum; the committed set is the top-q
    top4 = sorted(sorted(np.flatnonzero(masked), key=lambda i: (-c[i], i))[:4])
    assert od.select_factor(c, masked, 1e-9, quota=4).tolist() == top4
    # unmasked positions are never chosen, however confident
    c2 = c.copy()
    c2[2] = 1.0
    assert 2 not in od.select_factor(c2, masked, 1e9).tolist()


def test_topk_rule_hand_cases_and_limits():
    c = np.array([0.3, 0.9, 0.3, 0.5, 0.95, 0.1])
    masked = np.array([1, 1, 1, 1, 0, 1], np.uint8)
    assert od.select_topk(c, masked, 1).tolist() == [1]           # 0.95 is not masked
    assert od.select_topk(c, masked, 2).tolist() == [1, 3]
    assert od.select_topk(c, masked, 3).tolist() == [0, 1, 3]     # tie 0.3: lower position first
    assert od.select_topk(c, masked, 99).tolist() == [0, 1, 2, 3, 5]
    assert od.select_topk(c, masked, 2, quota=4).tolist() == [0, 1, 2, 3]
    assert od.select_topk(c, np.zeros(6), 3).tolist() == []


def test_topk_one_equals_threshold_above_one_and_large_k_equals_threshold_zero():
    rng = np.random.default_rng(21)
    for _ in range(200):
        m = int(rng.integers(1, 12))
        c = rng.uniform(0, 1, m)
        masked = (rng.random(m) < 0.7).astype(np.uint8)
        np.testing.assert_array_equal(od.select_topk(c, masked, 1), od.select(c, masked, 1.5))
        np.testing.assert_array_equal(od.select_topk(c, masked, m), od.select(c, masked, 0.0))


def test_unmask_step_factor_matches_select_factor():
    rng = np.random.default_rng(8)
    z = rng.standard_normal((3, 8, 40)) * 4
    flags = (rng.random((3, 8)) < 0.7).astype(np.uint8)
    ids = np.full((3, 8), -1)
    new_ids, new_flags, c, a, com, left = od.unmask_step(z, ids, flags, 0.9, 1, factor=1.0)
    for i in range(3):
        sel = od.select_factor(c[i], flags[i], 1.0)
        assert np.flatnonzero(com[i]).tolist() == sel.tolist()
        assert (new_ids[i, sel] == a[i, sel]).all() and not new_flags[i, sel].any()
