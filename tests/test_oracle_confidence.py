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
