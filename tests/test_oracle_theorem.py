"""Theorem 1 (greedy equivalence of joint and product-of-marginals decoding),
brute force on tiny vocabularies (CPU only)."""
import itertools

import numpy as np
import pytest

from oracle import decode as od
from oracle import theorem as th


def _joint_with_confident_mode(rng, n, V, eps):
    """A random joint whose mode x* = (0,..,0) has every marginal > 1 - eps."""
    r = rng.random((V,) * n) ** 3
    r /= r.sum()
    point = np.zeros((V,) * n)
    point[(0,) * n] = 1.0
    # smallest mixing weight lam with lam + (1-lam) * r_marg_j(0) > 1 - eps for all j
    rm = [m[0] for m in th.marginals(r)]
    lam = max(max((1 - eps - m) / (1 - m) for m in rm), 0.0)
    lam = min(1.0, lam + rng.random() * (1 - lam) * 0.5 + 1e-9)
    return lam * point + (1 - lam) * r


@pytest.mark.parametrize("n,V", [(1, 2), (2, 2), (2, 3), (3, 2), (3, 3), (4, 2)])
def test_greedy_equivalence_when_condition_holds(n, V):
    rng = np.random.default_rng(n * 10 + V)
    eps = 1.0 / (n + 1)
    for _ in range(300):
        e = eps * rng.random() ** 0.3  # eps' <= 1/(n+1)
        p = _joint_with_confident_mode(rng, n, V, e)
        assert all(m[0] > 1 - e for m in th.marginals(p))
        q = th.product_of_marginals(p)
        assert th.argmax_tuple(p) == (0,) * n
        assert th.argmax_tuple(q) == (0,) * n


@pytest.mark.parametrize("n,V", [(1, 2), (2, 2), (2, 3), (3, 2), (4, 2)])
def test_bound_is_tight(n, V):
    p = th.tightness_joint(n, V, delta=1e-3)
    eps = 1.0 / (n + 1) + 2e-3
    assert all(m[0] > 1 - eps for m in th.marginals(p))
    assert th.argmax_tuple(p) != (0,) * n
    if n >= 2:  # with one position the joint is its own marginal
        assert th.argmax_tuple(th.product_of_marginals(p)) == (0,) * n


@pytest.mark.parametrize("n,V", [(1, 2), (2, 2), (2, 3), (3, 2)])
def test_lp_worst_case(n, V):
    b = 1.0 / (n + 1)
    assert th.worst_case_gap(n, V, b * 0.9) < -1e-6
    assert abs(th.worst_case_gap(n, V, b)) < 1e-9
    assert th.worst_case_gap(n, V, b * 1.1) > 1e-6


def test_threshold_selection_agrees_with_joint_argmax():
    """Tokens the threshold rule commits together equal the argmax of the
    joint restricted to those positions when (|S| + 1)(1 - min c_S) < 1."""
    rng = np.random.default_rng(9)
    n, V, hits = 3, 3, 0
    for _ in range(400):
        p = _joint_with_confident_mode(rng, n, V, rng.random() * 0.3)
        margs = th.marginals(p)
        z = np.log(np.maximum(np.array(margs), 1e-300))
        c, a = od.confidence(z)
        sel = od.select(c, np.ones(n), 0.8)
        if (len(sel) + 1) * (1 - c[sel].min()) >= 1:
            continue
        rest = tuple(j for j in range(n) if j not in set(sel.tolist()))
        ps = p.sum(axis=rest) if rest else p
        assert th.argmax_tuple(ps) == tuple(int(a[j]) for j in sel)
        hits += 1
    assert hits > 50
