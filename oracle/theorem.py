"""Joint vs product-of-marginals greedy decoding on tiny vocabularies.

[commentary] §3.4.3 "Theorem 1: Formal Justification", part 1: for n
positions with a candidate x* whose every marginal exceeds 1 - eps, if
(n + 1) eps <= 1 then the argmax of the joint p and the argmax of the
product of its marginals q are both x*; the bound is tight (a joint that puts
slightly more than 1/(n+1) on each of the n sequences that differ from x* in
one position moves the joint argmax away from x*).

Joints are numpy arrays of shape (V,) * n holding probabilities.
"""
from __future__ import annotations

import itertools

import numpy as np


def marginals(p: np.ndarray):
    n = p.ndim
    return [p.sum(axis=tuple(a for a in range(n) if a != j)) for j in range(n)]


def product_of_marginals(p: np.ndarray) -> np.ndarray:
    q = np.ones(())
    for m in marginals(p):
        q = np.multiply.outer(q, m)
    return q


def argmax_tuple(p: np.ndarray):
    """Index tuple of the largest entry (first in C order on ties)."""
    return tuple(int(i) for i in np.unravel_index(int(np.argmax(p)), p.shape))


def is_unique_argmax(p: np.ndarray, idx) -> bool:
    v = p[idx]
    others = np.delete(p.reshape(-1), np.ravel_multi_index(idx, p.shape))
    return bool(np.all(others < v))


def tightness_joint(n: int, V: int, delta: float) -> np.ndarray:
    """Joint with x* = (0,...,0): each one-position deviation gets
    1/(n+1) + delta, x* gets the rest. Needs n/(n+1) + n*delta <= 1."""
    p = np.zeros((V,) * n)
    dev = 1.0 / (n + 1) + delta
    for j in range(n):
        idx = [0] * n
        idx[j] = 1
        p[tuple(idx)] = dev
    p[(0,) * n] = 1.0 - n * dev
    assert p[(0,) * n] >= 0
    return p


def worst_case_gap(n: int, V: int, eps: float) -> float:
    """max over joints p with p_j(x*_j) >= 1 - eps for all j of
    max_{z != x*} p(z) - p(x*), by linear programming (x* = all zeros)."""
    from scipy.optimize import linprog

    cells = list(itertools.product(range(V), repeat=n))
    ncell = len(cells)
    xstar = cells.index((0,) * n)
    best = -np.inf
    for zi in range(ncell):
        if zi == xstar:
            continue
        c = np.zeros(ncell)
        c[zi] = -1.0
        c[xstar] = 1.0
        a_ub, b_ub = [], []
        for j in range(n):  # -sum_{cells with z_j = 0} p <= -(1 - eps)
            row = np.array([-1.0 if cell[j] == 0 else 0.0 for cell in cells])
            a_ub.append(row)
            b_ub.append(-(1.0 - eps))
        res = linprog(c, A_ub=np.array(a_ub), b_ub=np.array(b_ub),
                      A_eq=np.ones((1, ncell)), b_eq=[1.0], bounds=[(0, 1)] * ncell,
                      method="highs")
        if res.status == 0:
            best = max(best, -res.fun)
    return float(best)
