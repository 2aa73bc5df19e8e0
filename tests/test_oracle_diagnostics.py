"""Pins of the K/V drift diagnostics (oracle/diagnostics.py)."""
import numpy as np
from scipy.spatial.distance import cosine as scipy_cosine_distance

from oracle import diagnostics as dg


def test_cosine_rows_matches_scipy():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((7, 3, 5))
    b = a + 0.3 * rng.standard_normal((7, 3, 5))
    got = dg.cosine_rows(a, b)
    want = [1.0 - scipy_cosine_distance(a[i].ravel(), b[i].ravel()) for i in range(7)]
    np.testing.assert_allclose(got, want, rtol=1e-12)


def test_cosine_rows_closed_forms():
    a = np.array([[1.0, 0.0], [3.0, 4.0], [1.0, 2.0], [0.0, 0.0], [2.0, -1.0]])
    b = np.array([[1.0, 1.0], [6.0, 8.0], [-1.0, -2.0], [5.0, 1.0], [1.0, 2.0]])
    np.testing.assert_allclose(dg.cosine_rows(a, b), [1 / np.sqrt(2), 1.0, -1.0, 0.0, 0.0], atol=1e-15)


def test_kv_cosine_and_drift_matrix():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((6, 2, 4))
    v = rng.standard_normal((6, 2, 4))
    same = dg.kv_cosine((k, v), (k.copy(), 2.5 * v), rows=slice(1, 5))
    np.testing.assert_allclose(same[0], 1.0)
    np.testing.assert_allclose(same[1], 1.0)
    snaps = [(k, v), (k + 0.1, v), (-k, -v)]
    m = dg.drift_matrix(snaps, slice(0, 6))
    assert m.shape == (3, 3) and np.allclose(np.diag(m), 1.0) and np.allclose(m, m.T)
    np.testing.assert_allclose(m[0, 2], -1.0)
    assert 0.9 < m[0, 1] < 1.0
