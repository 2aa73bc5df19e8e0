"""K/V drift diagnostics, float64. Test infrastructure, like the rest of
``oracle/``: only tests, the smoke check and the benchmark's CPU baseline use it.

[commentary] §3.4.2 "The Empirical Justification: Cosine Similarity of KV
Activations" (Figure 3): the approximate cache is justified by measuring how
similar a token's key-value activations are at two decoding steps, averaged
over tokens. Reading (the pages do not fix the vector): per token and layer,
the cosine over the token's keys of all kv heads, and separately over its
values; a zero vector gives 0.
"""
from __future__ import annotations

import numpy as np


def cosine_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Cosine similarity of matching rows of a and b ([N][...] each, the
    trailing axes flattened); 0 where either row is all zero."""
    a = np.asarray(a, dtype=np.float64).reshape(a.shape[0], -1)
    b = np.asarray(b, dtype=np.float64).reshape(b.shape[0], -1)
    dot = np.einsum("ij,ij->i", a, b)
    den = np.sqrt(np.einsum("ij,ij->i", a, a) * np.einsum("ij,ij->i", b, b))
    out = np.zeros(a.shape[0])
    nz = den > 0
    out[nz] = dot[nz] / den[nz]
    return out


def kv_cosine(layer_a, layer_b, rows=None):
    """(cos of K, cos of V) per token between two snapshots of one layer's
    cache, each (K [N][Hkv][D], V [N][Hkv][D]) as ``model.forward_full``
    returns them; ``rows`` selects tokens (default: all)."""
    (ka, va), (kb, vb) = layer_a, layer_b
    sel = slice(None) if rows is None else rows
    return cosine_rows(ka[sel], kb[sel]), cosine_rows(va[sel], vb[sel])


def drift_matrix(snapshots, rows) -> np.ndarray:
    """Figure 3's heatmap: entry (i, j) is the mean over ``rows`` of the K/V
    cosine between snapshot i and snapshot j (K and V averaged). Each
    snapshot is one layer's (K, V)."""
    n = len(snapshots)
    m = np.ones((n, n))
    for i in range(n):
        for j in range(i + 1, n):
            ck, cv = kv_cosine(snapshots[i], snapshots[j], rows)
            m[i, j] = m[j, i] = 0.5 * (ck.mean() + cv.mean())
    return m
