"""Measurement helpers (host side, not on the hot path).

The adjusted Rand index (P1 "The metric": pair-counting agreement of two
labelings, 1 when identical, about 0 when unrelated), computed from the
contingency table (Hubert and Arabie 1985).
"""
from __future__ import annotations

import numpy as np


def adjusted_rand_index(a, b) -> float:
    a = np.asarray(a).ravel()
    b = np.asarray(b).ravel()
    if a.size != b.size:
        raise ValueError("labelings differ in length")
    n = a.size
    if n < 2:
        return 1.0
    _, ia = np.unique(a, return_inverse=True)
    _, ib = np.unique(b, return_inverse=True)
    table = np.bincount(ia * (ib.max() + 1) + ib, minlength=(ia.max() + 1) * (ib.max() + 1))
    table = table.reshape(ia.max() + 1, ib.max() + 1).astype(np.float64)
    pairs = lambda x: (x * (x - 1.0) / 2.0).sum()  # noqa: E731
    s_ij = pairs(table)
    s_a = pairs(table.sum(axis=1))
    s_b = pairs(table.sum(axis=0))
    total = n * (n - 1.0) / 2.0
    expected = s_a * s_b / total
    top = 0.5 * (s_a + s_b)
    if top == expected:
        return 1.0
    return float((s_ij - expected) / (top - expected))
