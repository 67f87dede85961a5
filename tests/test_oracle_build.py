"""Pins for the oracle's dependence-matrix builders (CPU only).

|corr| is pinned to numpy.corrcoef (a library routine), the TPDM to its
invariants and to a hand-worked case under tests/golden/.
"""
import math
import os

import numpy as np
import pytest

import oracle
from symmetric_nmf_clustering_amd import synth


def _load_tpdm_case(golden_dir):
    X, ranks, days = [], [], []
    meta = {}
    with open(os.path.join(golden_dir, "tpdm_t4_n2.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "X":
                X.append([float(v) for v in vals])
            elif key == "ranks":
                ranks.append([int(v) for v in vals])
            elif key == "days":
                days = [int(v) for v in vals]
            else:
                meta[key] = float(vals[0])
    return np.array(X), np.array(ranks), days, meta


def test_abs_corr_matches_corrcoef():
    w = synth.gaussian_blocks(n=96, k=4, T=40, seed=3)
    S = oracle.abs_corr(w.X)
    ref = np.abs(np.corrcoef(w.X.astype(np.float64), rowvar=False))
    np.testing.assert_allclose(S, ref, rtol=0, atol=1e-12)


def test_abs_corr_invariants():
    w = synth.student_factor(n=300, k=4, T=60, seed=5, min_size=20)
    S = oracle.abs_corr(w.X)
    assert np.array_equal(S, S.T) or np.abs(S - S.T).max() < 1e-15
    np.testing.assert_allclose(np.diag(S), 1.0, atol=1e-12)
    assert S.min() >= 0.0 and S.max() <= 1.0 + 1e-12


def test_abs_corr_rows_consistent():
    w = synth.gaussian_blocks(n=64, k=4, T=30, seed=1)
    rows = [0, 5, 63, 17]
    np.testing.assert_allclose(oracle.abs_corr_rows(w.X, rows), oracle.abs_corr(w.X)[rows], atol=1e-14)


def test_abs_corr_scale_shift_invariant():
    # correlation ignores per-column affine maps with positive scale
    w = synth.gaussian_blocks(n=32, k=4, T=25, seed=2)
    X2 = w.X.astype(np.float64) * np.linspace(0.5, 3.0, 32) + np.linspace(-2, 2, 32)
    np.testing.assert_allclose(oracle.abs_corr(X2), oracle.abs_corr(w.X), atol=1e-12)


def test_constant_column_rejected():
    X = np.random.default_rng(0).standard_normal((10, 4))
    X[:, 2] = 1.5
    with pytest.raises(ValueError):
        oracle.abs_corr(X)


def test_tpdm_hand_case(golden_dir):
    X, ranks, days, meta = _load_tpdm_case(golden_dir)
    theta, sel, m = oracle.tpdm_angles(X, meta["tail_frac"])
    assert m == 2
    assert list(sel) == days
    a = math.sqrt(-1.0 / math.log(0.6))
    b = math.sqrt(-1.0 / math.log(0.4))
    den = a * a + b * b
    S_hand = np.array([[(0.5 + a * a / den) / 2, (0.5 + a * b / den) / 2],
                       [(0.5 + a * b / den) / 2, (0.5 + b * b / den) / 2]])
    S = oracle.tpdm(X, meta["tail_frac"])
    np.testing.assert_allclose(S, S_hand, rtol=1e-14, atol=0)
    # the ranks the derivation uses, via the Frechet values
    xt = np.sqrt(-1.0 / np.log(ranks / (X.shape[0] + 1.0)))
    np.testing.assert_allclose(theta[0], xt[days[0]] / np.linalg.norm(xt[days[0]]), rtol=1e-14)


def test_tpdm_invariants():
    w = synth.student_factor_stress(n=400, k=6, T=80, seed=4, min_size=20)
    theta, days, m = oracle.tpdm_angles(w.X, 0.05)
    assert m == math.ceil(0.05 * 80)
    S = oracle.tpdm(w.X, 0.05)
    assert S.min() > 0.0
    np.testing.assert_allclose(S, S.T, atol=1e-16)
    assert abs(np.trace(S) - 1.0) < 1e-12          # unit theta rows, 1/m scaling
    ev = np.linalg.eigvalsh(S)
    assert ev.min() > -1e-12                         # PSD
    assert (np.abs(ev) > 1e-10).sum() <= m           # rank <= m
    np.testing.assert_allclose(np.linalg.norm(theta, axis=1), 1.0, atol=1e-14)


def test_tpdm_picks_the_stressed_days():
    # a -5 sigma joint crash on every member of 4 groups produces the largest
    # loss radii, so the crash days are among the selected extreme days
    w = synth.student_factor_stress(n=600, k=8, T=120, seed=7, min_size=30)
    _, days, m = oracle.tpdm_angles(w.X, 0.05)
    d0 = w.meta["stress_day0"]
    stressed = set(range(d0, d0 + w.meta["stress_days"]))
    assert len(stressed & set(days.tolist())) >= min(m, len(stressed)) - 1


def test_tpdm_rows_consistent():
    w = synth.student_factor_stress(n=200, k=4, T=60, seed=2, min_size=20)
    rows = [3, 0, 199]
    np.testing.assert_allclose(oracle.tpdm_rows(w.X, rows), oracle.tpdm(w.X)[rows], atol=1e-15)


def test_shifted_window_continues_the_stream():
    """student_factor_next: the window one day on shares T - 1 days with the
    original window, keeps its groups, and adds a day of the same recipe."""
    from symmetric_nmf_clustering_amd import synth
    a = synth.student_factor(n=600, k=6, T=50, seed=4, min_size=20)
    b = synth.student_factor_next(n=600, k=6, T=50, seed=4, shift=1, min_size=20)
    c = synth.student_factor_next(n=600, k=6, T=50, seed=4, shift=3, min_size=20)
    assert b.X.shape == a.X.shape and np.array_equal(b.X[:-1], a.X[1:])
    assert np.array_equal(c.X[:-3], a.X[3:]) and np.array_equal(c.X[-3], b.X[-1])
    assert np.array_equal(b.labels, a.labels)
    # the new day carries the planted groups: members of a group co-move
    S_new = oracle.abs_corr(np.vstack([a.X, c.X[-3:]]))
    same = b.labels[:, None] == b.labels[None, :]
    assert S_new[same].mean() > 3 * S_new[~same].mean()
