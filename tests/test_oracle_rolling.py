"""Pins for the rolling-window monitoring (P1 "Tracking stability through time
with the Rand index" and the tail/body discussion): the ARI series, the calm
windows, the 3-sigma limit, the cross-sector block means, the warm-started
window chain and the stream generator; and the library's host-side versions
of the same statistics against these pinned definitions."""
import itertools
import math

import numpy as np
import pytest

import oracle
from symmetric_nmf_clustering_amd import rolling, synth


def test_ari_drift_hand_cases():
    a = np.array([0, 0, 1, 1, 2, 2])
    relabeled = np.array([5, 5, 3, 3, 9, 9])  # same partition, other names
    other = np.array([0, 1, 0, 1, 0, 1])
    seq = [a, relabeled, a, other]
    d = oracle.ari_drift(seq, 1)
    assert math.isnan(d[0])
    assert d[1] == 1.0 and d[2] == 1.0
    assert d[3] == pytest.approx(oracle.ari_pairs(a, other), abs=1e-15)
    d2 = oracle.ari_drift(seq, 2)
    assert np.isnan(d2[:2]).all() and d2[2] == 1.0


def test_calm_windows_hand_case():
    # T = 4, switch on day 8: window t holds max(0, t - 4) switched days, so
    # t <= 5 is before the majority flips; day 11 is stressed, held by t = 8..11
    calm = oracle.calm_windows(12, 4, 2, 8, 11, 11)
    assert calm.tolist() == [False, False, True, True, True, True,
                             False, False, False, False, False, False]


def test_control_limit_hand_case():
    v = [np.nan, np.nan, 0.9, 1.0, 0.95, 0.5, 0.85]
    calm = [False, False, True, True, True, False, False]
    limit, mu, sd, flags = oracle.control_limit(v, calm)
    assert mu == pytest.approx(0.95, abs=1e-15)
    assert sd == pytest.approx(0.05, abs=1e-15)
    assert limit == pytest.approx(0.80, abs=1e-14)
    assert flags.tolist() == [False, False, False, False, False, True, False]


def test_cross_block_means_brute_force():
    rng = np.random.default_rng(3)
    n = 14
    A = rng.random((n, n))
    S = (A + A.T) / 2
    lab = rng.integers(0, 4, n)
    lab[:4] = [0, 1, 2, 3]
    groups = [1, 3, 2]
    B = oracle.cross_block_means(S, lab, groups)
    for a, b in itertools.product(range(3), range(3)):
        vals = [S[i, j] for i in range(n) for j in range(n)
                if lab[i] == groups[a] and lab[j] == groups[b]]
        assert B[a, b] == pytest.approx(sum(vals) / len(vals), rel=1e-14)
    np.testing.assert_allclose(B, B.T, rtol=1e-14)


def _small_stream():
    return synth.rolling_stream(n=480, k=6, days=40, switch_day=25, switch_frac=0.1,
                                stress_groups=2, stress_first=31, stress_last=33, seed=7)


def test_rolling_fit_chain():
    """Window 0 is the plain seeded fit; window 1 continues from window 0's H
    with a fresh accumulator (warm start), or restarts from the seed (cold)."""
    st = _small_stream()
    T, k = 30, 6
    warm = oracle.rolling_fit(st.X, k, T, 2, iters=20)
    cold = oracle.rolling_fit(st.X, k, T, 2, iters=20, warm_start=False)
    S0 = oracle.abs_corr(st.window(0, T)).astype(np.float32).astype(np.float64)
    m0 = S0.mean()
    ref0 = oracle.fit_full(S0, oracle.init_uniform(480, k, oracle.init_scale_matched(m0, k), 0),
                           oracle.default_lr(m0, k), 20)
    np.testing.assert_array_equal(warm["H"][0], ref0["H"])
    S1 = oracle.abs_corr(st.window(1, T)).astype(np.float32).astype(np.float64)
    m1 = S1.mean()
    ref1 = oracle.fit_full(S1, ref0["H"], oracle.default_lr(m1, k), 20)
    np.testing.assert_array_equal(warm["H"][1], ref1["H"])
    refc = oracle.fit_full(S1, oracle.init_uniform(480, k, oracle.init_scale_matched(m1, k), 0),
                           oracle.default_lr(m1, k), 20)
    np.testing.assert_array_equal(cold["H"][1], refc["H"])


def test_stream_generator_events():
    st = synth.rolling_stream(n=2000, k=8, days=120, switch_day=70, switch_frac=0.05,
                              stress_groups=2, stress_first=100, stress_last=104, seed=5)
    assert st.X.shape == (120, 2000) and st.X.dtype == np.float32
    assert st.switched.size == 100
    moved = np.flatnonzero(st.labels_before != st.labels_after)
    np.testing.assert_array_equal(moved, st.switched)
    assert len(st.stress_groups) == 2
    mem = np.isin(st.labels_after, st.stress_groups)
    # the shock shows in the stressed days' mean and nowhere else
    assert st.X[100:105, mem].mean() < -4.5
    assert abs(st.X[100:105, ~mem].mean()) < 0.2
    assert abs(st.X[:100, mem].mean()) < 0.2
    # same seed, same stream
    again = synth.rolling_stream(n=2000, k=8, days=120, switch_day=70, switch_frac=0.05,
                                 stress_groups=2, stress_first=100, stress_last=104, seed=5)
    np.testing.assert_array_equal(st.X, again.X)


def test_rolling_workload_definition():
    cfg = synth.ROLLING["rolling_n20000_k24"]
    s = cfg["stream"]
    assert (s["n"], s["k"], s["days"], s["switch_day"], s["switch_frac"]) == (20000, 24, 501, 300, 0.05)
    assert (s["stress_groups"], s["stress_first"], s["stress_last"]) == (3, 420, 430)
    assert (cfg["T"], cfg["windows"], cfg["iters"], cfg["delta"]) == (252, 250, 100, 50)
    # 250 windows of 252 days slide over exactly 501 days
    assert cfg["windows"] + cfg["T"] - 1 == s["days"]


@pytest.mark.parametrize("W,T,delta,sw,s0,s1", [(12, 4, 2, 8, 11, 11), (250, 252, 50, 300, 420, 430),
                                                (41, 60, 10, 70, 85, 88)])
def test_library_calm_mask_and_limit_match_oracle(W, T, delta, sw, s0, s1):
    calm = rolling.calm_mask(W, T, delta, sw, s0, s1)
    np.testing.assert_array_equal(calm, oracle.calm_windows(W, T, delta, sw, s0, s1))
    rng = np.random.default_rng(W)
    v = rng.random(W)
    v[:delta] = np.nan
    if calm.sum() >= 2:
        got = rolling.three_sigma(v, calm)
        ref = oracle.control_limit(v, calm)
        assert got[0] == pytest.approx(ref[0], rel=1e-14)
        np.testing.assert_array_equal(got[3], ref[3])


# ---- spherical k-means (P1 "Spherical k-means for direct hard clustering") ----

def test_kmeans_recovers_noise_free_blocks():
    """S = blockdiag(1 1^T): rows of one block are identical unit vectors, so
    with one initial row per block the first assignment is already the planted
    partition and the run stops after one update."""
    k, size = 4, 16
    truth = np.repeat(np.arange(k), size)
    S = (truth[:, None] == truth[None, :]).astype(np.float64)
    seed = next(s for s in range(100)
                if len(set(truth[oracle.sample_blocks(s, 0, k * size, k)])) == k)
    out = oracle.spherical_kmeans(S, k, seed=seed)
    assert out["converged"] and out["iters"] == 1
    assert oracle.ari(out["labels"], truth) == 1.0
    # each row has similarity 1 with its own block's centroid
    assert out["objective"] == pytest.approx(k * size, rel=1e-14)


def test_kmeans_objective_closed_form_and_monotone():
    rng = np.random.default_rng(4)
    A = rng.random((60, 60)) ** 3
    S = (A + A.T) / 2
    out = oracle.spherical_kmeans(S, 5, seed=1)
    assert out["converged"]
    # at a fixed point c_j = s_j / ||s_j||, so sum_i <x_i, c_l(i)> = sum_j ||s_j||
    X = S / np.linalg.norm(S, axis=1, keepdims=True)
    lab = out["labels"]
    closed = sum(np.linalg.norm(X[lab == j].sum(axis=0)) for j in range(5))
    assert out["objective"] == pytest.approx(closed, rel=1e-12)
    # and every row sits with its most similar centroid
    sims = X @ out["C"].T
    assert np.all(sims[np.arange(60), lab] >= sims.max(axis=1) - 1e-12)
    # the summed similarity never falls from one iteration to the next
    objs = [oracle.spherical_kmeans(S, 5, max_iters=m, seed=1)["objective"] for m in range(out["iters"] + 1)]
    assert all(b >= a - 1e-12 for a, b in zip(objs, objs[1:]))


def test_kmeans_initial_rows_are_the_documented_draw():
    rng = np.random.default_rng(5)
    A = rng.random((40, 40))
    S = (A + A.T) / 2
    out = oracle.spherical_kmeans(S, 3, max_iters=0, seed=9)
    rows = oracle.sample_blocks(9, 0, 40, 3)
    X = S / np.linalg.norm(S, axis=1, keepdims=True)
    np.testing.assert_array_equal(out["C"], X[rows])
    np.testing.assert_array_equal(out["labels"], np.argmax(X @ X[rows].T, axis=1))


def test_boundary_fraction_hand_case():
    # ratios of second to first loading: 0, 0.6, 0.4, (zero row), 0.49, 0.5
    H = np.array([[1.0, 0.0], [1.0, 0.6], [0.4, 1.0], [0.0, 0.0], [1.0, 0.49], [0.5, 1.0]])
    assert oracle.boundary_fraction(H) == pytest.approx(2 / 6)


def test_library_boundary_share_matches_oracle():
    rng = np.random.default_rng(8)
    H = rng.random((500, 6)) ** 4
    H[::7] = 0.0
    H[3] = [1.0, 0.5, 0, 0, 0, 0]  # exactly at the ratio
    for ratio in (0.3, 0.5, 0.9):
        assert rolling.boundary_share(H, ratio) == oracle.boundary_fraction(H, ratio)


def test_library_summary_of_a_run_too_short_to_calibrate():
    """Fewer windows than delta: no ARI(t - delta, t), no limit; the digest
    still serialises (None where nothing is defined)."""
    import json
    st = _small_stream()
    W = 5
    ones = np.ones(W)
    r = {"build_s": ones * 1e-3, "fit_s": ones * 1e-2, "monitor_s": ones * 1e-3,
         "flags": np.zeros(W, bool), "ari_drift": np.full(W, np.nan), "calm_mean": float("nan"),
         "calm_sd": float("nan"), "limit": float("nan"), "first_window_iters": 10,
         "cross_dependence": ones, "cross_dependence_scaled": ones, "ari_vs_before": ones,
         "ari_vs_after": ones, "boundary_fraction": ones * 0}
    res = {"T": 30, "windows": W, "n": 480, "k": 6, "iters": 10, "delta": 50, "warm_start": True,
           "calm": np.zeros(W, bool), "kinds": {"abscorr": r}}
    d = json.loads(json.dumps(rolling.summary(res, st), allow_nan=False))
    k = d["kinds"]["abscorr"]
    assert k["limit"] is None and k["min_drift"] is None and k["first_flag"] is None
