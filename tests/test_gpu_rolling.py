"""The rolling workload on the GPU.

Small stream (n = 768, 41 windows of 160 days): every window against the oracle
from the same S and init — objective at the first and last step, labels, the
stressed-sector block means of S — and the ARI series and 3-sigma limit built
on them. Full stream (n = 20 000, 250 windows of 252 days, the rolling
workload): properties that hold at any size (labels valid, every fit descends,
the alert fires only once the switch fills a large share of the window, the
co-crash raises the TPDM's cross-sector dependence)."""
import numpy as np
import pytest

import oracle
from symmetric_nmf_clustering_amd import synth
from tests.gpu_util import require_gpu, s_close

pytestmark = pytest.mark.gpu

# T = 160 keeps m = 8 tail days, so the TPDM has rank >= k + 2 (with m < k the
# factorization is degenerate and fp32/fp64 noise picks different minima)
SMALL = dict(n=768, k=6, days=200, switch_day=150, switch_frac=0.05, stress_groups=2,
             stress_first=185, stress_last=188, seed=5)
T_SMALL, W_SMALL, DELTA_SMALL, ITERS = 160, 41, 10, 100


@pytest.fixture(scope="module")
def small():
    require_gpu()
    from symmetric_nmf_clustering_amd import rolling
    st = synth.rolling_stream(**SMALL)
    res = rolling.run(st, T=T_SMALL, windows=W_SMALL, k=SMALL["k"], iters=ITERS,
                      delta=DELTA_SMALL, keep_H=True, kmeans=True)
    return st, res


@pytest.mark.parametrize("kind", ["abscorr", "tpdm"])
def test_rolling_small_matches_oracle(small, kind):
    """Every window against the oracle from the same input: the device-built
    fp32 S of the window and the same init (the seeded init for the first
    window, fitted to convergence; the device's previous-window H after it,
    100 full-batch steps).
    Parity is defined per link of the warm-started chain: run end to end, two
    chains that differ in rounding drift apart over thousands of steps. The
    builds are checked against the oracle's own S on the first and last
    window."""
    torch = require_gpu()
    from symmetric_nmf_clustering_amd import api
    st, res = small
    r = res["kinds"][kind]
    n, k = SMALL["n"], SMALL["k"]
    groups = st.stress_groups
    ref_labels = []
    for t in range(W_SMALL):
        Xw = st.window(t, T_SMALL)
        S = api.build_S(torch.from_numpy(np.ascontiguousarray(Xw)).cuda(), kind)[0]
        S = S.cpu().numpy().astype(np.float64)
        assert S.shape == (n, n)
        if t in (0, W_SMALL - 1):
            S_own = oracle.abs_corr(Xw) if kind == "abscorr" else oracle.tpdm(Xw)
            ok, worst = s_close(S.astype(np.float32), S_own)
            assert ok, (t, worst)
        m = S.mean()
        if t == 0:
            # the first window is fitted to convergence; where fp32 noise in f
            # decides the exact stop step, parity means the same number of
            # steps: the oracle takes the device's count (f_t of the stop step
            # t needs one step more)
            H0 = oracle.init_uniform(n, k, oracle.init_scale_matched(m, k), 0)
            steps = r["first_window_iters"] + (1 if r["first_window_converged"] else 0)
            assert r["first_window_iters"] > ITERS
            ref = oracle.fit_full(S, H0, oracle.default_lr(m, k), steps, tol=0.0)
        else:
            H0 = r["H"][t - 1].astype(np.float64)
            ref = oracle.fit_full(S, H0, oracle.default_lr(m, k), ITERS)
        s2 = float((S * S).sum())
        for got, want in ((r["f_first"][t], ref["f"][0]), (r["f_last"][t], ref["f"][-1])):
            assert abs(got - want) <= 1e-3 * max(abs(want), 1e-6 * s2), (t, got, want)
        lab = oracle.labels(ref["H"])
        a = oracle.ari(r["labels"][t], lab)
        assert a >= 0.99, (t, a)
        ref_labels.append(lab)
        B = oracle.cross_block_means(S, st.labels_after, groups)
        np.testing.assert_allclose(r["block_means"][t], B, rtol=1e-5)
        # the boundary share of the device's H, and the k-means baseline on
        # the same S against the oracle's from the same seeded rows
        assert r["boundary_fraction"][t] == oracle.boundary_fraction(r["H"][t])
        km = oracle.spherical_kmeans(S, k, seed=0)
        a_km = oracle.ari(km["labels"], r["labels"][t])
        assert abs(r["kmeans_vs_symnmf_ari"][t] - a_km) <= 0.02, (t, r["kmeans_vs_symnmf_ari"][t], a_km)
    # the ARI series and its limit, from the oracle's labels
    d_ref = oracle.ari_drift(ref_labels, DELTA_SMALL)
    np.testing.assert_allclose(r["ari_drift"], d_ref, atol=0.02)
    calm = oracle.calm_windows(W_SMALL, T_SMALL, DELTA_SMALL, SMALL["switch_day"],
                               SMALL["stress_first"], SMALL["stress_last"])
    np.testing.assert_array_equal(res["calm"], calm)
    lim_ref = oracle.control_limit(d_ref, calm)[0]
    assert abs(r["limit"] - lim_ref) <= 0.05


def test_rolling_small_cold_start_is_per_window_seeded_fit():
    """Without the warm start every window is the seeded fit of its own S."""
    torch = require_gpu()
    from symmetric_nmf_clustering_amd import api, rolling
    st = synth.rolling_stream(**SMALL)
    res = rolling.run(st, T=T_SMALL, windows=3, k=SMALL["k"], iters=20, delta=1,
                      kinds=("abscorr",), warm_start=False, keep_H=True)
    for t in range(3):
        S, _ = api.build_S(torch.from_numpy(np.ascontiguousarray(st.window(t, T_SMALL))).cuda())
        one = api.fit(S, SMALL["k"], solver="full", max_iters=20, tol_rel=0.0, seed=0)
        np.testing.assert_array_equal(res["kinds"]["abscorr"]["H"][t], one.H.cpu().numpy())


@pytest.fixture(scope="module")
def full():
    torch = require_gpu()
    from symmetric_nmf_clustering_amd import rolling
    free, _ = torch.cuda.mem_get_info()
    if free < 4e9:
        pytest.skip("needs ~4 GB of free device memory")
    cfg = synth.ROLLING["rolling_n20000_k24"]
    st = synth.rolling_stream(**cfg["stream"])
    res = rolling.run(st, T=cfg["T"], windows=cfg["windows"], k=cfg["stream"]["k"],
                      iters=cfg["iters"], delta=cfg["delta"])
    return cfg, st, res


def test_rolling_full_workload_properties(full):
    cfg, st, res = full
    k, T, sw = cfg["stream"]["k"], cfg["T"], cfg["stream"]["switch_day"]
    W = cfg["windows"]
    t = np.arange(W)
    stressed = (t + T - 1 >= st.stress_first) & (t <= st.stress_last)
    assert res["calm"].sum() >= 100
    for kind in ("abscorr", "tpdm"):
        r = res["kinds"][kind]
        assert r["labels"].min() >= 0 and r["labels"].max() < k
        # every warm-started window's 100 steps lower the objective
        assert np.all(r["f_last"][1:] < r["f_first"][1:])
        # the first window is fitted to convergence before the series starts
        assert r["first_window_iters"] > cfg["iters"]
    c = res["kinds"]["abscorr"]
    # |corr| finds the planted groups before the switch and the moved ones after it
    assert c["ari_vs_before"][0] >= 0.99
    assert c["ari_vs_after"][-1] >= 0.9
    # the alert fires, and only once a large share of a window's days follow
    # the switch (window t holds t + T - switch_day of them)
    flagged = np.flatnonzero(c["flags"])
    assert flagged.size > 0
    assert flagged.min() + T - sw >= 0.4 * T, flagged[:5]
    # the co-crash raises the TPDM's dependence between the stressed sectors
    for key in ("cross_dependence", "cross_dependence_scaled"):
        d = res["kinds"]["tpdm"][key]
        assert d[stressed].max() > 1.3 * d[~stressed].mean(), key
