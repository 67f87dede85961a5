"""The rolling workload on the GPU.

Small stream (n = 768, 41 windows of 160 days), on the oracle's S of every
window: the |corr| chain end to end and the TPDM chain link by link against the
oracle — objectives, labels, the stressed-sector block means, the k-means
baseline, the ARI series and its 3-sigma limit. Full stream (n = 20 000, 250 windows of 252 days, the rolling
workload): properties that hold at any size (labels valid, every fit descends,
the alert fires only once the switch fills a large share of the window, the
co-crash raises the TPDM's cross-sector dependence)."""
import numpy as np
import pytest
from sklearn.metrics import adjusted_rand_score

import oracle
from symmetric_nmf_clustering_amd import synth
from tests.gpu_util import S_to_dev, require_gpu, to_dev

pytestmark = pytest.mark.gpu

# T = 160 keeps m = 8 tail days, so the TPDM has rank >= k + 2 (with m < k the
# factorization is degenerate and fp32/fp64 noise picks different minima)
SMALL = dict(n=768, k=6, days=200, switch_day=150, switch_frac=0.05, stress_groups=2,
             stress_first=185, stress_last=188, seed=5)
T_SMALL, W_SMALL, DELTA_SMALL, ITERS = 160, 41, 10, 100


def _oracle_S(st, kind):
    """Each window's S built by the oracle from the returns, rounded to fp32:
    the input both sides factorize."""
    out = []
    for t in range(W_SMALL):
        Xw = st.window(t, T_SMALL)
        S = oracle.abs_corr(Xw) if kind == "abscorr" else oracle.tpdm(Xw)
        out.append(S.astype(np.float32))
    return out


@pytest.fixture(scope="module")
def small():
    require_gpu()
    from symmetric_nmf_clustering_amd import rolling
    st = synth.rolling_stream(**SMALL)
    S_win = {kind: _oracle_S(st, kind) for kind in ("abscorr", "tpdm")}
    res = rolling.run(st, T=T_SMALL, windows=W_SMALL, k=SMALL["k"], iters=ITERS,
                      delta=DELTA_SMALL, keep_H=True, kmeans=True, S_windows=S_win)
    return st, S_win, res


def test_rolling_small_corr_chain_matches_oracle(small):
    """|corr|: the whole warm-started chain (first window to convergence, then
    100 steps per window) on the oracle's S of every window, against the
    oracle's chain from the same seeded init: objective at the first and last
    step of every window, labels, the stressed sectors' block means, the
    k-means baseline's agreement with SymNMF, the boundary share, and the ARI
    series with its 3-sigma limit. (On |corr| two chains that differ only in
    rounding stay together; see the TPDM test for the per-window form.)"""
    st, S_win, res = small
    r = res["kinds"]["abscorr"]
    k = SMALL["k"]
    ref = oracle.rolling_fit(st.X, k, T_SMALL, W_SMALL, kind="abscorr", iters=ITERS,
                             S_windows=S_win["abscorr"], first_max_iters=2000, first_tol=1e-6)
    for t in range(W_SMALL):
        S = S_win["abscorr"][t].astype(np.float64)
        s2 = float((S * S).sum())
        fr = ref["f"][t]
        for got, want in ((r["f_first"][t], fr[0]), (r["f_last"][t], fr[-1])):
            assert abs(got - want) <= 1e-3 * max(abs(want), 1e-6 * s2), (t, got, want)
        assert adjusted_rand_score(r["labels"][t], ref["labels"][t]) >= 0.99, t
        B = oracle.cross_block_means(S, st.labels_after, st.stress_groups)
        np.testing.assert_allclose(r["block_means"][t], B, rtol=1e-5)
        assert abs(r["boundary_fraction"][t] - oracle.boundary_fraction(ref["H"][t])) <= 0.01, t
        km = oracle.spherical_kmeans(S, k, seed=0)
        want = adjusted_rand_score(km["labels"], ref["labels"][t])
        assert abs(r["kmeans_vs_symnmf_ari"][t] - want) <= 0.02, (t, r["kmeans_vs_symnmf_ari"][t], want)
    d_ref = oracle.ari_drift(ref["labels"], DELTA_SMALL)
    np.testing.assert_allclose(r["ari_drift"], d_ref, atol=0.02)
    calm = oracle.calm_windows(W_SMALL, T_SMALL, DELTA_SMALL, SMALL["switch_day"],
                               SMALL["stress_first"], SMALL["stress_last"])
    np.testing.assert_array_equal(res["calm"], calm)
    assert abs(r["limit"] - oracle.control_limit(d_ref, calm)[0]) <= 0.05


def test_rolling_small_tpdm_links_match_oracle(small):
    """TPDM: each link of the warm-started chain from the same input — the
    oracle's S of window t and the oracle chain's H of window t-1 (the seeded
    init for window 0) — on the device through the C ABI against the oracle.

    A warm start sits near a stationary point, and AdaGrad's first step moves
    every coordinate by lr sign(g) (G starts at 0), so where many gradients are
    at rounding level fp32 and fp64 take different signs (several correct
    first steps). What is unique is compared: the first step on every
    coordinate whose gradient is decided (|g| > 1e-3 max|g|); then, from the
    device's own state after that step (H_1 and G_1), the oracle's remaining
    99 steps against the device's, on every link: objective trajectory within
    1e-3 (of max(f, 1e-6 ||S||^2)) and labels ARI >= 0.99. The driver's own
    TPDM chain is checked for its block means."""
    torch = require_gpu()
    from symmetric_nmf_clustering_amd import api
    st, S_win, res = small
    k = SMALL["k"]
    H_prev = None
    for t in range(W_SMALL):
        S = S_win["tpdm"][t].astype(np.float64)
        m = S.mean()
        lr = oracle.default_lr(m, k)
        H0 = (oracle.init_uniform(S.shape[0], k, oracle.init_scale_matched(m, k), 0)
              if H_prev is None else H_prev.astype(np.float32).astype(np.float64))
        Sd, H0d = S_to_dev(S_win["tpdm"][t], torch), to_dev(H0, torch)
        # the first step on decided coordinates
        ref1 = oracle.fit_full(S, H0, lr, 1)
        first = api.fit(Sd, k, solver="full", max_iters=1, tol_rel=0.0, H0=H0d, return_G=True)
        one = first.H.cpu().numpy()
        g = oracle.gradient(S, H0)
        decided = np.abs(g) > 1e-3 * np.abs(g).max()
        assert np.abs(one - ref1["H"])[decided].max() <= 1e-4 * lr, t
        assert one.min() >= 0.0 and np.abs(one - H0).max() <= lr * (1 + 1e-5), t
        # the remaining steps from the device's state after the first one
        ref = oracle.fit_full(S, one.astype(np.float64), lr, ITERS - 1,
                              G0=first.G.cpu().numpy().astype(np.float64))
        got = api.fit(Sd, k, solver="full", max_iters=ITERS, tol_rel=0.0, H0=H0d)
        s2 = float((S * S).sum())
        fg, fr = got.f_trace[1:], np.asarray(ref["f"])
        Hg = got.H.cpu().numpy()
        assert Hg.min() >= 0.0, t
        rel = np.abs(fg - fr) / np.maximum(np.abs(fr), 1e-6 * s2)
        assert rel.max() <= 1e-3, (t, float(rel.max()), int(rel.argmax()))
        ari = adjusted_rand_score(Hg.argmax(axis=1), oracle.labels(ref["H"]))
        assert ari >= 0.99, (t, ari)
        H_prev = ref["H"]
        B = oracle.cross_block_means(S, st.labels_after, st.stress_groups)
        np.testing.assert_allclose(res["kinds"]["tpdm"]["block_means"][t], B, rtol=1e-5)


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
