"""GPU parity of the fit (full batch, Block-SVRG, AdaptGrow) and the spectral
probe against the oracle, on the seeded workloads."""
import math

import numpy as np
import pytest
from sklearn.metrics import adjusted_rand_score

import oracle
from symmetric_nmf_clustering_amd import synth
from tests.gpu_util import S_to_dev, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return require_gpu()


@pytest.fixture(scope="module")
def api(torch):
    from symmetric_nmf_clustering_amd import api as a
    return a


def traj_rel(f_gpu, f_ref, S_fro2):
    """Objective trajectory error relative to max(f_ref, 1e-6 ||S||^2)."""
    f_gpu = np.asarray(f_gpu, np.float64)
    f_ref = np.asarray(f_ref, np.float64)
    den = np.maximum(np.abs(f_ref), 1e-6 * S_fro2)
    return np.abs(f_gpu - f_ref) / den


def labels_agree(h_gpu, h_ref):
    """Device labels (row argmax, first index on ties) against the oracle's."""
    lg, lr = np.argmax(h_gpu, axis=1), oracle.labels(h_ref)
    if np.array_equal(lg, lr):
        return True, 1.0
    a = adjusted_rand_score(lg, lr)
    return a >= 0.99, a


def gamma_of(ev, k):
    """gamma_{k+1} of a device eigenvalue list (for comparison only)."""
    ev = np.asarray(ev, np.float64)
    return ev[k] / max(abs(ev[k + 1]), 1e-6 * abs(ev[0]))


@pytest.fixture(scope="module")
def c1(torch):
    w = synth.workload("blocks_n1024_k8")
    S = oracle.abs_corr(w.X).astype(np.float32)
    return w, S


def test_fit_full_c1_trajectory(torch, api, c1):
    """n=1024, k=8, H0 ~ U(0, 0.1), lr 0.05, 200 full-batch steps."""
    w, S = c1
    res = api.fit(S_to_dev(S, torch), w.k, solver="full", init="uniform", init_scale=0.1, seed=0,
                  lr=0.05, max_iters=200, tol_rel=0.0, return_G=True)
    # the oracle evaluates f as ||S - H H^T||_F^2 directly (no trace identity)
    ref = oracle.fit_full(S, oracle.init_uniform(w.n, w.k, 0.1, 0), 0.05, 200, tol=0.0,
                          objective="explicit")
    s2 = float((S.astype(np.float64) ** 2).sum())
    assert res.report["iterations"] == 200 and len(res.f_trace) == 200
    rel = traj_rel(res.f_trace, ref["f"], s2)
    assert rel.max() <= 1e-3, rel.max()
    H = res.H.cpu().numpy()
    assert H.min() >= 0.0
    # H itself after the 200 steps, element by element: every entry within
    # 1e-4 of the largest (fp32 and fp64 trajectories of the same steps)
    dH = np.abs(H.astype(np.float64) - ref["H"])
    print(f"c1 H after 200 steps: max |H - H_ref| = {dH.max():.2e} (max H {ref['H'].max():.3f})")
    assert dH.max() <= 1e-4 * ref["H"].max(), dH.max()
    ok, a = labels_agree(H, ref["H"])
    assert ok, a
    assert adjusted_rand_score(H.argmax(axis=1), w.labels) > 0.99
    assert abs(res.report["S_fro2"] - s2) <= 1e-6 * s2
    # the report's f_last is the last exact objective, f_199
    assert res.report["f_last_iter"] == 199
    assert res.report["f_last"] == pytest.approx(res.f_trace[-1])


def test_fit_init_matches_oracle_generator(torch, api, c1):
    w, S = c1
    res = api.fit(S_to_dev(S, torch), w.k, solver="full", init="uniform", init_scale=0.1, seed=7,
                  max_iters=0, tol_rel=0.0)
    np.testing.assert_array_equal(res.H.cpu().numpy(),
                                  oracle.init_uniform(w.n, w.k, 0.1, 7).astype(np.float32))


def test_fit_resume_equals_uninterrupted(torch, api, c1):
    w, S = c1
    Sd = S_to_dev(S, torch)
    kw = dict(solver="full", lr=0.05, tol_rel=0.0)
    one = api.fit(Sd, w.k, init="uniform", init_scale=0.1, seed=0, max_iters=60, **kw)
    a = api.fit(Sd, w.k, init="uniform", init_scale=0.1, seed=0, max_iters=25, return_G=True, **kw)
    b = api.fit(Sd, w.k, H0=a.H, G0=a.G, max_iters=35, **kw)
    assert torch.equal(one.H, b.H)


def test_fit_full_c2_to_convergence(torch, api):
    """n=8192, k=24 Student-t factors: full batch to relative change < 1e-6."""
    w = synth.workload("tfactor_n8192_k24")
    S = oracle.abs_corr(w.X).astype(np.float32)
    S64 = S.astype(np.float64)
    res = api.fit(S_to_dev(S, torch), w.k, solver="full", max_iters=2000, tol_rel=1e-6, seed=1)
    m = S64.mean()
    H0 = oracle.init_uniform(w.n, w.k, oracle.init_scale_matched(m, w.k), 1)
    at = (0, 1, 2, 5, 10, 30, 100, 199)
    ref = oracle.fit_full(S64, H0, oracle.default_lr(m, w.k), 2000, tol=1e-6, snapshots=at)
    s2 = float((S64 ** 2).sum())
    assert res.converged and ref["converged"]
    L = min(200, len(ref["f"]), len(res.f_trace))
    assert traj_rel(res.f_trace[:L], ref["f"][:L], s2).max() <= 1e-3
    # the same trajectory against ||S - H H^T||_F^2 evaluated directly on the
    # oracle's H_t (no trace identity; 0.5 s per evaluation at this size)
    f_dir = np.array([oracle.objective_explicit(S64, ref["H_at"][t]) for t in at])
    assert traj_rel(res.f_trace[list(at)], f_dir, s2).max() <= 1e-3
    f_end = oracle.objective_explicit(S64, ref["H"])
    assert abs(res.report["f_last"] - f_end) <= 1e-3 * f_end
    ok, a = labels_agree(res.H.cpu().numpy(), ref["H"])
    assert ok, a
    print(f"c2 iterations gpu={res.report['iterations']} oracle={ref['iters']}")


def test_fit_block_svrg_c3(torch, api):
    """n=8192, k=24 TPDM with a joint tail-stress episode; Block-SVRG with
    row blocks of 1024 and the same block stream on both sides."""
    w = synth.workload("tstress_n8192_k24")
    S = oracle.tpdm(w.X, 0.05).astype(np.float32)
    S64 = S.astype(np.float64)
    iters = 240
    res = api.fit(S_to_dev(S, torch), w.k, solver="block_svrg", phi0=1.0 / 8, block_rows=1024,
                  max_iters=iters, tol_rel=1e-6, seed=1)
    m = S64.mean()
    H0 = oracle.init_uniform(w.n, w.k, oracle.init_scale_matched(m, w.k), 1)
    ref = oracle.fit_adaptgrow(S64, H0, oracle.default_lr(m, w.k), iters,
                               solver=oracle.SOLVER_BLOCK_SVRG, phi0=1.0 / 8, block_rows=1024,
                               tol=1e-6, seed=1)
    rep = res.report
    assert rep["start_branch"] == 1 and rep["n_blocks"] == 8
    assert rep["iterations"] == ref["iters"]
    assert rep["doublings"] == len(ref["history"])
    fg, fr = np.asarray(res.f_trace), np.asarray(ref["f"])
    assert np.array_equal(np.isnan(fg), np.isnan(fr))        # anchors at the same steps
    s2 = float((S64 ** 2).sum())
    ex = ~np.isnan(fr)
    assert traj_rel(fg[ex], fr[ex], s2).max() <= 1e-3
    ok, a = labels_agree(res.H.cpu().numpy(), ref["H"])
    assert ok, a


def test_fit_svrg_growth_to_full(torch, api):
    """|corr| input with a flat post-rank spectrum: Block-SVRG stalls, doubles
    its sample and finishes full batch; same decisions as the oracle."""
    w = synth.student_factor(n=4096, k=8, T=252, seed=3, min_size=64)
    S = oracle.abs_corr(w.X).astype(np.float32)
    S64 = S.astype(np.float64)
    res = api.fit(S_to_dev(S, torch), w.k, solver="block_svrg", phi0=0.25, block_rows=512,
                  max_iters=800, tol_rel=1e-6, seed=2)
    m = S64.mean()
    H0 = oracle.init_uniform(w.n, w.k, oracle.init_scale_matched(m, w.k), 2)
    ref = oracle.fit_adaptgrow(S64, H0, oracle.default_lr(m, w.k), 800,
                               solver=oracle.SOLVER_BLOCK_SVRG, phi0=0.25, block_rows=512,
                               tol=1e-6, seed=2)
    assert ref["final_branch"] == "full"
    assert res.report["final_branch"] == 0
    assert res.report["doublings"] == len(ref["history"])
    s2 = float((S64 ** 2).sum())
    fg, fr = np.asarray(res.f_trace), np.asarray(ref["f"])
    L = min(len(fg), len(fr), 200)
    ex = ~np.isnan(fr[:L])
    assert np.array_equal(np.isnan(fg[:L]), ~ex)
    assert traj_rel(fg[:L][ex], fr[:L][ex], s2).max() <= 1e-3
    ok, a = labels_agree(res.H.cpu().numpy(), ref["H"])
    assert ok, a


@pytest.mark.parametrize("n,seed", [(1024, 0), (8192, 1)])
def test_probe_matches_eigvalsh(torch, api, n, seed):
    if n == 1024:
        w = synth.workload("blocks_n1024_k8")
    else:
        w = synth.workload("tfactor_n8192_k24")
    S = oracle.abs_corr(w.X).astype(np.float32)
    p, tol = 64, 1e-6
    ev, its, conv = api.spectral_probe(S_to_dev(S, torch), p=p, max_iters=400, tol=tol, seed=seed)
    ref = oracle.top_eigenvalues(S.astype(np.float64), p)
    lam1 = abs(ref[0])
    err = np.abs(ev - ref) / lam1
    print(f"probe n={n} iters={its} converged={conv} max err/|l1|={err.max():.2e}")
    assert conv
    assert err.max() <= 100 * tol, err.max()
    # the gap ratio the solver choice reads agrees
    assert gamma_of(ev, w.k) == pytest.approx(oracle.gap_ratio(ref, w.k), rel=1e-3)


def test_probe_widest_subspace(torch, api):
    """p = 112 (a 128-column subspace, the widest the probe takes) on a matrix
    with a planted geometric spectrum of mixed signs: the top 112 eigenvalues
    by magnitude, signs kept, against LAPACK."""
    n, p, tol = 600, 112, 1e-6
    rng = np.random.default_rng(21)
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    lam = 100.0 * 0.97 ** np.arange(n)
    lam[2::3] *= -1.0
    S = ((Q * lam) @ Q.T).astype(np.float32)
    S = (S + S.T) / 2
    ev, its, conv = api.spectral_probe(S_to_dev(S, torch), p=p, max_iters=400, tol=tol, seed=3)
    ref = oracle.top_eigenvalues(S.astype(np.float64), p)
    err = np.abs(ev - ref) / abs(ref[0])
    assert conv, its
    assert err.max() <= 100 * tol, err.max()
    assert np.array_equal(np.sign(ev), np.sign(ref))


@pytest.mark.parametrize("n,p", [(70, 40), (100, 40), (200, 8), (33, 1), (1000, 100)])
def test_probe_width_rule_edges(torch, api, n, p):
    """The subspace width at its edges: 2p capped by n (n = 70: 64 = p + 24
    columns, n = 100: 80), the p + 16 floor (p = 8: 32 columns where 2p is 16;
    p = 1: 32 of n = 33; p = 100: 128 = p + 28). Planted mixed-sign spectrum
    against LAPACK."""
    rng = np.random.default_rng(n + p)
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    lam = 50.0 * 0.97 ** np.arange(n)
    lam[1::4] *= -1.0
    S = ((Q * lam) @ Q.T).astype(np.float32)
    S = (S + S.T) / 2
    tol = 1e-6
    ev, its, conv = api.spectral_probe(S_to_dev(S, torch), p=p, max_iters=400, tol=tol, seed=1)
    ref = oracle.top_eigenvalues(S.astype(np.float64), p)
    assert conv, its
    assert (np.abs(ev - ref) / abs(ref[0])).max() <= 100 * tol
    assert np.array_equal(np.sign(ev), np.sign(ref))


def test_probe_deterministic(torch, api):
    """Same S, p and seed give bitwise identical eigenvalues and step counts:
    every sum in the probe (the S.Q split partials, the cross-Grams, the host
    algebra) runs in a fixed order."""
    w = synth.workload("blocks_n1024_k8")
    Sd = S_to_dev(oracle.abs_corr(w.X).astype(np.float32), torch)
    a = api.spectral_probe(Sd, p=24, max_iters=200, tol=1e-6, seed=4)
    b = api.spectral_probe(Sd, p=24, max_iters=200, tol=1e-6, seed=4)
    np.testing.assert_array_equal(a[0], b[0])
    assert a[1] == b[1] and a[2] == b[2]


def test_probe_rank_deficient_tpdm(torch, api):
    w = synth.workload("tstress_n8192_k24")
    S = oracle.tpdm(w.X, 0.05).astype(np.float32)
    ev, its, conv = api.spectral_probe(S_to_dev(S, torch), p=26, max_iters=200, tol=1e-6)
    ref = oracle.top_eigenvalues(S.astype(np.float64), 26)
    err = np.abs(ev - ref) / abs(ref[0])
    assert err.max() <= 1e-4, err.max()
    assert gamma_of(ev, 24) < 5.0 and oracle.gap_ratio(ref, 24) < 5.0


def test_fit_auto_branch_from_probe(torch, api):
    """AUTO reads gamma_{k+1} from the probe: on the c2 |corr| input the
    post-rank spectrum is flat (gamma ~ 1.6 < 5), so it starts sampled with
    the same |B|0 as the oracle's reading on the exact spectrum."""
    w = synth.workload("tfactor_n8192_k24")
    S = oracle.abs_corr(w.X).astype(np.float32)
    Sd = S_to_dev(S, torch)
    ev, _, _ = api.spectral_probe(Sd, p=64, max_iters=400, tol=1e-6)
    res = api.fit(Sd, w.k, eigvals=ev, max_iters=50, tol_rel=1e-6, seed=1)
    ref_ev = oracle.top_eigenvalues(S.astype(np.float64), 64)
    nb = 8
    expect = oracle.initial_blocks(oracle.gap_ratio(ref_ev, w.k), nb)
    assert res.report["start_branch"] == (0 if expect >= nb else 1)
    assert res.report["gamma"] == pytest.approx(oracle.gap_ratio(ref_ev, w.k), rel=1e-3)


def test_fit_edge_cases(torch, api):
    from symmetric_nmf_clustering_amd._lib import SymNMFError, E_NONFINITE
    # n = 1, k = 1: S = [[s]] -> h^2 -> s
    S = np.array([[0.81]], np.float32)
    res = api.fit(S_to_dev(S, torch), 1, solver="full", init="uniform", init_scale=0.5, lr=0.05,
                  max_iters=400, tol_rel=0.0)
    ref = oracle.fit_full(S, oracle.init_uniform(1, 1, 0.5, 0), 0.05, 400)
    assert res.H.item() == pytest.approx(ref["H"][0, 0], rel=1e-4)
    # k = n
    S5 = synth.random_symmetric_nonneg(5, seed=2)
    res = api.fit(S_to_dev(S5, torch), 5, solver="full", init="uniform", init_scale=0.5, lr=0.01,
                  max_iters=50, tol_rel=0.0)
    ref = oracle.fit_full(S5, oracle.init_uniform(5, 5, 0.5, 0), 0.01, 50)
    assert traj_rel(res.f_trace, ref["f"], (S5.astype(np.float64) ** 2).sum()).max() <= 1e-4
    # max_iters = 0 returns H0
    res = api.fit(S_to_dev(S5, torch), 2, solver="full", init="uniform", init_scale=0.5,
                  max_iters=0, tol_rel=0.0)
    assert res.report["iterations"] == 0 and len(res.f_trace) == 0
    # non-finite S
    Sn = S5.copy(); Sn[1, 2] = Sn[2, 1] = np.inf
    with pytest.raises(SymNMFError) as e:
        api.fit(S_to_dev(Sn, torch), 2, solver="full", max_iters=5)
    assert e.value.status == E_NONFINITE


def test_fit_deterministic(torch, api, c1):
    w, S = c1
    Sd = S_to_dev(S, torch)
    a = api.fit(Sd, w.k, solver="block_svrg", phi0=0.5, block_rows=256, max_iters=60, seed=3)
    b = api.fit(Sd, w.k, solver="block_svrg", phi0=0.5, block_rows=256, max_iters=60, seed=3)
    assert torch.equal(a.H, b.H)
    np.testing.assert_array_equal(a.f_trace, b.f_trace)


@pytest.mark.parametrize("phi0", [0.25, 0.5, 0.75])
def test_fit_block_svrg_multiblock_splits(torch, api, phi0):
    """16, 32 and 48 of 64 row blocks per sampled step. 16 and 32: one whole
    block per split of the sampled pass (32 is the split cap, the boundary
    between the two plans); 48: each split covers two blocks (the multi-block
    path of the S.H kernel)."""
    w = synth.student_factor(n=4096, k=12, T=252, seed=5, min_size=64)
    S = oracle.abs_corr(w.X).astype(np.float32)
    S64 = S.astype(np.float64)
    res = api.fit(S_to_dev(S, torch), w.k, solver="block_svrg", phi0=phi0, block_rows=64,
                  max_iters=60, tol_rel=0.0, seed=4)
    m = S64.mean()
    H0 = oracle.init_uniform(w.n, w.k, oracle.init_scale_matched(m, w.k), 4)
    ref = oracle.fit_adaptgrow(S64, H0, oracle.default_lr(m, w.k), 60,
                               solver=oracle.SOLVER_BLOCK_SVRG, phi0=phi0, block_rows=64,
                               tol=0.0, seed=4)
    assert res.report["n_blocks"] == 64 and res.report["start_branch"] == 1
    assert res.report["doublings"] == len(ref["history"])
    fg, fr = np.asarray(res.f_trace), np.asarray(ref["f"])
    assert np.array_equal(np.isnan(fg), np.isnan(fr))
    ex = ~np.isnan(fr)
    assert traj_rel(fg[ex], fr[ex], float((S64 ** 2).sum())).max() <= 1e-3
    ok, a = labels_agree(res.H.cpu().numpy(), ref["H"])
    assert ok, a


@pytest.mark.parametrize("solver,phi0", [("full", 0.0), ("block_svrg", 0.5)])
def test_fit_widest_factor(torch, api, solver, phi0):
    """k = 64, the widest factor the fit takes (four MFMA tiles and no
    vector-ALU columns in the S.H pass; the sampled pass at that width):
    60 steps against the oracle."""
    w = synth.student_factor(n=1536, k=64, T=252, seed=7, min_size=16)
    S = oracle.abs_corr(w.X).astype(np.float32)
    S64 = S.astype(np.float64)
    res = api.fit(S_to_dev(S, torch), 64, solver=solver, phi0=phi0, block_rows=128,
                  max_iters=60, tol_rel=0.0, seed=4)
    m = S64.mean()
    H0 = oracle.init_uniform(w.n, 64, oracle.init_scale_matched(m, 64), 4)
    ref = oracle.fit_adaptgrow(S64, H0, oracle.default_lr(m, 64), 60,
                               solver=(oracle.SOLVER_FULL if solver == "full"
                                       else oracle.SOLVER_BLOCK_SVRG),
                               phi0=phi0, block_rows=128, tol=0.0, seed=4)
    fg, fr = np.asarray(res.f_trace), np.asarray(ref["f"])
    assert len(fg) == len(fr) and np.array_equal(np.isnan(fg), np.isnan(fr))
    ex = ~np.isnan(fr)
    assert traj_rel(fg[ex], fr[ex], float((S64 ** 2).sum())).max() <= 1e-3
    ok, a = labels_agree(res.H.cpu().numpy(), ref["H"])
    assert ok, a


@pytest.mark.parametrize("solver", ["full", "block_svrg"])
def test_fit_rmsprop_matches_oracle(torch, api, c1, solver):
    """RMSprop's accumulator (rms_decay = 0.9) on the config-1 input, full batch
    for 200 steps and Block-SVRG (blocks of 128 rows, 2 of 8 sampled) for 60.
    lr = 0.01: RMSprop's steps do not shrink like AdaGrad's (about
    lr / sqrt(1 - rho) per coordinate), and at the config's lr = 0.05 they are
    three times the entries of H, the run turns oscillatory after ~60 steps and
    rounding decides a transient (measured: the first 60 steps agree to 1e-7,
    f_199 agrees, the middle parts); at 0.01 the trajectory is smooth (5e-5)."""
    w, S = c1
    s2 = float((S.astype(np.float64) ** 2).sum())
    H0 = oracle.init_uniform(w.n, w.k, 0.1, 0)
    if solver == "full":
        res = api.fit(S_to_dev(S, torch), w.k, solver="full", init="uniform", init_scale=0.1,
                      seed=0, lr=0.01, max_iters=200, tol_rel=0.0, rms_decay=0.9)
        ref = oracle.fit_full(S, H0, 0.01, 200, tol=0.0, rho=0.9)
    else:
        res = api.fit(S_to_dev(S, torch), w.k, solver="block_svrg", init="uniform", init_scale=0.1,
                      seed=0, lr=0.01, max_iters=60, tol_rel=0.0, rms_decay=0.9, block_rows=128,
                      phi0=0.25)
        ref = oracle.fit_adaptgrow(S.astype(np.float64), H0, 0.01, 60, solver=oracle.SOLVER_BLOCK_SVRG,
                                   phi0=0.25, block_rows=128, tol=0.0, seed=0, rho=0.9)
    fg, fr = np.asarray(res.f_trace), np.asarray(ref["f"])
    assert np.array_equal(np.isnan(fg), np.isnan(fr))
    ex = ~np.isnan(fr)
    assert traj_rel(fg[ex], fr[ex], s2).max() <= 1e-3
    ok, a = labels_agree(res.H.cpu().numpy(), ref["H"])
    assert ok, a


def test_fit_adaptgrow_c3_auto_to_stop(torch, api):
    """Config 3 end to end: the n = 8192 TPDM (rank <= 13 < k + 2, so the
    post-rank gap is a ratio of null-space eigenvalues and AUTO starts sampled
    at one block of 1024 rows) under AUTO from the device probe's eigenvalues,
    to the anchor stop test, against the oracle's AdaptGrow from LAPACK's
    eigenvalues on the same fp32 S and block stream.

    Same start branch and |B|0, no doublings on either side, the same anchors
    up to the stop; the stop falls on the same anchor, or, where the test sits
    within rounding of its threshold at the earlier of the two stop anchors,
    within two epochs (the later side's test ratio at the earlier stop must
    then be within 2% of 1). Exact objectives at every common anchor within
    1e-3 (of max(f, 1e-6 ||S||^2)), also against ||S - H H^T||^2 evaluated
    directly at a few anchors; labels ARI >= 0.99."""
    w = synth.workload("tstress_n8192_k24")
    S = oracle.tpdm(w.X, 0.05).astype(np.float32)
    S64 = S.astype(np.float64)
    Sd = S_to_dev(S, torch)
    ev_dev, _, _ = api.spectral_probe(Sd, p=w.k + 2, seed=1)
    ev_ref = oracle.top_eigenvalues(S64, w.k + 2)
    res = api.fit(Sd, w.k, eigvals=ev_dev, block_rows=1024, max_iters=2000, tol_rel=1e-6,
                  seed=1, return_state=True)
    m = S64.mean()
    H0 = oracle.init_uniform(w.n, w.k, oracle.init_scale_matched(m, w.k), 1)
    at = tuple(range(0, 2001, 8 * 25))
    ref = oracle.fit_adaptgrow(S64, H0, oracle.default_lr(m, w.k), 2000, eigvals=ev_ref, k=w.k,
                               block_rows=1024, tol=1e-6, seed=1, snapshots=at)
    rep = res.report
    print(f"c3 AUTO: gpu iters {rep['iterations']} conv {rep['converged']} gamma {rep['gamma']:.3e};"
          f" oracle iters {ref['iters']} conv {ref['converged']} gamma {ref['gamma']:.3e}")
    assert rep["start_branch"] == 1 and ref["start_branch"] == "sampled"
    assert rep["n_blocks"] == 8 and rep["blocks_final"] == ref["nsel"] == 1
    assert rep["doublings"] == len(ref["history"]) == 0
    assert rep["converged"] and ref["converged"]
    E = 8
    fg, fr = np.asarray(res.f_trace), np.asarray(ref["f"])
    ig, ir = rep["iterations"], ref["iters"]
    assert ig % E == 0 and ir % E == 0
    assert abs(ig - ir) <= 2 * E, (ig, ir)
    s2 = float((S64 ** 2).sum())
    floor = 0.05 * s2
    common = np.arange(0, min(ig, ir) + 1, E)
    assert np.all(np.isfinite(fg[common])) and np.all(np.isfinite(fr[common]))
    assert traj_rel(fg[common], fr[common], s2).max() <= 1e-3
    if ig != ir:
        t_stop = min(ig, ir)
        later = fg if ig > ir else fr
        ratio = abs(later[t_stop - E] - later[t_stop]) / (
            1e-6 * E * max(abs(later[t_stop - E]), floor))
        assert abs(ratio - 1.0) <= 0.02, ratio
    # directly evaluated objective on the oracle's H at anchors every 200 steps
    for t in sorted(ref["H_at"]):
        if t <= min(ig, ir):
            f_dir = oracle.objective_explicit(S64, ref["H_at"][t])
            assert traj_rel([fg[t]], [f_dir], s2)[0] <= 1e-3, t
    if ig == ir:
        ok, a = labels_agree(res.H.cpu().numpy(), ref["H"])
        assert ok, a
    st = res.state
    assert st.iter == ig and st.blocks == 1 and st.anchor_iter == ig - E
    assert res.H.min().item() >= 0.0


def test_fit_resume_block_svrg_equals_uninterrupted(torch, api):
    """A Block-SVRG AdaptGrow run on the config-3 TPDM split mid-epoch, on an
    anchor and after the sample has grown (stall_tol 0.5 doubles at most
    anchors), resumed from the returned state (|B|, anchor H~ P~, anchor and
    previous objectives, absolute step index) and G: bit for bit the
    uninterrupted run, including where it stops."""
    w = synth.workload("tstress_n8192_k24")
    S = oracle.tpdm(w.X, 0.05).astype(np.float32)
    Sd = S_to_dev(S, torch)
    kw = dict(solver="block_svrg", phi0=1.0 / 8, block_rows=1024, tol_rel=1e-6, stall_tol=0.5,
              seed=3)
    one = api.fit(Sd, w.k, max_iters=60, return_G=True, return_state=True, **kw)
    for split in (5, 8, 19, 30):
        a = api.fit(Sd, w.k, max_iters=split, return_G=True, return_state=True, **kw)
        assert a.state.iter == split
        b = api.fit(Sd, w.k, max_iters=60 - split, H0=a.H, G0=a.G, state=a.state,
                    return_state=True, **kw)
        assert torch.equal(b.H, one.H), split
        assert torch.equal(b.G, one.G), split
        assert b.state.iter == one.state.iter and b.state.blocks == one.state.blocks
        assert b.state.anchor_iter == one.state.anchor_iter
        assert torch.equal(b.state.H_anchor, one.state.H_anchor)
        ft = np.concatenate([a.f_trace, b.f_trace])
        np.testing.assert_array_equal(np.isnan(ft), np.isnan(one.f_trace))
        np.testing.assert_array_equal(ft[~np.isnan(ft)], one.f_trace[~np.isnan(one.f_trace)])
        assert a.report["doublings"] + b.report["doublings"] == one.report["doublings"]
    assert one.report["doublings"] >= 2 and one.report["final_branch"] == 0


def test_fit_resume_full_batch_with_stop_test(torch, api, c1):
    """Full batch with the stop test on: the resumed call tests its first step
    against the restored previous objective, so split and uninterrupted runs
    stop at the same step with the same H."""
    w, S = c1
    Sd = S_to_dev(S, torch)
    kw = dict(solver="full", seed=0, lr=0.05, tol_rel=2e-4)
    init = dict(init="uniform", init_scale=0.1)
    one = api.fit(Sd, w.k, max_iters=400, return_G=True, return_state=True, **init, **kw)
    assert one.converged and 10 < one.report["iterations"] < 400
    # the stop falls on the second resumed step, whose test needs the first's f
    split = one.report["iterations"] - 1
    a = api.fit(Sd, w.k, max_iters=split, return_G=True, return_state=True, **init, **kw)
    assert a.state.f_prev_valid == 1
    b = api.fit(Sd, w.k, max_iters=400 - split, H0=a.H, G0=a.G, state=a.state, **kw)
    assert b.converged and b.report["iterations"] == 1
    assert torch.equal(b.H, one.H)
    # the stop falls on the first resumed step: only the restored f_prev can fire it
    a2 = api.fit(Sd, w.k, max_iters=split + 1, return_G=True, return_state=True, **init, **kw)
    assert not a2.converged and a2.state.f_prev_valid == 1
    b2 = api.fit(Sd, w.k, max_iters=10, H0=a2.H, G0=a2.G, state=a2.state, **kw)
    assert b2.converged and b2.report["iterations"] == 0
    assert torch.equal(b2.H, one.H)


def test_fit_launches_stop_at_the_stop_step(torch, api):
    """Passes enqueued after the device stop flag return without work and are
    not timed: the upper-triangle pass is counted once per exact step actually
    evaluated (anchors plus full-batch steps up to and including the stop
    step)."""
    w = synth.workload("tfactor_n8192_k24")
    S = oracle.abs_corr(w.X).astype(np.float32)
    Sd = S_to_dev(S, torch)
    from symmetric_nmf_clustering_amd import _lib as L
    api.profile_enable(True)
    api.profile_reset()
    res = api.fit(Sd, w.k, solver="full", max_iters=2000, tol_rel=1e-6, seed=1, sh_pass="upper",
                  check_every=16)
    sym = api.profile_read(L.PROF_SH_SYM)
    upd = api.profile_read(L.PROF_UPDATE)
    api.profile_enable(False)
    it = res.report["iterations"]
    print(f"stop step {it}: {15 - it % 16} passes enqueued after it")
    assert res.converged
    assert sym["launches"] == it + 1, (sym["launches"], it)
    assert upd["launches"] == it + 1
