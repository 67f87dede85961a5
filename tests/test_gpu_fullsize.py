"""Full-size parity at n = 100 000, k = 24 (40 GB S), in the launch configuration
the benchmark times. The oracle computes sampled rows one by one from the
returns window; whole-matrix facts are checked as properties that hold at any
size."""
import numpy as np
import pytest
from sklearn.metrics import adjusted_rand_score

import oracle
from symmetric_nmf_clustering_amd import synth
from tests.gpu_util import require_gpu, s_close, to_dev

pytestmark = pytest.mark.gpu

N, K = 100000, 24


@pytest.fixture(scope="module")
def big():
    torch = require_gpu()
    from symmetric_nmf_clustering_amd import api
    free, total = torch.cuda.mem_get_info()
    if free < 48e9:
        pytest.skip("needs ~48 GB of free device memory")
    w = synth.workload("tfactor_n100000_k24")
    S, fro = api.build_S(to_dev(w.X, torch), "abscorr")
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, 511, 512, 4095, 50000, N - 2, N - 1],
                                     rng.integers(0, N, 40)]))
    yield torch, api, w, S, fro, rows
    del S
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def oracle_S(big):
    """The oracle's own fp64 S of the window (80 GB of host memory), built
    block by block from the returns, and its ||S||_F^2."""
    import psutil
    if psutil.virtual_memory().available < 110e9:
        pytest.skip("needs ~100 GB of free host memory for the oracle's fp64 S")
    w = big[2]
    Sh = np.empty((N, N), np.float64)
    fro_o = 0.0
    for r0 in range(0, N, 2000):
        blk = oracle.abs_corr_rows(w.X, np.arange(r0, min(N, r0 + 2000)))
        Sh[r0:r0 + blk.shape[0]] = blk
        fro_o += float(np.square(blk).sum())
        del blk
    yield Sh, fro_o
    del Sh


def test_fullsize_S_rows_and_symmetry(big):
    torch, api, w, S, fro, rows = big
    got = S[torch.from_numpy(rows).cuda()].cpu().numpy()
    ref = oracle.abs_corr_rows(w.X, rows)
    ok, worst = s_close(got, ref)
    assert ok, worst
    # bitwise symmetric: row i equals column i
    cols = S[:, torch.from_numpy(rows).cuda()].cpu().numpy().T
    assert np.array_equal(got, cols)
    assert np.isfinite(fro) and fro > 0


def test_fullsize_sh_rows(big):
    torch, api, w, S, fro, rows = big
    H = synth.random_factor(N, K, seed=3, scale=0.1)
    P, tr = api.sh(S, to_dev(H, torch))
    Pg = P.cpu().numpy().astype(np.float64)
    S_rows = oracle.abs_corr_rows(w.X, rows)
    Pr, _ = oracle.sh_product(S_rows, H, rows=rows)
    rel = np.abs(Pg[rows] - Pr) / np.abs(Pr)
    assert rel.max() <= 1e-4, rel.max()
    # tr(H^T S H) = sum_i <H_i, P_i> over all rows (a property of the outputs)
    assert abs(tr - float((H.astype(np.float64) * Pg).sum())) <= 1e-9 * abs(tr)


def test_fullsize_probe_width_pass(big):
    """The probe's S.Q pass at width 80 (64 + 16 oversampling) with a signed
    basis, as the probe runs it (the LDS-ring kernel): sampled rows against the
    oracle, bounded relative to |S||Q|, and bit for bit against the register
    panel kernel, which a misaligned Q selects."""
    torch, api, w, S, fro, rows = big
    W = 80
    rng = np.random.default_rng(5)
    Q = (rng.standard_normal((N, W)) / np.sqrt(N)).astype(np.float32)
    Qd = to_dev(Q, torch)
    P, _ = api.sh(S, Qd)
    Pg = P.cpu().numpy().astype(np.float64)
    S_rows = oracle.abs_corr_rows(w.X, rows)
    Pr, _ = oracle.sh_product(S_rows, Q, rows=rows)
    # bounded relative to |S||Q| (signed terms cancel), as for the small signed
    # case; the fp32 S and the fixed-order fp32 sums measure ~3e-8 here
    scale = np.abs(S_rows) @ np.abs(Q.astype(np.float64))
    err = (np.abs(Pg[rows] - Pr) / scale).max()
    print(f"probe-width pass: max |P - P_ref| / (|S||Q|) = {err:.2e}")
    assert err <= 1e-5, err
    buf = torch.empty(N * W + 4, dtype=torch.float32, device="cuda")
    Qm = buf[1:1 + N * W].view(N, W)
    Qm.copy_(Qd)
    assert Qd.data_ptr() % 16 == 0 and Qm.data_ptr() % 16 == 4
    Pm, _ = api.sh(S, Qm)
    assert torch.equal(P, Pm)


@pytest.mark.parametrize("W", [80, 128])
def test_fullsize_probe_product(big, W):
    """symnmf_sq, the probe's pass (bf16 matrix cores, exact three-part operand
    split), at probe widths with a signed basis: sampled rows against the
    oracle, bounded relative to |S||Q|, and against the fp32 S.H pass."""
    torch, api, w, S, fro, rows = big
    rng = np.random.default_rng(W)
    Q = (rng.standard_normal((N, W)) / np.sqrt(N)).astype(np.float32)
    Qd = to_dev(Q, torch)
    Y = api.sq(S, Qd)
    Yg = Y.cpu().numpy().astype(np.float64)
    S_rows = oracle.abs_corr_rows(w.X, rows)
    Yr, _ = oracle.sh_product(S_rows, Q, rows=rows)
    scale = np.abs(S_rows) @ np.abs(Q.astype(np.float64))
    err = (np.abs(Yg[rows] - Yr) / scale).max()
    print(f"probe product w={W}: max |Y - Y_ref| / (|S||Q|) = {err:.2e}")
    assert err <= 1e-5, err
    P, _ = api.sh(S, Qd)
    d = (np.abs(Yg[rows] - P.cpu().numpy()[rows]) / scale).max()
    assert d <= 1e-5, d


def test_fullsize_probe_against_oracle_subspace(big, oracle_S):
    """The probe as the benchmark runs it (p = 64, tol 1e-6, 128 columns)
    against the oracle's fp64 subspace iteration on its own S: the 24
    planted-factor eigenvalues, which a clear gap separates from the bulk (so
    12 oracle steps pin them to their residuals), within the probe's bound;
    the squares of all 64 values below the oracle's ||S||_F^2."""
    torch, api, w, S, fro, rows = big
    Sh, fro_o = oracle_S
    tol = 1e-6
    ev, its, conv = api.spectral_probe(S, p=64, max_iters=400, tol=tol, seed=0)
    assert conv
    print(f"probe: {its} steps, theta_1 = {ev[0]:.6f}")
    theta, resid = oracle.subspace_top_eigenvalues(lambda V: Sh @ V, N, 32, iters=12, seed=1)
    lam1 = abs(theta[0])
    assert resid[:24].max() <= 1e-6 * lam1, resid[:24].max()
    err = np.abs(ev[:24] - theta[:24])
    print(f"max |theta_gpu - theta_oracle| / |lambda_1| over the top 24 = {err.max() / lam1:.2e}")
    assert np.all(err <= 100 * tol * lam1 + resid[:24]), err.max() / lam1
    assert float(np.square(ev).sum()) <= fro_o * (1 + 1e-6)
    assert abs(fro - fro_o) <= 1e-5 * fro_o  # the library's ||S||^2 from the build


def test_fullsize_block_svrg_two_steps(big, oracle_S):
    """Block-SVRG as the benchmark starts it (32 of 98 blocks of 1024 rows):
    an anchor step (exact S H) and a sampled step (the anchor's P plus
    98/32 times the sampled rows' correction S[B,:]^T (H - H~)[B,:]), every
    row of H against the oracle's AdaptGrow on its fp64 S. AdaGrad's steps
    are lr g / sqrt(G): compared where both gradients are decided well above
    the fp32 noise."""
    torch, api, w, S, fro, rows = big
    Sh, fro_o = oracle_S
    lr, phi0, seed = 0.05, 32.0 / 98.0, 5
    res = api.fit(S, K, solver="block_svrg", phi0=phi0, init="uniform", init_scale=0.1,
                  seed=seed, lr=lr, max_iters=2, tol_rel=0.0)
    assert res.report["blocks_final"] == 32 and res.report["anchors"] == 1
    H0 = oracle.init_uniform(N, K, 0.1, seed)
    ref = oracle.fit_adaptgrow(Sh, H0, lr, 2, solver=oracle.SOLVER_BLOCK_SVRG, phi0=phi0,
                               seed=seed, tol=0.0)
    assert ref["nsel"] == 32
    # the two gradients, to mask where a step's sign is decided by rounding
    P0 = Sh @ H0
    g0 = 4.0 * (H0 @ (H0.T @ H0) - P0)
    H1 = np.maximum(H0 - lr * g0 / (np.sqrt(g0 * g0) + 1e-8), 0.0)
    blocks = oracle.sample_blocks(seed, 1, 98, 32)
    g1 = 4.0 * (H1 @ (H1.T @ H1) - oracle.svrg_sh_estimate(Sh, H1, H0, P0, blocks, 1024))
    decided = (np.abs(g0) > 1e-3 * np.abs(g0).max()) & (np.abs(g1) > 1e-3 * np.abs(g1).max())
    assert decided.mean() > 0.8, decided.mean()
    H2 = res.H.cpu().numpy().astype(np.float64)
    err = np.abs(H2 - ref["H"])[decided].max()
    print(f"Block-SVRG two steps: max |H - H_ref| (decided entries) = {err:.2e}")
    assert err <= 1e-5, err
    assert abs(res.f_trace[0] - ref["f"][0]) <= 1e-6 * ref["f"][0]
    assert np.isnan(res.f_trace[1]) and np.isnan(ref["f"][1])


def test_fullsize_tpdm_rows_trace_and_spectrum(big):
    """The TPDM of the same window at n = 100 000 (rank <= m = 13 tail days):
    sampled rows against the oracle's rows, bitwise symmetry, tr S = 1 (unit
    angular components, 1/m scaling), and the closed form of its spectrum:
    the nonzero eigenvalues of Theta^T Theta / m are those of the m x m matrix
    Theta Theta^T / m, which pins ||S||^2 from the build and the probe's
    values (the rest of the probe's values are the null space, ~0)."""
    torch, api, w, S, fro, rows = big
    St, fro_t = api.build_S(to_dev(w.X, torch), "tpdm")
    try:
        theta, _, m = oracle.tpdm_angles(w.X)
        got = St[torch.from_numpy(rows).cuda()].cpu().numpy()
        ok, worst = s_close(got, oracle.tpdm_rows(w.X, rows))
        assert ok, worst
        assert np.array_equal(got, St[:, torch.from_numpy(rows).cuda()].cpu().numpy().T)
        assert abs(float(torch.diagonal(St).double().sum()) - 1.0) <= 1e-5
        lam = np.sort(np.linalg.eigvalsh(theta @ theta.T / m))[::-1]
        fro_ref = float(np.square(lam).sum())
        assert abs(fro_t - fro_ref) <= 1e-5 * fro_ref
        ev, its, conv = api.spectral_probe(St, p=26, max_iters=200, tol=1e-6, seed=0)
        print(f"TPDM probe: {its} steps, lambda_1 = {ev[0]:.6e} (closed form {lam[0]:.6e})")
        assert np.all(np.abs(ev[:m] - lam) <= 1e-4 * lam[0])
        assert np.all(np.abs(ev[m:]) <= 1e-4 * lam[0])
    finally:
        del St
        torch.cuda.empty_cache()


def test_fullsize_sh_sym_rows(big):
    """The upper-triangle pass as the benchmark's fit runs it (k = 24, 512-column
    strips, 2048-row chunks): sampled rows, strip and chunk edges among them,
    against the oracle's rows built from the returns; the trace against the sum
    of its own outputs; and the row-panel pass on the same rows."""
    torch, api, w, S, fro, rows = big
    rows = np.unique(np.concatenate([rows, [2047, 2048, 4095, 4096, 8191, 8192, 99839, 99840]]))
    H = synth.random_factor(N, K, seed=3, scale=0.1)
    Hd = to_dev(H, torch)
    P, tr = api.sh_sym(S, Hd)
    Pg = P.cpu().numpy().astype(np.float64)
    S_rows = oracle.abs_corr_rows(w.X, rows)
    Pr, _ = oracle.sh_product(S_rows, H, rows=rows)
    rel = np.abs(Pg[rows] - Pr) / np.abs(Pr)  # S, H >= 0: |P| = |S||H|
    print(f"upper-triangle pass: max rel error over {rows.size} rows = {rel.max():.2e}")
    assert rel.max() <= 1e-4, rel.max()
    assert abs(tr - float((H.astype(np.float64) * Pg).sum())) <= 1e-9 * abs(tr)
    Pf, trf = api.sh(S, Hd)
    d = np.abs(Pg[rows] - Pf.cpu().numpy()[rows]) / np.abs(Pr)
    assert d.max() <= 1e-4, d.max()
    assert abs(tr - trf) <= 1e-5 * abs(trf)


@pytest.mark.parametrize("sh_pass", ["rows", "upper"])
def test_fullsize_first_step_and_objective(big, sh_pass):
    torch, api, w, S, fro, rows = big
    lr = 0.05
    res = api.fit(S, K, solver="full", init="uniform", init_scale=0.1, seed=5, lr=lr,
                  max_iters=1, tol_rel=0.0, sh_pass=sh_pass)
    H0 = oracle.init_uniform(N, K, 0.1, 5)
    K0 = H0.T @ H0
    S_rows = oracle.abs_corr_rows(w.X, rows)
    P_rows, _ = oracle.sh_product(S_rows, H0, rows=rows)
    g = 4.0 * (H0[rows] @ K0 - P_rows)
    H1_ref = np.maximum(H0[rows] - lr * g / (np.abs(g) + 1e-8), 0.0)
    H1 = res.H.cpu().numpy()[rows].astype(np.float64)
    # the first AdaGrad step is lr * sign(g) unless |g| is tiny; compare where
    # the sign is decided well above the fp32 noise of g
    decided = np.abs(g) > 1e-3 * np.abs(g).max()
    assert decided.mean() > 0.9
    assert np.abs(H1 - H1_ref)[decided].max() <= 1e-5
    # f_0 by the trace identity equals ||S||^2 - 2 tr + ||K0||^2 with the
    # build's ||S||^2 and the S.H pass's trace
    _, tr0 = (api.sh if sh_pass == "rows" else api.sh_sym)(S, to_dev(H0, torch))
    f0 = fro - 2.0 * tr0 + float((K0 * K0).sum())
    assert abs(res.f_trace[0] - f0) <= 1e-6 * f0
    assert abs(res.report["S_fro2"] - fro) <= 1e-9 * fro


def test_fullsize_labels_property(big):
    torch, api, w, S, fro, rows = big
    res = api.fit(S, K, solver="full", max_iters=30, tol_rel=0.0, seed=0)
    lab = api.labels(res.H).cpu().numpy()
    H = res.H.cpu().numpy()
    # argmax property on every row, lowest index on ties
    mx = H.max(axis=1)
    assert np.all(H[np.arange(N), lab] == mx)
    first = np.argmax(H == mx[:, None], axis=1)
    assert np.array_equal(first, lab)
    assert res.H.min().item() >= 0.0


def test_fullsize_spherical_kmeans(big):
    """Spherical k-means at n = 100 000 in the benchmark's S: converges, the
    labels are the row argmax of S C^T against the returned centroids on
    sampled rows (recomputed in fp64 from the returns), and the planted groups
    are found up to a few merged ones."""
    torch, api, w, S, fro, rows = big
    res = api.spherical_kmeans(S, K, seed=0, return_centroids=True)
    assert res.converged
    lab = res.labels.cpu().numpy()
    C = res.centroids.cpu().numpy().astype(np.float64)
    S_rows = oracle.abs_corr_rows(w.X, rows)
    sims = S_rows @ C
    best = sims.max(axis=1)
    # the chosen centroid is the most similar one up to fp32 noise of S C^T
    assert np.all(sims[np.arange(rows.size), lab[rows]] >= best - 1e-5 * np.abs(best))
    # a local optimum from k seeded random rows (measured ARI 0.89)
    assert adjusted_rand_score(lab, w.labels) >= 0.8


def test_fullsize_warm_start_next_window(big):
    """Cold vs warm start at full size: the window one day on (the returns moved
    by a day plus one new day of the recipe), fitted from the current window's
    H with a fresh accumulator, as Block-SVRG starts here (32 of 98 blocks).
    Its first two steps on sampled rows against the oracle, which builds those
    rows of the new S from the shifted returns: the anchor step (exact S' H),
    then, from the device's state after it, the sampled step (the anchor's
    product plus 98/32 times the sampled blocks' correction). Compared where
    the gradient is decided well above fp32 noise, as the cold-start tests."""
    torch, api, w, S, fro, rows = big
    lr_b, phi0, seed = 0.05, 32.0 / 98.0, 5
    base = api.fit(S, K, solver="full", init="uniform", init_scale=0.1, seed=0, lr=lr_b,
                   max_iters=100, tol_rel=0.0, sh_pass="upper")
    Ht = base.H
    nxt = synth.student_factor_next(n=N, k=K, T=w.T, seed=w.seed, shift=1)
    S2, _ = api.build_S(to_dev(nxt.X, torch), "abscorr")
    kw = dict(solver="block_svrg", phi0=phi0, seed=seed, tol_rel=0.0, sh_pass="upper", H0=Ht,
              return_G=True)
    one = api.fit(S2, K, max_iters=1, **kw)
    two = api.fit(S2, K, max_iters=2, **kw)
    del S2
    assert one.report["blocks_final"] == 32 and one.report["anchors"] == 1
    lr, eps = one.report["lr_used"], 1e-8
    H0 = Ht.cpu().numpy().astype(np.float64)
    S_rows = oracle.abs_corr_rows(nxt.X, rows)          # rows of the new S, fp64
    P0, _ = oracle.sh_product(S_rows, H0, rows=rows)
    g0 = 4.0 * (H0[rows] @ (H0.T @ H0) - P0)
    H1_ref = np.maximum(H0[rows] - lr * g0 / (np.abs(g0) + eps), 0.0)
    dec0 = np.abs(g0) > 1e-3 * np.abs(g0).max()
    assert dec0.mean() > 0.8, dec0.mean()
    H1 = one.H.cpu().numpy().astype(np.float64)
    err1 = np.abs(H1[rows] - H1_ref)[dec0].max()
    # the sampled step from the device's (H1, G1): the correction of row i is
    # sum over the sampled blocks' rows j of S'[i, j] (H1 - H0)[j]
    G1 = one.G.cpu().numpy().astype(np.float64)
    blocks = oracle.sample_blocks(seed, 1, 98, 32)
    cols = np.concatenate([np.arange(b * 1024, min(N, (b + 1) * 1024)) for b in blocks])
    corr = S_rows[:, cols] @ (H1[cols] - H0[cols])
    P1 = P0 + (98.0 / 32.0) * corr
    g1 = 4.0 * (H1[rows] @ (H1.T @ H1) - P1)
    G2 = G1[rows] + g1 * g1
    H2_ref = np.maximum(H1[rows] - lr * g1 / (np.sqrt(G2) + eps), 0.0)
    dec1 = np.abs(g1) > 1e-3 * np.abs(g1).max()
    H2 = two.H.cpu().numpy().astype(np.float64)[rows]
    err2 = np.abs(H2 - H2_ref)[dec1].max()
    print(f"warm start, next window: first step {err1:.2e}, sampled step {err2:.2e} "
          f"(decided {dec0.mean():.3f} / {dec1.mean():.3f})")
    assert err1 <= 1e-5 and err2 <= 1e-5, (err1, err2)
    assert np.isnan(two.f_trace[1]) and np.isfinite(two.f_trace[0])
