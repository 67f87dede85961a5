"""Pins for the oracle's objective, gradient, AdaGrad step and full-batch fit."""
import json
import os

import numpy as np
import pytest

import oracle


def _rand_sym(n, seed):
    rng = np.random.default_rng(seed)
    A = rng.random((n, n))
    return (A + A.T) / 2


def test_page_constants(golden_dir):
    c = json.load(open(os.path.join(golden_dir, "page_constants.json")))
    # the oracle's defaults are the sketch's
    import inspect
    sig = inspect.signature(oracle.adagrad_step)
    assert sig.parameters["eps"].default == c["eps"]["value"]
    assert inspect.signature(oracle.gap_ratio).parameters["k"] is not None
    assert inspect.signature(oracle.initial_blocks).parameters["threshold"].default == c["gap_threshold"]["value"]
    # 4 n^2 bytes for fp32 S: 40 GB at 1e5, 4 TB at 1e6
    for n, b in zip(c["dense_S_bytes"]["n"], c["dense_S_bytes"]["approx_bytes"]):
        assert abs(4 * n * n - b) / b < 0.01


@pytest.mark.parametrize("n,k,seed", [(5, 2, 0), (12, 3, 1), (30, 7, 2)])
def test_trace_identity_equals_explicit(n, k, seed):
    S = _rand_sym(n, seed)
    H = np.random.default_rng(seed + 10).random((n, k))
    f_exp = oracle.objective_explicit(S, H)
    f_tr = oracle.objective_trace((S * S).sum(), H, S @ H)
    assert abs(f_exp - f_tr) <= 1e-12 * f_exp


def test_gradient_central_differences():
    n, k = 8, 3
    S = _rand_sym(n, 4)
    H = np.random.default_rng(5).random((n, k))
    g = oracle.gradient(S, H)
    h = 1e-6
    fd = np.zeros_like(H)
    for i in range(n):
        for c in range(k):
            Hp = H.copy(); Hp[i, c] += h
            Hm = H.copy(); Hm[i, c] -= h
            fd[i, c] = (oracle.objective_explicit(S, Hp) - oracle.objective_explicit(S, Hm)) / (2 * h)
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-6 * np.abs(g).max())


def test_first_step_closed_form():
    # from G = 0, sqrt(G + g^2) = |g|, so H1 = max(H0 - eta g/(|g| + eps), 0)
    n, k, eta, eps = 10, 3, 0.05, 1e-8
    S = _rand_sym(n, 6)
    H0 = np.random.default_rng(7).random((n, k)) * 0.3
    out = oracle.fit_full(S, H0, eta, max_iters=1, eps=eps)
    g = oracle.gradient(S, H0)
    np.testing.assert_allclose(out["H"], np.maximum(H0 - eta * g / (np.abs(g) + eps), 0), rtol=1e-15, atol=0)
    np.testing.assert_allclose(out["G"], g * g, rtol=1e-15)
    assert out["iters"] == 1 and len(out["f"]) == 1


def test_eps_outside_root_and_minus_sign():
    # a single coordinate: G = 4, g = 2 -> step eta*2/(2+eps); a wrong sign or
    # eps inside the root changes the value
    H, G = oracle.adagrad_step(np.array([[1.0]]), np.array([[0.0]]), np.array([[2.0]]), 0.5, eps=0.25)
    assert G[0, 0] == 4.0
    assert H[0, 0] == pytest.approx(1.0 - 0.5 * 2.0 / (2.0 + 0.25), rel=1e-15)


def test_projection_keeps_H_nonnegative_every_step():
    n, k = 40, 4
    S = _rand_sym(n, 8)
    H = np.random.default_rng(9).random((n, k))
    G = np.zeros_like(H)
    for _ in range(50):
        g = oracle.gradient(S, H)
        H, G = oracle.adagrad_step(H, G, g, 0.2)
        assert H.min() >= 0.0
    assert (H == 0).any()  # the projection is active on this input


def test_fit_objective_paths_agree():
    S = _rand_sym(20, 11)
    H0 = oracle.init_uniform(20, 3, 0.5, 3)
    a = oracle.fit_full(S, H0, 0.05, 30, objective="trace")
    b = oracle.fit_full(S, H0, 0.05, 30, objective="explicit")
    np.testing.assert_allclose(a["f"], b["f"], rtol=1e-12)
    np.testing.assert_array_equal(a["H"], b["H"])


def test_planted_blocks_recovered():
    # noise-free planted S = blockdiag(1 1^T): f -> 0 and argmax recovers the blocks
    n, k = 64, 4
    truth = np.repeat(np.arange(k), n // k)
    S = (truth[:, None] == truth[None, :]).astype(np.float64)
    a = oracle.init_scale_matched(S.mean(), k)
    H0 = oracle.init_uniform(n, k, a, 0)
    out = oracle.fit_full(S, H0, oracle.default_lr(S.mean(), k), 2000, tol=0.0)
    assert out["f"][-1] < 1e-6 * (S * S).sum()
    assert oracle.ari(oracle.labels(out["H"]), truth) == 1.0


def test_convergence_rule_stops_before_update():
    S = _rand_sym(16, 12)
    H0 = oracle.init_uniform(16, 2, 0.3, 1)
    full = oracle.fit_full(S, H0, 0.02, 400, tol=0.0)
    f = np.array(full["f"])
    tol = 1e-4
    rel = np.abs(np.diff(f)) / np.abs(f[:-1])
    t_stop = int(np.argmax(rel < tol)) + 1
    out = oracle.fit_full(S, H0, 0.02, 400, tol=tol)
    assert out["converged"] and out["iters"] == t_stop
    np.testing.assert_allclose(out["f"], f[: t_stop + 1], rtol=0, atol=0)
    # the returned H is H_t (before the update of step t)
    ref = oracle.fit_full(S, H0, 0.02, t_stop, tol=0.0)
    np.testing.assert_array_equal(out["H"], ref["H"])


def test_default_init_and_lr_readings():
    # E[(H0 H0^T)_ij] = k (a/2)^2 = mean(S) for U(0, a)
    a = oracle.init_scale_matched(0.06, 24)
    assert 24 * (a / 2) ** 2 == pytest.approx(0.06)
    assert oracle.default_lr(0.06, 24) == pytest.approx(a / 2)


def test_sh_product_rows_match_full():
    S = _rand_sym(30, 13)
    H = np.random.default_rng(14).random((30, 4))
    P, tr = oracle.sh_product(S, H)
    rows = np.array([3, 7, 29])
    Pr, trr = oracle.sh_product(S[rows], H, rows=rows)
    np.testing.assert_allclose(Pr, P[rows], rtol=1e-14)
    assert trr == pytest.approx(float((H[rows] * P[rows]).sum()), rel=1e-13)
    assert tr == pytest.approx(float(np.trace(H.T @ S @ H)), rel=1e-13)


def test_rmsprop_first_step_and_constant_gradient():
    """RMSprop (Tieleman and Hinton 2012): from G = 0 the first step is
    lr g / (sqrt(1 - rho) |g| + eps); under a constant gradient the moving
    average is the geometric sum G_t = (1 - rho^t) g^2; rho = 0 in fit_full is
    AdaGrad."""
    rho, lr, eps = 0.9, 0.05, 1e-8
    H0 = np.array([[1.0, 0.5, 0.2]])
    g = np.array([[2.0, -0.3, 1e-3]])
    H1, G1 = oracle.rmsprop_step(H0, np.zeros_like(H0), g, lr, rho, eps)
    np.testing.assert_allclose(G1, (1 - rho) * g * g, rtol=1e-15)
    np.testing.assert_allclose(H1, np.maximum(H0 - lr * g / (np.sqrt(1 - rho) * np.abs(g) + eps), 0),
                               rtol=1e-15)
    G = np.zeros_like(H0)
    H = np.full_like(H0, 10.0)
    for t in range(1, 30):
        H, G = oracle.rmsprop_step(H, G, g, lr, rho, eps)
        np.testing.assert_allclose(G, (1 - rho ** t) * g * g, rtol=1e-12)
    S = _rand_sym(12, 21)
    Hs = oracle.init_uniform(12, 3, 0.3, 2)
    a = oracle.fit_full(S, Hs, 0.02, 20, rho=0.0)
    b = oracle.fit_full(S, Hs, 0.02, 20)
    np.testing.assert_array_equal(a["H"], b["H"])
    c = oracle.fit_full(S, Hs, 0.02, 20, rho=0.9)
    assert not np.array_equal(c["H"], b["H"]) and c["H"].min() >= 0.0
