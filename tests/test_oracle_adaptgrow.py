"""Pins for the oracle's AdaptGrow schedule: anchor steps, sample doubling, the
switch to full batch with the accumulator kept, the stopping test at anchors
and in the full branch (with its objective-scale floor), and resumption.

Each run is checked against a hand composition of pinned pieces (the exact
product S @ H, ``svrg_sh_estimate`` pinned by enumeration, ``sample_blocks``
and ``adagrad_step`` pinned elsewhere) that follows a schedule written out
here from the rule (the AdaptGrow sketch of "GPU-Accelerated SymNMF Clustering
Scales to a Million Financial Instruments": phi doubles toward 1 when progress
stalls; "GPU-Accelerated Clustering for Financial Instruments at Scale",
"Factorizing with SymNMF" and "Why this solver": sampled SVRG steps first, the
sample grown toward the full gradient), not by re-running the oracle's loop.
"""
import numpy as np
import pytest

import oracle


def _problem(n=64, k=3, seed=0):
    rng = np.random.default_rng(seed)
    A = rng.random((n, n))
    S = (A + A.T) / 2
    H0 = oracle.init_uniform(n, k, 0.4, seed + 1)
    return S, H0


def _compose(S, H0, lr, schedule, seed, block_rows, steps):
    """H_t, G_t for t = 0..steps following ``schedule(t)`` ->
    ('anchor', None) | ('sampled', nsel) | ('full', None)."""
    n = S.shape[0]
    nb = -(-n // block_rows)
    H, G = H0.copy(), np.zeros_like(H0)
    Hs, Gs, kinds = [H.copy()], [G.copy()], []
    Ha = Pa = None
    for t in range(steps):
        kind, nsel = schedule(t)
        kinds.append(kind)
        if kind in ("anchor", "full"):
            P = S @ H
            if kind == "anchor":
                Ha, Pa = H.copy(), P.copy()
        else:
            blocks = oracle.sample_blocks(seed, t, nb, nsel)
            P = oracle.svrg_sh_estimate(S, H, Ha, Pa, blocks, block_rows)
        g = 4.0 * (H @ (H.T @ H) - P)
        H, G = oracle.adagrad_step(H, G, g, lr)
        Hs.append(H.copy())
        Gs.append(G.copy())
    return Hs, Gs, kinds


def test_growth_schedule_doubles_at_every_stalled_anchor():
    """stall_tol = 1: every anchor after the first counts as stalled (its
    objective fell by less than all of the previous one), so with nb = 8 and
    |B|0 = 1 the anchors are t = 0 (E = 8), 8 (|B| 2, E = 4), 12 (|B| 4,
    E = 2) and 14 (|B| 8 = nb: full batch from here, G kept)."""
    S, H0 = _problem()
    lr, seed, br, steps = 0.02, 5, 8, 22

    def schedule(t):
        if t in (0, 8, 12, 14):
            return "anchor", None
        if t < 8:
            return "sampled", 1
        if t < 12:
            return "sampled", 2
        if t < 14:
            return "sampled", 4
        return "full", None

    Hs, Gs, kinds = _compose(S, H0, lr, schedule, seed, br, steps)
    out = oracle.fit_adaptgrow(S, H0, lr, steps, solver=oracle.SOLVER_BLOCK_SVRG, phi0=1 / 8,
                               block_rows=br, tol=0.0, stall_tol=1.0, seed=seed)
    assert out["history"] == [(8, 2), (12, 4), (14, 8)]
    assert out["anchors"] == [0, 8, 12, 14]
    assert out["final_branch"] == "full" and out["nsel"] == 8
    f = np.asarray(out["f"])
    sampled = np.array([k == "sampled" for k in kinds])
    assert np.array_equal(np.isnan(f), sampled)
    np.testing.assert_allclose(out["H"], Hs[steps], rtol=1e-13, atol=0)
    np.testing.assert_allclose(out["G"], Gs[steps], rtol=1e-13, atol=0)   # G kept at the switch
    # step by step: every prefix of the run is the composition's prefix
    for t in (1, 7, 8, 9, 12, 13, 14, 15):
        o = oracle.fit_adaptgrow(S, H0, lr, t, solver=oracle.SOLVER_BLOCK_SVRG, phi0=1 / 8,
                                 block_rows=br, tol=0.0, stall_tol=1.0, seed=seed)
        np.testing.assert_allclose(o["H"], Hs[t], rtol=1e-13, atol=0)
    # anchor objectives are the exact ones of the composed H
    for t in (0, 8, 12, 14, 20):
        assert f[t] == pytest.approx(oracle.objective_explicit(S, Hs[t]), rel=1e-10)


def test_no_stall_keeps_the_sample_and_epoch():
    """stall_tol = -1 never doubles: anchors every E = ceil(nb/|B|) steps,
    |B| unchanged, the sampled branch to the end."""
    S, H0 = _problem(n=60, seed=3)
    lr, seed, br, steps = 0.02, 2, 8, 20      # nb = 8, |B| = 3 -> E = 3

    def schedule(t):
        return ("anchor", None) if t % 3 == 0 else ("sampled", 3)

    Hs, _, _ = _compose(S, H0, lr, schedule, seed, br, steps)
    out = oracle.fit_adaptgrow(S, H0, lr, steps, solver=oracle.SOLVER_BLOCK_SVRG, phi0=3 / 8,
                               block_rows=br, tol=0.0, stall_tol=-1.0, seed=seed)
    assert out["history"] == [] and out["anchors"] == list(range(0, steps, 3))
    assert out["final_branch"] == "sampled" and out["nsel"] == 3
    np.testing.assert_allclose(out["H"], Hs[steps], rtol=1e-13, atol=0)


def _stop_tol_for(f_anchor_seq, steps_seq, floor_abs, j):
    """A tolerance at which the anchor test first passes at anchor j: between
    the ratio at j and the smallest ratio before it."""
    r = [abs(a - b) / (e * max(abs(a), floor_abs))
         for a, b, e in zip(f_anchor_seq[:-1], f_anchor_seq[1:], steps_seq)]
    lo = r[j - 1]
    hi = min(r[: j - 1]) if j > 1 else np.inf
    assert lo < hi
    return lo * 1.01 if hi == np.inf else float(np.sqrt(lo * hi)) if lo > 0 else hi / 2


def test_sampled_branch_stops_at_an_anchor_and_returns_its_H():
    """The anchor stop test, |f~prev - f~| < tol E_j max(|f~prev|, floor),
    ends the run at that anchor: iterations = the anchor's step, H = H_t
    before the anchor's update, converged."""
    S, H0 = _problem(n=64, seed=7)
    lr, seed, br = 0.02, 1, 16                 # nb = 4, |B| = 1 -> E = 4
    s2 = float((S * S).sum())
    ref = oracle.fit_adaptgrow(S, H0, lr, 40, solver=oracle.SOLVER_BLOCK_SVRG, phi0=0.25,
                               block_rows=br, tol=0.0, stall_tol=-1.0, seed=seed)
    f = np.asarray(ref["f"])
    anchors = list(range(0, 40, 4))
    assert ref["anchors"] == anchors
    fa = [f[t] for t in anchors]
    j = 4                                      # stop at the anchor of step 16
    tol = _stop_tol_for(fa, [4] * (len(fa) - 1), 0.0, j)
    out = oracle.fit_adaptgrow(S, H0, lr, 40, solver=oracle.SOLVER_BLOCK_SVRG, phi0=0.25,
                               block_rows=br, tol=tol, stall_tol=-1.0, obj_floor=0.0, seed=seed)
    assert out["converged"] and out["iters"] == anchors[j]
    short = oracle.fit_adaptgrow(S, H0, lr, anchors[j], solver=oracle.SOLVER_BLOCK_SVRG,
                                 phi0=0.25, block_rows=br, tol=0.0, stall_tol=-1.0, seed=seed)
    np.testing.assert_array_equal(out["H"], short["H"])
    np.testing.assert_array_equal(np.asarray(out["f"])[:-1], np.asarray(short["f"]))
    assert out["f"][-1] == f[anchors[j]]
    # the floor: with obj_floor large enough that max(|f|, floor) = floor, the
    # same test on the same trajectory fires where |df| < tol E floor
    big = 2.0
    r = [abs(a - b) / (4 * big * s2) for a, b in zip(fa[:-1], fa[1:])]
    assert max(fa) < big * s2 and r[0] > r[1] > r[2]
    tol2 = 0.5 * (r[1] + r[2])
    o2 = oracle.fit_adaptgrow(S, H0, lr, 40, solver=oracle.SOLVER_BLOCK_SVRG, phi0=0.25,
                              block_rows=br, tol=tol2, stall_tol=-1.0, obj_floor=big, seed=seed)
    assert o2["converged"] and o2["iters"] == anchors[3]


def test_floor_lets_an_exactly_factorable_fit_stop():
    """Noise-free planted S = blockdiag(1 1^T) is factored exactly, f -> 0:
    the plain relative test keeps seeing large relative changes and never
    stops within the budget, while with the floor the test turns absolute
    (tol * obj_floor ||S||^2) once f is small and stops at the first step where
    the trajectory's change falls below it."""
    n, k = 64, 4
    truth = np.repeat(np.arange(k), n // k)
    S = (truth[:, None] == truth[None, :]).astype(np.float64)
    s2 = float((S * S).sum())
    H0 = oracle.init_uniform(n, k, oracle.init_scale_matched(S.mean(), k), 0)
    lr = oracle.default_lr(S.mean(), k)
    free = oracle.fit_full(S, H0, lr, 3000, tol=0.0)
    f = np.asarray(free["f"])
    tol = 1e-6
    plain = oracle.fit_full(S, H0, lr, 3000, tol=tol, obj_floor=0.0)
    floored = oracle.fit_full(S, H0, lr, 3000, tol=tol, obj_floor=0.05)
    # where the plain relative test would stop, if anywhere
    rel = np.abs(np.diff(f)) / np.abs(f[:-1])
    absd = np.abs(np.diff(f))
    t_floor = int(np.argmax(absd < tol * np.maximum(np.abs(f[:-1]), 0.05 * s2))) + 1
    assert floored["converged"] and floored["iters"] == t_floor
    assert f[t_floor] < 0.05 * s2                       # the floor is what fired
    assert rel[t_floor - 1] > 10 * tol                  # the plain test would not have
    assert (not plain["converged"]) or plain["iters"] > t_floor
    np.testing.assert_array_equal(floored["H"], oracle.fit_full(S, H0, lr, t_floor)["H"])
    assert oracle.ari(oracle.labels(floored["H"]), truth) == 1.0


def test_full_branch_after_growth_tests_against_the_anchor_objective():
    """After the switch to full batch the first full step's test compares with
    the switching anchor's exact f (an anchor's f counts as the previous exact
    objective)."""
    S, H0 = _problem()
    lr, seed, br = 0.02, 5, 8
    ref = oracle.fit_adaptgrow(S, H0, lr, 30, solver=oracle.SOLVER_BLOCK_SVRG, phi0=1 / 8,
                               block_rows=br, tol=0.0, stall_tol=1.0, seed=seed)
    f = np.asarray(ref["f"])
    # the full branch starts after the anchor at 14; a tolerance that passes
    # first at step 15 against f_14
    d = np.abs(np.diff(f[14:])) / np.abs(f[14:-1])
    tol = d[0] * 1.001
    out = oracle.fit_adaptgrow(S, H0, lr, 30, solver=oracle.SOLVER_BLOCK_SVRG, phi0=1 / 8,
                               block_rows=br, tol=tol, stall_tol=1.0, obj_floor=0.0, seed=seed)
    # no earlier anchor test passes (ratios at anchors 8 and 12 are larger)
    fa = f[[0, 8, 12, 14]]
    E = [8, 4, 2]
    assert all(abs(a - b) / (e * abs(a)) >= tol for a, b, e in zip(fa[:-1], fa[1:], E))
    assert out["converged"] and out["iters"] == 15
    np.testing.assert_array_equal(out["H"], oracle.fit_adaptgrow(
        S, H0, lr, 15, solver=oracle.SOLVER_BLOCK_SVRG, phi0=1 / 8, block_rows=br, tol=0.0,
        stall_tol=1.0, seed=seed)["H"])


@pytest.mark.parametrize("split", [5, 8, 11, 14, 17])
def test_resume_reproduces_the_uninterrupted_run(split):
    """Two calls joined by the returned state (step index, |B|, anchor H~ P~,
    anchor objective, previous exact f) and G take the same steps as one call,
    whether the split falls mid-epoch, on an anchor, or in the full branch."""
    S, H0 = _problem()
    kw = dict(solver=oracle.SOLVER_BLOCK_SVRG, phi0=1 / 8, block_rows=8, tol=1e-9,
              stall_tol=1.0, seed=5)
    one = oracle.fit_adaptgrow(S, H0, 0.02, 24, **kw)
    a = oracle.fit_adaptgrow(S, H0, 0.02, split, **kw)
    b = oracle.fit_adaptgrow(S, a["H"], 0.02, 24 - split, G0=a["G"], state=a["state"], **kw)
    np.testing.assert_array_equal(b["H"], one["H"])
    np.testing.assert_array_equal(b["G"], one["G"])
    np.testing.assert_array_equal(np.asarray(a["f"] + b["f"]), np.asarray(one["f"]))
    assert a["history"] + b["history"] == one["history"]
    assert a["anchors"] + b["anchors"] == one["anchors"]
    assert b["state"]["t"] == 24


def test_adaptgrow_explicit_objective_matches_trace():
    S, H0 = _problem(n=40, seed=9)
    kw = dict(solver=oracle.SOLVER_BLOCK_SVRG, phi0=0.2, block_rows=8, tol=0.0, stall_tol=1.0,
              seed=3)
    a = oracle.fit_adaptgrow(S, H0, 0.02, 20, objective="trace", **kw)
    b = oracle.fit_adaptgrow(S, H0, 0.02, 20, objective="explicit", **kw)
    np.testing.assert_allclose(a["f"], b["f"], rtol=1e-12)
    np.testing.assert_array_equal(a["H"], b["H"])


def test_objective_explicit_slices_agree():
    rng = np.random.default_rng(2)
    A = rng.random((50, 50))
    S = A + A.T
    H = rng.random((50, 4))
    R = S - H @ H.T
    for rows in (1, 7, 50, 1024):
        assert oracle.objective_explicit(S, H, rows_per_slice=rows) == pytest.approx(
            float((R * R).sum()), rel=1e-13)


def test_first_doubling_at_the_first_anchor_whose_decrease_is_below_stall_tol():
    """A stall fraction between the relative decreases of the first two epochs
    (composed with |B| = 1: anchors at 0, 8, 16) leaves the sample alone at the
    anchor of step 8, where the objective still fell by more than that
    fraction, and doubles it at step 16, where it fell by less."""
    S, H0 = _problem()
    lr, seed, br = 0.02, 5, 8

    def schedule(t):
        return ("anchor", None) if t % 8 == 0 else ("sampled", 1)

    Hs, _, _ = _compose(S, H0, lr, schedule, seed, br, 16)
    f0, f8, f16 = (oracle.objective_explicit(S, Hs[t]) for t in (0, 8, 16))
    d1, d2 = (f0 - f8) / f0, (f8 - f16) / f8
    assert d1 > d2 > 0
    stall = float(np.sqrt(d1 * d2))
    out = oracle.fit_adaptgrow(S, H0, lr, 20, solver=oracle.SOLVER_BLOCK_SVRG, phi0=1 / 8,
                               block_rows=br, tol=0.0, stall_tol=stall, seed=seed)
    assert out["history"][0] == (16, 2)
    assert out["anchors"][:3] == [0, 8, 16]
