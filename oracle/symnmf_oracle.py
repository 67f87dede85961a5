"""Plain, slow, fp64 CPU oracle for the SymNMF clustering hot path.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the library. It shares no code with
the HIP path. Every function follows the pages in the pages' order and notation,
with numpy as its only helper (a matmul, an argsort, LAPACK's eigvalsh):

* P1 = "GPU-Accelerated Clustering for Financial Instruments at Scale"
  (sections "Factorization at scale", "Choosing the rank k", "Factorizing with
  SymNMF", "Why this solver", "The metric").
* P2 = "GPU-Accelerated SymNMF Clustering Scales to a Million Financial
  Instruments" (the same post; the displayed diagonal AdaGrad update and the
  AdaptGrow algorithm sketch).
* P3 = the paper-card page "GEM-KMeans: Memory-Efficient and Accurate
  Clustering on Massive Scale with GPU Optimization", second abstract (the
  SymNMF study: absolute Pearson correlation and TPDM inputs, trace identity,
  Block-SVRG AdaptGrow).

Where the pages leave a step open, the function says which reading it takes.
Pins (what each function is checked against, other than itself) live in
``tests/test_oracle_*.py``. Functions whose constants the pages do not fix and
that nothing outside this file can pin say "parity unpinned" below:

* ``tpdm`` constants (loss sign, F = R/(T+1), the 5% tail, 1/m scaling):
  parity unpinned for the constants; the structure is pinned by invariants.
* ``fit_adaptgrow`` stagnation rule and phi seeding, and the constants of the
  stopping test (``converged_test``: the 1e-3 stall fraction, the 0.05 floor
  of the objective scale): parity unpinned for the constants (the pages name
  ``stagnating()``, the seeding and convergence but define none of them). The
  schedule these rules drive (anchor steps, doublings, the switch to full
  batch, the stop step, resumption) is pinned by hand-composed runs.
* ``calm_windows`` (which windows calibrate the 3-sigma limit) and the
  warm start of ``rolling_fit``: readings of the pages, parity unpinned.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "standardize", "abs_corr", "abs_corr_rows", "tpdm_angles", "tpdm",
    "tpdm_rows", "splitmix64", "uniform24", "init_uniform", "init_scale_matched",
    "default_lr", "sh_product", "objective_explicit", "objective_trace", "gradient",
    "adagrad_step", "rmsprop_step", "converged_test", "fit_full", "sample_blocks", "svrg_sh_estimate",
    "gap_ratio", "initial_blocks", "fit_adaptgrow", "top_eigenvalues",
    "subspace_top_eigenvalues",
    "ari_drift", "calm_windows", "control_limit", "cross_block_means", "rolling_fit",
    "spherical_kmeans", "boundary_fraction",
    "labels", "ari", "ari_pairs", "SOLVER_AUTO", "SOLVER_FULL",
    "SOLVER_BLOCK_SVRG",
]

SOLVER_AUTO, SOLVER_FULL, SOLVER_BLOCK_SVRG = 0, 1, 2

# --------------------------------------------------------------------------
# Dependence matrices (P1 introduction: absolute Pearson correlation for
# broad co-movement, TPDM for joint behaviour in extreme observations; P3).
# --------------------------------------------------------------------------


def standardize(X):
    """Column-standardise a T x n returns window: z_ti = (x_ti - mu_i) / ||x_.i - mu_i||.

    Unit-norm centred columns make Z^T Z the Pearson correlation matrix with no
    ddof convention to choose. A constant column has no correlation; it raises.
    """
    X = np.asarray(X, dtype=np.float64)
    mu = X.mean(axis=0)
    C = X - mu
    nrm = np.sqrt((C * C).sum(axis=0))
    if np.any(nrm == 0):
        raise ValueError("constant column: correlation undefined")
    return C / nrm


def abs_corr(X):
    """S = |corr(X)|, n x n fp64 (P1 introduction: absolute Pearson correlation).

    The diagonal is kept as computed (1 up to rounding)."""
    Z = standardize(X)
    return np.abs(Z.T @ Z)


def abs_corr_rows(X, rows):
    """Rows ``rows`` of |corr(X)| without forming the n x n matrix."""
    Z = standardize(X)
    rows = np.asarray(rows)
    return np.abs(Z[:, rows].T @ Z)


def tpdm_angles(X, tail_frac=0.05):
    """The extreme-day angular components behind the TPDM.

    Reading (parity unpinned for the constants; P1 introduction and P3 name
    the TPDM from extreme value theory but print no recipe):
      losses L = -X;  R_ti = ordinal rank of L_ti within column i (1..T,
      ties to the earlier day);  F = R / (T + 1);  Frechet margins with
      alpha = 2:  x_ti = (-1 / ln F_ti)^(1/2);  radius r_t = ||x_t.||_2;
      the m = ceil(tail_frac * T - 1e-4) days of largest radius (ties to the
      earlier day; the slack keeps a tail fraction whose product with T is an
      integer up to rounding at that integer);  theta_t = x_t. / r_t.
    Returns (theta m x n, selected days in radius order, m).
    """
    L = -np.asarray(X, dtype=np.float64)
    T, n = L.shape
    order = np.argsort(L, axis=0, kind="stable")
    R = np.empty((T, n), dtype=np.int64)
    np.put_along_axis(R, order, np.repeat(np.arange(1, T + 1)[:, None], n, axis=1), axis=0)
    F = R / (T + 1.0)
    xt = np.sqrt(-1.0 / np.log(F))
    r = np.sqrt((xt * xt).sum(axis=1))
    m = int(math.ceil(tail_frac * T - 1e-4))
    m = max(1, min(T, m))
    days = np.argsort(-r, kind="stable")[:m]
    theta = xt[days] / r[days, None]
    return theta, days, m


def tpdm(X, tail_frac=0.05):
    """S_ij = (1/m) sum over the m extreme days of theta_ti * theta_tj (n x n fp64)."""
    theta, _, m = tpdm_angles(X, tail_frac)
    return theta.T @ theta / m


def tpdm_rows(X, rows, tail_frac=0.05):
    theta, _, m = tpdm_angles(X, tail_frac)
    rows = np.asarray(rows)
    return theta[:, rows].T @ theta / m


# --------------------------------------------------------------------------
# Counter-based generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable
# pseudorandom number generators", OOPSLA 2014), written from its published
# definition. Stream ``key``, counter c -> the (c+1)-th output of the
# SplitMix64 sequence whose state starts at ``key``.
# --------------------------------------------------------------------------

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
SAMPLER_KEY_XOR = 0x5851F42D4C957F2D


def splitmix64(key, counter):
    """Vectorised SplitMix64 output for state key + (counter + 1) * golden gamma."""
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (np.asarray(counter, dtype=np.uint64) + np.uint64(1)) * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def uniform24(key, counter):
    """Uniform on [0, 1): the top 24 bits of the SplitMix64 output times 2^-24."""
    return (splitmix64(key, counter) >> np.uint64(40)).astype(np.float64) * 2.0 ** -24


# --------------------------------------------------------------------------
# Initialisation (P1 "Factorizing with SymNMF": the same fixed-seed
# initialisation for every window, no warm start; P2 sketch: a scale-matched
# init).
# --------------------------------------------------------------------------


def init_uniform(n, k, scale, seed):
    """H0[i, c] = scale * u(seed, i*k + c)."""
    idx = np.arange(n * k, dtype=np.uint64)
    return (scale * uniform24(seed, idx)).reshape(n, k)


def init_scale_matched(S_mean, k):
    """Reading of the undefined scale-matched init: U(0, a) with
    a = 2 sqrt(mean(S)/k), so E[(H0 H0^T)_ij] = k (a/2)^2 = mean(S)."""
    return 2.0 * math.sqrt(S_mean / k)


def default_lr(S_mean, k):
    """Reading of the unspecified learning rate: eta = sqrt(mean(S)/k), the
    mean entry of the scale-matched H0."""
    return math.sqrt(S_mean / k)


# --------------------------------------------------------------------------
# Objective and gradient (P1 "Factorization at scale": the trace formulation
# avoids n x n intermediates; P2 sketch: g = 4 (H (H^T H) - S H)).
# --------------------------------------------------------------------------


def sh_product(S, H, rows=None):
    """P = S H and tr(H^T S H) = sum_i <H_i, P_i> (the product every full-batch
    step needs; P1 "Factorization at scale").

    With ``rows`` given, ``S`` holds only those rows of the n x n matrix and
    the result is those rows of S H and their terms of the trace."""
    H = np.asarray(H, dtype=np.float64)
    P = np.asarray(S, dtype=np.float64) @ H
    Hr = H if rows is None else H[np.asarray(rows)]
    return P, float((Hr * P).sum())


def objective_explicit(S, H, rows_per_slice=1024):
    """f(H) = ||S - H H^T||_F^2, the plain definition: the residual is formed
    entry by entry, a slice of rows at a time (so that n = 8192 needs no
    0.5 GB temporary), and its squares summed."""
    S = np.asarray(S, dtype=np.float64)
    H = np.asarray(H, dtype=np.float64)
    n = S.shape[0]
    f = 0.0
    for r0 in range(0, n, rows_per_slice):
        R = S[r0:r0 + rows_per_slice] - H[r0:r0 + rows_per_slice] @ H.T
        f += float((R * R).sum())
    return f


def objective_trace(S_fro2, H, P):
    """f = ||S||^2 - 2 tr(H^T S H) + ||H^T H||^2, with P = S H given."""
    K = H.T @ H
    return float(S_fro2 - 2.0 * (H * P).sum() + (K * K).sum())


def gradient(S, H):
    """grad f = 4 (H (H^T H) - S H) for symmetric S."""
    return 4.0 * (H @ (H.T @ H) - S @ H)


def adagrad_step(H, G, g, lr, eps=1e-8):
    """P2 displayed update, element-wise: G <- G + g*g, then
    H <- max(H - lr * g / (sqrt(G) + eps), 0). eps sits outside the root."""
    G = G + g * g
    H = np.maximum(H - lr * g / (np.sqrt(G) + eps), 0.0)
    return H, G


def rmsprop_step(H, G, g, lr, rho, eps=1e-8):
    """RMSprop (Tieleman and Hinton 2012), one of the AdaGrad-family solvers the
    P3 abstract names: the squared-gradient accumulator becomes an exponential
    moving average, G <- rho G + (1 - rho) g*g, with the same projected step
    H <- max(H - lr g / (sqrt(G) + eps), 0) as AdaGrad."""
    G = rho * G + (1.0 - rho) * (g * g)
    H = np.maximum(H - lr * g / (np.sqrt(G) + eps), 0.0)
    return H, G


def _step(H, G, g, lr, eps, rho):
    return adagrad_step(H, G, g, lr, eps) if not rho else rmsprop_step(H, G, g, lr, rho, eps)


# --------------------------------------------------------------------------
# Full-batch projected AdaGrad (P1 "Factorizing with SymNMF"; P2 sketch).
# --------------------------------------------------------------------------


def converged_test(f_prev, f, tol, steps, floor_abs):
    """The stopping test (config 2: relative objective change below tol).

    True when |f_prev - f| < tol * steps * max(|f_prev|, floor_abs): the
    average change per step over ``steps`` steps (1 in the full branch, the
    epoch length between two Block-SVRG anchors) relative to the objective.
    Reading: the relative change is ill-posed when the attainable objective is
    near zero (a TPDM has rank at most m, the number of extreme days, below
    k, and is factored almost exactly, while AdaGrad's f decays as a power
    law), so the denominator never falls below ``floor_abs`` =
    obj_floor * ||S||^2 (obj_floor 0.05: below the 7-10% of ||S||^2 that the
    |corr| fits keep at convergence, so their test is the plain relative one).
    """
    return abs(f_prev - f) < tol * steps * max(abs(f_prev), floor_abs)


def fit_full(S, H0, lr, max_iters, tol=0.0, eps=1e-8, G0=None, objective="trace", rho=0.0,
             obj_floor=0.05, snapshots=()):
    """Full-batch projected AdaGrad (RMSprop's accumulator when rho > 0).

    Iteration t: P = S H_t; f_t = f(H_t) (before the update); if t >= 1 and
    ``converged_test(f_{t-1}, f_t, tol, 1, obj_floor ||S||^2)``, stop and
    return H_t; otherwise take the AdaGrad step. At most ``max_iters`` steps.
    ``objective`` "explicit" evaluates f as ||S - H H^T||^2 directly, "trace"
    by the identity ||S||^2 - 2 tr(H^T P) + ||H^T H||^2.
    Returns dict(H, G, f (list of f_t), iters (steps taken), converged, H_at
    (a copy of H_t for every t in ``snapshots`` that the run reaches)).
    """
    S = np.asarray(S, dtype=np.float64)
    H = np.array(H0, dtype=np.float64)
    G = np.zeros_like(H) if G0 is None else np.array(G0, dtype=np.float64)
    s2 = float(np.einsum("ij,ij->", S, S))  # ||S||_F^2 without an n x n temporary
    fs = []
    converged = False
    H_at = {}
    t = 0
    while t < max_iters:
        if t in snapshots:
            H_at[t] = H.copy()
        P = S @ H
        f = objective_trace(s2, H, P) if objective == "trace" else objective_explicit(S, H)
        fs.append(f)
        if tol > 0 and t >= 1 and converged_test(fs[-2], f, tol, 1, obj_floor * s2):
            converged = True
            break
        g = 4.0 * (H @ (H.T @ H) - P)
        H, G = _step(H, G, g, lr, eps, rho)
        t += 1
    if t in snapshots:
        H_at[t] = H.copy()
    return dict(H=H, G=G, f=fs, iters=t, converged=converged, H_at=H_at)


# --------------------------------------------------------------------------
# Block-SVRG AdaptGrow (P1 "Factorizing with SymNMF" and "Why this solver";
# P2 sketch; P3 abstract).
# --------------------------------------------------------------------------


def sample_blocks(seed, t, nb, nsel):
    """|B| = nsel distinct row blocks out of nb for step t, ascending.

    Partial Fisher-Yates over [0, nb): for j < nsel, swap slot j with slot
    j + (r_j mod (nb - j)), r_j = SplitMix64(seed ^ SAMPLER_KEY_XOR,
    t * 2^32 + j)."""
    key = np.uint64((int(seed) ^ SAMPLER_KEY_XOR) & 0xFFFFFFFFFFFFFFFF)
    perm = list(range(nb))
    for j in range(nsel):
        r = int(splitmix64(key, np.uint64((t << 32) + j)))
        pick = j + r % (nb - j)
        perm[j], perm[pick] = perm[pick], perm[j]
    return sorted(perm[:nsel])


def svrg_sh_estimate(S, H, H_anchor, P_anchor, blocks, block_rows):
    """Reading of block_svrg_grad's S H estimate: SVRG over row blocks.

    C = sum over rows i of the sampled blocks of S[i, :]^T (H - H~)[i, :];
    P_est = P~ + (nb / |B|) C. Unbiased since each block is drawn with
    probability |B|/nb and S = S^T; H (H^T H) stays exact."""
    n = S.shape[0]
    nb = -(-n // block_rows)
    C = np.zeros_like(np.asarray(P_anchor, dtype=np.float64))
    for b in blocks:  # block by block over row slices (views of S), in list order
        r0, r1 = b * block_rows, min(n, (b + 1) * block_rows)
        C += S[r0:r1].T @ (H[r0:r1] - H_anchor[r0:r1])
    return P_anchor + (nb / len(blocks)) * C


def gap_ratio(eigvals, k, floor_rel=1e-6):
    """P1 "Why this solver": gamma_{k+1} = lambda_{k+1} / |lambda_{k+2}|,
    eigenvalues 1-based in descending |lambda| with the sign kept. Reading: if
    |lambda_{k+2}| <= floor_rel |lambda_1| the denominator is floor_rel |lambda_1|."""
    ev = np.asarray(eigvals, dtype=np.float64)
    lam1 = abs(ev[0])
    den = abs(ev[k + 1])
    if den <= floor_rel * lam1:
        den = floor_rel * lam1
    return float(ev[k] / den)


def initial_blocks(gamma, nb, threshold=5.0):
    """Reading of the phi seeding: gamma >= threshold -> all nb blocks (full
    gradient); else |B|0 = 2^floor(log2(max(1, (gamma/threshold) nb)))."""
    if gamma >= threshold:
        return nb
    x = max(1.0, gamma / threshold * nb)
    return min(nb, 1 << int(math.floor(math.log2(x))))


def fit_adaptgrow(S, H0, lr, max_iters, *, solver=SOLVER_AUTO, eigvals=None, k=None,
                  phi0=0.0, block_rows=1024, gap_threshold=5.0, tol=1e-6,
                  stall_tol=1e-3, obj_floor=0.05, eps=1e-8, seed=0, rho=0.0,
                  objective="trace", G0=None, state=None, snapshots=()):
    """AdaptGrow: full-batch AdaGrad or Block-SVRG with sample growth.

    Branch choice: FULL -> full; otherwise |B|0 from phi0 > 0
    (ceil(phi0 nb) clamped to [1, nb]) or from gamma_{k+1} (``initial_blocks``);
    |B|0 = nb means full.

    Sampled branch (reading; the stall and stop constants are parity
    unpinned): with E = ceil(nb/|B|), a step is an anchor when no anchor exists
    yet or E steps have passed since the last one. An anchor computes P = S H
    and f exactly, then, against the previous anchor (E_j steps earlier):
      * stop: ``converged_test(f~prev, f, tol, E_j, obj_floor ||S||^2)`` ends
        the run and returns this H (the anchor's update is not taken);
      * stall: (f~prev - f) < stall_tol f~prev doubles |B| (capped at nb; at
        nb the run continues as full batch, keeping G);
    and becomes H~ = H, P~ = P; the anchor's own step uses the exact gradient.
    Other steps draw ``sample_blocks(seed, t, nb, |B|)`` with the absolute step
    index t and use ``svrg_sh_estimate``; their f is not computed (NaN in the
    trace). The full branch tests convergence as ``fit_full`` does, against the
    previous step's exact f (an anchor's f counts).

    Resumption: ``state`` (from a previous call's result) restores the step
    index, |B|, the anchor (H~, P~, its step and f) and the previous exact f,
    and ``G0`` the accumulator, so that the two calls take the same steps as one
    uninterrupted call. ``max_iters`` counts the steps of this call.
    Returns dict(H, G, f (this call's f_t), iters (steps taken in this call),
    converged, history [(t, |B|) at each doubling, absolute t], gamma,
    start_branch, final_branch, nsel, anchors (absolute steps), state, H_at (a
    copy of H_t for every absolute t in ``snapshots`` that the run reaches)).
    """
    S = np.asarray(S, dtype=np.float64)
    H = np.array(H0, dtype=np.float64)
    n, kk = H.shape
    if k is None:
        k = kk
    G = np.zeros_like(H) if G0 is None else np.array(G0, dtype=np.float64)
    s2 = float(np.einsum("ij,ij->", S, S))  # ||S||_F^2 without an n x n temporary
    floor_abs = obj_floor * s2
    nb = -(-n // block_rows)
    gamma = None
    if state is not None:
        t = int(state["t"])
        nsel = int(state["nsel"])
        anchor_t = state["anchor_t"]
        f_anchor = state["f_anchor"]
        H_a = None if state["H_a"] is None else np.array(state["H_a"], dtype=np.float64)
        P_a = None if state["P_a"] is None else np.array(state["P_a"], dtype=np.float64)
        prev_exact = state["f_prev"]
    else:
        t = 0
        if solver == SOLVER_FULL:
            nsel = nb
        elif phi0 > 0:
            nsel = min(nb, max(1, int(math.ceil(phi0 * nb - 1e-12))))
        else:
            if eigvals is None:
                raise ValueError("AdaptGrow needs eigenvalues or phi0")
            gamma = gap_ratio(eigvals, k)
            nsel = initial_blocks(gamma, nb, gap_threshold)
        anchor_t = f_anchor = H_a = P_a = prev_exact = None
    full = nsel >= nb
    start_branch = "full" if full else "sampled"

    def f_of(P):
        if objective == "trace":
            K = H.T @ H
            return float(s2 - 2.0 * (H * P).sum() + (K * K).sum())
        return objective_explicit(S, H)

    fs = []
    history = []
    anchors = []
    H_at = {}
    converged = False
    t0 = t
    while t < t0 + max_iters:
        if t in snapshots:
            H_at[t] = H.copy()
        E = -(-nb // nsel)
        if full:
            P = S @ H
            f = f_of(P)
            fs.append(f)
            if tol > 0 and prev_exact is not None and converged_test(prev_exact, f, tol, 1, floor_abs):
                converged = True
                break
            prev_exact = f
        elif anchor_t is None or t - anchor_t >= E:
            P = S @ H
            f = f_of(P)
            fs.append(f)
            if anchor_t is not None:
                if tol > 0 and converged_test(f_anchor, f, tol, t - anchor_t, floor_abs):
                    converged = True
                    break
                if (f_anchor - f) < stall_tol * f_anchor:
                    nsel = min(2 * nsel, nb)
                    history.append((t, nsel))
                    full = nsel >= nb
            anchors.append(t)
            anchor_t, f_anchor = t, f
            H_a, P_a = H.copy(), P.copy()
            prev_exact = f
        else:
            blocks = sample_blocks(seed, t, nb, nsel)
            P = svrg_sh_estimate(S, H, H_a, P_a, blocks, block_rows)
            fs.append(float("nan"))
            prev_exact = None
        g = 4.0 * (H @ (H.T @ H) - P)
        H, G = _step(H, G, g, lr, eps, rho)
        t += 1
    if t in snapshots:
        H_at[t] = H.copy()
    out_state = dict(t=t, nsel=nsel, anchor_t=anchor_t, f_anchor=f_anchor, H_a=H_a, P_a=P_a,
                     f_prev=prev_exact)
    return dict(H=H, G=G, f=fs, iters=t - t0, converged=converged, history=history,
                gamma=gamma, start_branch=start_branch,
                final_branch="full" if full else "sampled", nsel=nsel, anchors=anchors,
                state=out_state, H_at=H_at)


# --------------------------------------------------------------------------
# Spectral probe (P1 "Choosing the rank k" and "Why this solver"): the
# leading eigenvalues by magnitude, sign kept.
# --------------------------------------------------------------------------


def top_eigenvalues(S, p):
    """The p eigenvalues of symmetric S of largest |lambda|, in descending
    |lambda| (LAPACK eigvalsh is the plain definition here)."""
    w = np.linalg.eigvalsh(np.asarray(S, dtype=np.float64))
    order = np.argsort(-np.abs(w), kind="stable")
    return w[order[:p]]


def subspace_top_eigenvalues(matmat, n, m, iters, seed=0):
    """Eigenvalues of largest |lambda| of a symmetric n x n operator known only
    through its products with n x m blocks (``matmat(V) -> S V``), for sizes
    where S cannot be factorised whole: fp64 subspace iteration, V <- qr(S V)
    ``iters`` times from a seeded Gaussian block, then Rayleigh-Ritz on the
    last basis (P1 "Choosing the rank k": the leading eigenvalues of S).

    Returns (theta, resid): the m Ritz values in descending |theta| with the
    sign kept, and resid_i = ||S v_i - theta_i v_i||_2 for the unit Ritz
    vector v_i (an eigenvalue lies within resid_i of theta_i)."""
    rng = np.random.default_rng(seed)
    V = np.linalg.qr(rng.standard_normal((n, m)))[0]
    for _ in range(iters):
        V = np.linalg.qr(matmat(V))[0]
    Y = matmat(V)
    T = V.T @ Y
    T = 0.5 * (T + T.T)
    theta, U = np.linalg.eigh(T)
    order = np.argsort(-np.abs(theta), kind="stable")
    theta, U = theta[order], U[:, order]
    resid = np.linalg.norm(Y @ U - (V @ U) * theta, axis=0)
    return theta, resid


# --------------------------------------------------------------------------
# Labels and the adjusted Rand index (P1 "Factorizing with SymNMF": argmax of
# a row of H is the hard label; "The metric": ARI).
# --------------------------------------------------------------------------


def labels(H):
    """Row argmax of H, lowest column index on ties (an all-zero row -> 0)."""
    H = np.asarray(H)
    return np.argmax(H, axis=1).astype(np.int32)


def ari(a, b):
    """Adjusted Rand index (Hubert and Arabie 1985) from the contingency table."""
    a = np.asarray(a)
    b = np.asarray(b)
    n = a.size
    _, ai = np.unique(a, return_inverse=True)
    _, bi = np.unique(b, return_inverse=True)
    M = np.zeros((ai.max() + 1, bi.max() + 1), dtype=np.float64)
    np.add.at(M, (ai, bi), 1.0)

    def c2(x):
        return x * (x - 1) / 2.0

    sij = c2(M).sum()
    sa = c2(M.sum(axis=1)).sum()
    sb = c2(M.sum(axis=0)).sum()
    tot = c2(float(n))
    expected = sa * sb / tot if tot > 0 else 0.0
    mx = 0.5 * (sa + sb)
    if mx == expected:
        return 1.0
    return float((sij - expected) / (mx - expected))


def ari_pairs(a, b):
    """The same index by brute force over all pairs (for pins on tiny n)."""
    a = list(a)
    b = list(b)
    n = len(a)
    n11 = n10 = n01 = n00 = 0
    for i in range(n):
        for j in range(i + 1, n):
            sa = a[i] == a[j]
            sb = b[i] == b[j]
            if sa and sb:
                n11 += 1
            elif sa:
                n10 += 1
            elif sb:
                n01 += 1
            else:
                n00 += 1
    tot = n11 + n10 + n01 + n00
    if tot == 0:
        return 1.0
    expected = (n11 + n10) * (n11 + n01) / tot
    mx = 0.5 * ((n11 + n10) + (n11 + n01))
    if mx == expected:
        return 1.0
    return (n11 - expected) / (mx - expected)


# --------------------------------------------------------------------------
# Re-clustering through time (P1 "Tracking stability through time with the
# Rand index" and the tail/body discussion after it).
# --------------------------------------------------------------------------


def ari_drift(label_seq, delta):
    """ARI(t - delta, t) of window t's hard labels against window t - delta's;
    NaN for t < delta (no earlier window that far back)."""
    W = len(label_seq)
    out = np.full(W, np.nan)
    for t in range(delta, W):
        out[t] = ari(label_seq[t - delta], label_seq[t])
    return out


def calm_windows(W, T, delta, switch_day, stress_first, stress_last):
    """Windows that calibrate the control limit: the pages calibrate on the
    calm windows before the break. Reading: window t (days t .. t+T-1) is calm
    when ARI(t - delta, t) exists, fewer than half of its days come after the
    membership switch (so no switched label can have flipped yet) and it holds
    no stressed day. Parity unpinned (the pages give no rule)."""
    calm = np.zeros(W, dtype=bool)
    for t in range(W):
        after = max(0, t + T - switch_day)
        stressed = not (t + T - 1 < stress_first or t > stress_last)
        calm[t] = t >= delta and 2 * after < T and not stressed
    return calm


def control_limit(values, calm):
    """The self-calibrating 3-sigma limit: mean minus three sample standard
    deviations of the calm values; a value below it is flagged."""
    v = np.asarray(values, dtype=np.float64)
    c = v[np.asarray(calm, dtype=bool)]
    mu = float(c.mean())
    sd = float(c.std(ddof=1))
    limit = mu - 3.0 * sd
    flags = np.zeros(v.size, dtype=bool)
    ok = ~np.isnan(v)
    flags[ok] = v[ok] < limit
    return limit, mu, sd, flags


def cross_block_means(S, labels_, groups):
    """m x m means of S over the blocks of the listed planted groups: entry
    (a, b) is the mean of S_ij over i in group a and j in group b. The pages
    track the off-diagonal (cross-sector) entries to see a co-crash."""
    S = np.asarray(S, dtype=np.float64)
    lab = np.asarray(labels_)
    m = len(groups)
    B = np.zeros((m, m))
    for a in range(m):
        ia = np.flatnonzero(lab == groups[a])
        for b in range(m):
            ib = np.flatnonzero(lab == groups[b])
            B[a, b] = S[np.ix_(ia, ib)].mean()
    return B


def rolling_fit(X_stream, k, T, windows, kind="abscorr", iters=100, seed=0, warm_start=True,
                tail=0.05, S_windows=None, first_max_iters=None, first_tol=1e-6):
    """Fit every window t = 0 .. windows-1 (days t .. t+T-1) with ``iters``
    full-batch AdaGrad steps. The first window (every window without
    warm_start) starts from the scale-matched seeded init; with warm_start a
    window starts from the previous window's H with a fresh accumulator G
    (a reading: the pages fit each window independently, the rolling
    workload asks for a warm start; both are offered). lr is the default
    reading per window. ``S_windows`` (optional) supplies each window's S
    instead of building it. With warm_start and ``first_max_iters`` the first
    window runs to convergence (relative change below ``first_tol``, at most
    ``first_max_iters`` steps), the later ones ``iters`` steps. Returns
    per-window H, labels and objective traces."""
    X_stream = np.asarray(X_stream)
    Hs, labs, fs = [], [], []
    H = None
    for t in range(windows):
        if S_windows is not None:
            S = np.asarray(S_windows[t], dtype=np.float64)
        else:
            Xw = X_stream[t:t + T].astype(np.float32)
            S = abs_corr(Xw) if kind == "abscorr" else tpdm(Xw, tail)
            S = S.astype(np.float32).astype(np.float64)
        m = S.mean()
        if H is None or not warm_start:
            H0 = init_uniform(S.shape[0], k, init_scale_matched(m, k), seed)
        else:
            H0 = H
        if warm_start and H is None and first_max_iters is not None:
            out = fit_full(S, H0, default_lr(m, k), first_max_iters, tol=first_tol)
        else:
            out = fit_full(S, H0, default_lr(m, k), iters, tol=0.0)
        H = out["H"]
        Hs.append(H)
        labs.append(labels(H))
        fs.append(np.asarray(out["f"]))
    return dict(H=Hs, labels=labs, f=fs)


# --------------------------------------------------------------------------
# Spherical k-means, the hard-clustering baseline (P1 "Spherical k-means for
# direct hard clustering", "Between spherical k-means and SymNMF").
# --------------------------------------------------------------------------


def spherical_kmeans(S, k, max_iters=100, seed=0):
    """Spherical k-means (Dhillon and Modha 2001) on the rows of S scaled to
    unit length, similarity = cosine. Initial centroids: the rows drawn by
    ``sample_blocks(seed, 0, n, k)`` (ascending). Each iteration assigns every
    row to its most similar centroid (lowest index on ties) and stops when no
    label changed; otherwise every centroid becomes the normalised sum of its
    rows (an empty cluster keeps its centroid). ``iters`` counts the centroid
    updates; ``objective`` is the summed similarity of the final assignment."""
    S = np.asarray(S, dtype=np.float64)
    n = S.shape[0]
    r = np.sqrt((S * S).sum(axis=1))
    X = np.zeros_like(S)
    nz = r > 0
    X[nz] = S[nz] / r[nz, None]
    C = X[sample_blocks(seed, 0, n, k)].copy()
    labels_ = np.full(n, k)
    updates = 0
    converged = False
    while True:
        sims = X @ C.T
        new = np.argmax(sims, axis=1)
        obj = float(sims[np.arange(n), new].sum())
        changed = int((new != labels_).sum())
        labels_ = new
        if changed == 0:
            converged = True
            break
        if updates >= max_iters:
            break
        for j in range(k):
            s_j = X[labels_ == j].sum(axis=0)
            norm = np.linalg.norm(s_j)
            if norm > 0:
                C[j] = s_j / norm
        updates += 1
    return dict(labels=labels_.astype(np.int32), C=C, iters=updates, converged=converged,
                objective=obj)


def boundary_fraction(H, ratio=0.5):
    """Share of rows whose second-largest loading is at least ``ratio`` times
    their largest (rows split across two clusters; an all-zero row is not
    counted). Reading: the pages count "boundary" instruments whose soft
    loadings stay split but give no rule; parity unpinned."""
    H = np.asarray(H, dtype=np.float64)
    top2 = np.sort(H, axis=1)[:, -2:]
    return float(np.mean((top2[:, 1] > 0) & (top2[:, 0] >= ratio * top2[:, 1])))
