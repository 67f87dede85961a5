"""GPU parity of the upper-triangle S.H pass (symnmf_sh_sym: each 32 x 32
block on or above the diagonal read once, both products on the bf16 matrix
cores with exactly split operands) against the oracle's fp64 S H, element by
element, and its trace against the oracle's tr(H^T S H)."""
import numpy as np
import pytest

import oracle
from symmetric_nmf_clustering_amd import synth
from tests.gpu_util import S_to_dev, require_gpu, to_dev

pytestmark = pytest.mark.gpu

# Bound on |P - S H| relative to sum_j |S_ij H_jc| (the size of the terms):
# a dropped split term (x1 y2 is 2^-8 of x y), a block counted twice or
# missed, or a transposed block read as itself shows as 1e-3 or more. The
# bound allows fp32 accumulation: a column-side accumulator takes 4 or 6 matrix-core
# steps per 32-row panel over up to 128 panels of a chunk, then the strip and
# chunk partials are added in the fold.
REL = 2e-5


@pytest.fixture(scope="module")
def torch():
    return require_gpu()


@pytest.fixture(scope="module")
def api(torch):
    from symmetric_nmf_clustering_amd import api as a
    return a


def _check(P, tr, S64, H64, rel=REL):
    ref, tr_ref = oracle.sh_product(S64, H64)
    scale = np.abs(S64) @ np.abs(H64)
    err = np.abs(np.asarray(P, np.float64) - ref)
    worst = float((err / np.maximum(scale, 1e-30)).max())
    assert (err <= rel * scale + 1e-37).all(), worst
    assert abs(tr - tr_ref) <= rel * float((np.abs(H64) * scale).sum()) + 1e-30
    return worst


# n: one block, ragged blocks, one strip (512) and its edges, several strips,
# several 2048-row chunks (2049, 4097, 5000, 9000) with a ragged tail; k: one and two
# 16-column tiles, full and partial. A last tile with at most 8 factors runs as
# a half tile (two parts of H per operand: k = 1, 8, 17, 20, 24); one with more
# runs as a full tile with zero factors (k = 9, 13, 28, 31) or none (k = 16, 32).
# n = 2048 and 6144 end exactly on a chunk edge, 6145 one row past it.
SYM_CASES = [(1, 1), (5, 8), (32, 16), (33, 24), (100, 17), (511, 24), (512, 32), (513, 24),
             (1000, 8), (1537, 24), (4097, 24), (5000, 32), (9000, 24), (2048, 1), (3001, 20),
             (777, 13), (2050, 28), (2048, 24), (6144, 31), (6145, 9)]


@pytest.mark.parametrize("n,k", SYM_CASES)
def test_sh_sym_matches_oracle(torch, api, n, k):
    S = synth.random_symmetric_nonneg(n, seed=n + 11)
    H = synth.random_factor(n, k, seed=k + 3, scale=0.5)
    P, tr = api.sh_sym(S_to_dev(S, torch), to_dev(H, torch))
    _check(P.cpu().numpy(), tr, S.astype(np.float64), H.astype(np.float64))


def _upper_mirror(S, blk=32):
    """The matrix the pass reads: blocks on or above the block diagonal as
    stored, blocks below it replaced by the transposes of their mirrors."""
    n = S.shape[0]
    b = np.arange(n) // blk
    above = b[:, None] <= b[None, :]
    return np.where(above, S, S.T)


def test_sh_sym_reads_only_the_upper_blocks(torch, api):
    """Blocks strictly below the block diagonal hold NaN and padding columns
    (lds > n) hold NaN: neither may reach P, which then equals the product with
    the block-upper mirror of S (diagonal blocks used as stored, so an
    asymmetric diagonal block is read in full)."""
    n, k, lds = 1003, 24, 1008
    rng = np.random.default_rng(4)
    S = rng.random((n, n)).astype(np.float32)      # not symmetric
    b = np.arange(n) // 32
    Sn = np.where(b[:, None] > b[None, :], np.float32(np.nan), S)
    buf = torch.full((n, lds), float("nan"), dtype=torch.float32, device="cuda")
    buf[:, :n] = torch.from_numpy(Sn).cuda()
    H = synth.random_factor(n, k, seed=5)
    P, tr = api.sh_sym(buf[:, :n], to_dev(H, torch))
    P = P.cpu().numpy()
    assert np.isfinite(P).all() and np.isfinite(tr)
    _check(P, tr, _upper_mirror(S).astype(np.float64), H.astype(np.float64))


def test_sh_sym_agrees_with_full_pass(torch, api):
    """On a symmetric S the two passes compute the same product (different
    summation orders and arithmetic): within the combined fp32 rounding."""
    n, k = 6000, 24
    S = synth.random_symmetric_nonneg(n, seed=21)
    H = synth.random_factor(n, k, seed=22, scale=0.2)
    Sd, Hd = S_to_dev(S, torch), to_dev(H, torch)
    P1, t1 = api.sh(Sd, Hd)
    P2, t2 = api.sh_sym(Sd, Hd)
    scale = np.abs(S.astype(np.float64)) @ H.astype(np.float64)
    d = np.abs(P1.cpu().numpy().astype(np.float64) - P2.cpu().numpy())
    assert (d <= 2 * REL * scale).all(), float((d / scale).max())
    assert abs(t1 - t2) <= 2 * REL * abs(t1)


def test_sh_sym_wide_exponents(torch, api):
    """Entries over 2^-40 .. 2^40 with random signs: the split keeps every
    fp32 bit of both operands, whatever their magnitude."""
    n, k = 700, 16
    rng = np.random.default_rng(8)
    A = (rng.random((n, n)) + 0.5) * np.exp2(rng.integers(-40, 41, (n, n)))
    A = np.where(rng.random((n, n)) < 0.5, -A, A)
    S = (np.triu(A) + np.triu(A, 1).T).astype(np.float32)
    H = (rng.standard_normal((n, k)) * np.exp2(rng.integers(-20, 21, (n, k)))).astype(np.float32)
    P, tr = api.sh_sym(S_to_dev(S, torch), to_dev(H, torch))
    ref, _ = oracle.sh_product(S.astype(np.float64), H.astype(np.float64))
    scale = np.abs(S.astype(np.float64)) @ np.abs(H.astype(np.float64))
    err = np.abs(P.cpu().numpy().astype(np.float64) - ref)
    assert (err <= REL * scale).all(), float((err / scale).max())


def test_sh_sym_deterministic(torch, api):
    n, k = 5000, 24
    Sd = S_to_dev(synth.random_symmetric_nonneg(n, seed=3), torch)
    Hd = to_dev(synth.random_factor(n, k, seed=3), torch)
    a, ta = api.sh_sym(Sd, Hd)
    b, tb = api.sh_sym(Sd, Hd)
    np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
    assert ta == tb


def test_sh_sym_rejects_wide_factor(torch, api):
    n = 64
    Sd = S_to_dev(synth.random_symmetric_nonneg(n, seed=1), torch)
    with pytest.raises(ValueError):
        api.sh_sym(Sd, to_dev(np.zeros((n, 33)), torch))


# ---- the fit with the upper-triangle pass (sh_pass='upper') -----------------

def _traj_rel(fg, fr, s2):
    fg, fr = np.asarray(fg, np.float64), np.asarray(fr, np.float64)
    return np.abs(fg - fr) / np.maximum(np.abs(fr), 1e-12 * s2)


def _labels_agree(Hg, Hr):
    from sklearn.metrics import adjusted_rand_score
    return adjusted_rand_score(np.asarray(Hg).argmax(axis=1), np.asarray(Hr).argmax(axis=1))


def test_fit_upper_c1_trajectory(torch, api):
    """n=1024, k=8, H0 ~ U(0, 0.1), lr 0.05, 200 full-batch steps, every S H
    from the upper triangle: the oracle's fp64 trajectory to 1e-3 of ||S||^2."""
    w = synth.workload("blocks_n1024_k8")
    S = oracle.abs_corr(w.X).astype(np.float32)
    res = api.fit(S_to_dev(S, torch), w.k, solver="full", init="uniform", init_scale=0.1, seed=0,
                  lr=0.05, max_iters=200, tol_rel=0.0, sh_pass="upper")
    ref = oracle.fit_full(S, oracle.init_uniform(w.n, w.k, 0.1, 0), 0.05, 200, tol=0.0)
    s2 = float((S.astype(np.float64) ** 2).sum())
    assert res.report["iterations"] == 200
    assert _traj_rel(res.f_trace, ref["f"], s2).max() <= 1e-3
    assert _labels_agree(res.H.cpu().numpy(), ref["H"]) >= 0.99


def test_fit_upper_block_svrg_c3(torch, api):
    """n=8192, k=24 TPDM, Block-SVRG from 1 of 8 blocks: the anchors' exact
    products and the full-batch tail from the upper triangle, the sampled
    steps from row panels; same anchors, doublings and trajectory as the
    oracle's AdaptGrow."""
    w = synth.workload("tstress_n8192_k24")
    S = oracle.tpdm(w.X, 0.05).astype(np.float32)
    S64 = S.astype(np.float64)
    iters = 240
    res = api.fit(S_to_dev(S, torch), w.k, solver="block_svrg", phi0=1.0 / 8, block_rows=1024,
                  max_iters=iters, tol_rel=1e-6, seed=1, sh_pass="upper")
    m = S64.mean()
    H0 = oracle.init_uniform(w.n, w.k, oracle.init_scale_matched(m, w.k), 1)
    ref = oracle.fit_adaptgrow(S64, H0, oracle.default_lr(m, w.k), iters,
                               solver=oracle.SOLVER_BLOCK_SVRG, phi0=1.0 / 8, block_rows=1024,
                               tol=1e-6, seed=1)
    rep = res.report
    assert rep["iterations"] == ref["iters"]
    assert rep["doublings"] == len(ref["history"])
    fg, fr = np.asarray(res.f_trace), np.asarray(ref["f"])
    assert np.array_equal(np.isnan(fg), np.isnan(fr))
    ex = ~np.isnan(fr)
    assert _traj_rel(fg[ex], fr[ex], float((S64 ** 2).sum())).max() <= 1e-3
    assert _labels_agree(res.H.cpu().numpy(), ref["H"]) >= 0.99


def test_fit_upper_agrees_with_rows_and_is_deterministic(torch, api):
    """The two products differ only in rounding, which the iteration carries
    along: over 300 full-batch steps the trajectories stay within the bound both
    keep to the oracle's (1e-3) and the labels agree; two upper runs are
    identical."""
    w = synth.workload("blocks_n1024_k8")
    S = oracle.abs_corr(w.X).astype(np.float32)
    Sd = S_to_dev(S, torch)
    kw = dict(solver="full", init="uniform", init_scale=0.1, seed=2, lr=0.05, max_iters=300,
              tol_rel=0.0)
    rows = api.fit(Sd, w.k, **kw)
    up1 = api.fit(Sd, w.k, sh_pass="upper", **kw)
    up2 = api.fit(Sd, w.k, sh_pass="upper", **kw)
    assert torch.equal(up1.H, up2.H)
    s2 = float((S.astype(np.float64) ** 2).sum())
    assert _traj_rel(up1.f_trace, rows.f_trace, s2).max() <= 1e-3
    assert _labels_agree(up1.H.cpu().numpy(), rows.H.cpu().numpy()) >= 0.99
    with pytest.raises(Exception):
        api.fit(Sd, 33, solver="full", max_iters=1, sh_pass="upper")   # k > 32


@pytest.mark.parametrize("k", [5, 17])
def test_fit_upper_odd_width(torch, api, k):
    """k not a multiple of 4 (the partial products' row pitch is rounded up to
    4): 60 full-batch steps with the upper-triangle product against the
    oracle's trajectory on a ragged n."""
    n = 1003
    S = synth.random_symmetric_nonneg(n, seed=k).astype(np.float32) / n
    res = api.fit(S_to_dev(S, torch), k, solver="full", init="uniform", init_scale=0.1, seed=k,
                  lr=0.02, max_iters=60, tol_rel=0.0, sh_pass="upper")
    ref = oracle.fit_full(S.astype(np.float64), oracle.init_uniform(n, k, 0.1, k), 0.02, 60, tol=0.0)
    s2 = float((S.astype(np.float64) ** 2).sum())
    assert _traj_rel(res.f_trace, ref["f"], s2).max() <= 1e-3
    assert np.abs(res.H.cpu().numpy() - ref["H"]).max() <= 1e-3 * np.abs(ref["H"]).max()
