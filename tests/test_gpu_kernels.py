"""GPU parity of the single kernels against the oracle: labels, the S.H pass,
the |corr| and TPDM builds (through the C ABI via the binding)."""
import math
import os

import numpy as np
import pytest

import oracle
from symmetric_nmf_clustering_amd import synth
from tests.gpu_util import S_to_dev, require_gpu, s_close, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return require_gpu()


@pytest.fixture(scope="module")
def api(torch):
    from symmetric_nmf_clustering_amd import api as a
    return a


# ---- labels -------------------------------------------------------------------
def test_labels_hand_cases(torch, api):
    H = np.array([[0.0, 0.0, 0.0], [0.2, 0.5, 0.5], [0.7, 0.1, 0.7], [0.1, 0.2, 0.3]], np.float32)
    got = api.labels(to_dev(H, torch)).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.labels(H))
    np.testing.assert_array_equal(got, [0, 1, 0, 2])


@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (1000, 24), (70001, 24), (513, 64)])
def test_labels_random_bitexact(torch, api, n, k):
    rng = np.random.default_rng(n + k)
    H = rng.random((n, k)).astype(np.float32)
    H[rng.random(n) < 0.05] = 0.0                # all-zero rows
    H[:, 3 % k] = np.where(rng.random(n) < 0.1, H.max(1), H[:, 3 % k])  # ties
    got = api.labels(to_dev(H, torch)).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.labels(H))


def test_labels_empty(torch, api):
    out = api.labels(torch.empty((0, 4), dtype=torch.float32, device="cuda"))
    assert out.numel() == 0


# ---- S.H pass -----------------------------------------------------------------
# every MFMA-tile / vector-ALU split of the width (4 or 8 vector columns, a
# padded tile for remainders above 8), ragged n, one and two column groups
SH_CASES = [(1, 1), (5, 2), (300, 4), (301, 12), (333, 14), (64, 16), (257, 8), (520, 20),
            (1000, 24), (600, 30), (1000, 33), (777, 40), (2000, 48), (1023, 56), (900, 64),
            (1100, 80), (900, 100), (900, 112), (700, 128), (4099, 24), (8192, 24),
            (5, 80), (17, 128), (63, 52)]


@pytest.mark.parametrize("n,k", SH_CASES)
def test_sh_matches_oracle(torch, api, n, k):
    S = synth.random_symmetric_nonneg(n, seed=n)
    H = synth.random_factor(n, k, seed=k, scale=0.5)
    P, tr = api.sh(S_to_dev(S, torch), to_dev(H, torch))
    P = P.cpu().numpy().astype(np.float64)
    Pr, trr = oracle.sh_product(S.astype(np.float64), H.astype(np.float64))
    # every term is >= 0: no cancellation, so a per-element relative bound
    rel = np.abs(P - Pr) / np.maximum(np.abs(Pr), 1e-30)
    assert rel.max() <= 1e-4, rel.max()
    assert abs(tr - trr) <= 1e-5 * abs(trr)


# Widths of three or more MFMA tiles stream S through a per-wave LDS ring when
# H is 16-byte aligned; an H that is not takes the register panel kernel. Both
# use the same lanes, operands and accumulation order, so they agree bit for
# bit (n ragged, vector-ALU columns, a last tile wider than the width).
@pytest.mark.parametrize("n,k", [(777, 52), (1100, 80), (900, 72), (901, 76), (700, 128),
                                 (4099, 56), (1000, 120), (5, 80), (17, 128)])
def test_sh_ring_matches_panel_bitwise(torch, api, n, k):
    S = synth.random_symmetric_nonneg(n, seed=n + 1)
    H = synth.random_factor(n, k, seed=k + 1, scale=0.5)
    Sd = S_to_dev(S, torch)
    Ha = to_dev(H, torch)
    buf = torch.empty(n * k + 4, dtype=torch.float32, device="cuda")
    Hm = buf[1:1 + n * k].view(n, k)
    Hm.copy_(Ha)
    assert Ha.data_ptr() % 16 == 0 and Hm.data_ptr() % 16 == 4
    Pa, tra = api.sh(Sd, Ha)
    Pm, trm = api.sh(Sd, Hm)
    assert torch.equal(Pa, Pm)
    assert tra == trm


def test_sh_signed_inputs(torch, api):
    # signed H and S (the probe's basis is signed): bound relative to |S||H|
    n, k = 1500, 80
    rng = np.random.default_rng(3)
    A = rng.standard_normal((n, n))
    S = ((A + A.T) / 2).astype(np.float32)
    H = rng.standard_normal((n, k)).astype(np.float32)
    P, _ = api.sh(S_to_dev(S, torch), to_dev(H, torch))
    Pr, _ = oracle.sh_product(S, H)
    scale = np.abs(S.astype(np.float64)) @ np.abs(H.astype(np.float64))
    assert (np.abs(P.cpu().numpy() - Pr) / scale).max() <= 1e-5


def test_sh_ignores_padding_garbage(torch, api):
    # columns beyond n in each padded row must not leak into the product
    n, k = 1001, 24
    S = synth.random_symmetric_nonneg(n, seed=5)
    Sd = api.alloc_S(n)
    base = Sd.as_strided((n, Sd.stride(0)), (Sd.stride(0), 1))
    base.fill_(float("nan"))
    Sd.copy_(torch.from_numpy(S))
    H = synth.random_factor(n, k, seed=1)
    P, tr = api.sh(Sd, to_dev(H, torch))
    assert torch.isfinite(P).all().item() and math.isfinite(tr)
    Pr, _ = oracle.sh_product(S, H)
    assert (np.abs(P.cpu().numpy() - Pr) / Pr).max() <= 1e-4


# ---- |corr| build ---------------------------------------------------------------
@pytest.mark.parametrize("n,T,seed", [(1024, 256, 0), (1000, 37, 1), (130, 5, 2), (1, 2, 3),
                                      (300, 252, 4)])
def test_build_abscorr(torch, api, n, T, seed):
    if n == 1:
        X = np.array([[0.5], [-1.0]], np.float32)
    else:
        X = synth.gaussian_blocks(n=n - n % 2, k=2, T=T, seed=seed).X
        if X.shape[1] != n:
            X = np.concatenate([X, np.random.default_rng(seed).standard_normal((T, 1))], 1).astype(np.float32)
    S, fro = api.build_S(to_dev(X, torch), "abscorr")
    Sg = S.cpu().numpy()
    ref = oracle.abs_corr(X)
    ok, worst = s_close(Sg, ref)
    assert ok, worst
    assert np.array_equal(Sg, Sg.T)                       # bitwise symmetric
    assert abs(fro - (ref * ref).sum()) <= 1e-5 * (ref * ref).sum()


def test_build_abscorr_workload_c1(torch, api):
    w = synth.workload("blocks_n1024_k8")
    S, _ = api.build_S(to_dev(w.X, torch), "abscorr")
    ok, worst = s_close(S.cpu().numpy(), oracle.abs_corr(w.X))
    assert ok, worst


def test_build_errors(torch, api):
    from symmetric_nmf_clustering_amd._lib import SymNMFError, E_NONFINITE, E_DEGENERATE
    X = np.random.default_rng(0).standard_normal((20, 50)).astype(np.float32)
    Xc = X.copy(); Xc[:, 7] = 3.0
    with pytest.raises(SymNMFError) as e:
        api.build_S(to_dev(Xc, torch), "abscorr")
    assert e.value.status == E_DEGENERATE
    Xn = X.copy(); Xn[4, 9] = np.nan
    for kind in ("abscorr", "tpdm"):
        with pytest.raises(SymNMFError) as e:
            api.build_S(to_dev(Xn, torch), kind)
        assert e.value.status == E_NONFINITE


# ---- TPDM build -------------------------------------------------------------------
def test_build_tpdm_hand_case(torch, api, golden_dir):
    X = np.array([[0.0, 0.1], [-1.0, -2.0], [1.0, 2.0], [0.5, -0.5]], np.float32)
    S, fro = api.build_S(to_dev(X, torch), "tpdm", tail_frac=0.5)
    a = math.sqrt(-1.0 / math.log(0.6))
    b = math.sqrt(-1.0 / math.log(0.4))
    den = a * a + b * b
    hand = np.array([[(0.5 + a * a / den) / 2, (0.5 + a * b / den) / 2],
                     [(0.5 + a * b / den) / 2, (0.5 + b * b / den) / 2]])
    np.testing.assert_allclose(S.cpu().numpy(), hand, rtol=2e-7)


# windows longer than the LDS-staged ranking (more than 16 000 days), and one
# past 46 340 days, where the day x rank histogram's offsets exceed 2^31
@pytest.mark.parametrize("n,T", [(40, 16001), (8, 46400)])
def test_build_tpdm_long_window(torch, api, n, T):
    w = synth.student_factor_stress(n=n, k=2, T=T, seed=3, min_size=4, stress_groups=2)
    S, fro = api.build_S(to_dev(w.X, torch), "tpdm", tail_frac=0.05)
    ref = oracle.tpdm(w.X, 0.05)
    ok, worst = s_close(S.cpu().numpy(), ref)
    assert ok, worst
    assert abs(fro - (ref * ref).sum()) <= 1e-5 * (ref * ref).sum()


@pytest.mark.parametrize("n,T,seed", [(1000, 60, 0), (333, 252, 1), (8192, 252, 1)])
def test_build_tpdm(torch, api, n, T, seed):
    w = synth.student_factor_stress(n=n, k=6 if n < 8192 else 24, T=T, seed=seed,
                                    min_size=20 if n < 8192 else 64)
    S, fro = api.build_S(to_dev(w.X, torch), "tpdm", tail_frac=0.05)
    Sg = S.cpu().numpy()
    ref = oracle.tpdm(w.X, 0.05)
    ok, worst = s_close(Sg, ref)
    assert ok, worst
    assert np.array_equal(Sg, Sg.T)
    assert abs(np.trace(Sg.astype(np.float64)) - 1.0) < 1e-5   # unit theta rows, 1/m
    assert abs(fro - (ref * ref).sum()) <= 1e-5 * (ref * ref).sum()
