"""GPU test of symnmf_sh_noalloc, the S.H pass for callers that cannot
allocate device memory: called through the C ABI, its P and trace must be bit
for bit those of symnmf_sh (the same kernels on the static scratch), on calls
in a row whose sizes shrink, so that nothing of an earlier call's scratch
leaks into a later one."""
import ctypes

import numpy as np
import pytest

from symmetric_nmf_clustering_amd import synth
from tests.gpu_util import S_to_dev, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _case(torch, n, k, seed):
    S = synth.random_symmetric_nonneg(n, seed)
    H = synth.random_factor(n, k, seed + 1)
    return S_to_dev(S, torch), to_dev(H, torch)


def _check(api, Sd, Hd):
    P_ref, tr_ref = api.sh(Sd, Hd)
    P, tr = api.sh_noalloc(Sd, Hd)
    assert P.shape == P_ref.shape
    assert bool((P == P_ref).all()), float((P - P_ref).abs().max())
    assert tr.item() == tr_ref


def test_sh_noalloc_equals_sh_on_calls_that_shrink():
    torch = require_gpu()
    from symmetric_nmf_clustering_amd import api
    # the largest size the scratch takes at k = 24, then smaller and ragged
    # ones: each result must not depend on what the previous call left
    for n, k, seed in ((21800, 24, 1), (5000, 24, 2), (777, 17, 3), (64, 1, 4), (3001, 80, 5),
                       (9, 5, 6)):
        Sd, Hd = _case(torch, n, k, seed)
        _check(api, Sd, Hd)
        del Sd
    torch.cuda.synchronize()


def test_sh_noalloc_trace_optional_and_raw_c_call():
    torch = require_gpu()
    from symmetric_nmf_clustering_amd import _lib as L, api
    Sd, Hd = _case(torch, 1500, 24, 7)
    P_ref, _ = api.sh(Sd, Hd)
    P = torch.full_like(Hd, float("nan"))
    lib = L.load()
    st = lib.symnmf_sh_noalloc(ctypes.c_void_p(Sd.data_ptr()), 1500, Sd.stride(0),
                               ctypes.c_void_p(Hd.data_ptr()), 24, ctypes.c_void_p(P.data_ptr()),
                               None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == L.OK
    torch.cuda.synchronize()
    assert bool((P == P_ref).all())
    # too large: rejected, output untouched
    big = api.alloc_S(22000)
    Hb = torch.zeros((22000, 24), dtype=torch.float32, device="cuda")
    Pb = torch.full_like(Hb, 7.0)
    st = lib.symnmf_sh_noalloc(ctypes.c_void_p(big.data_ptr()), 22000, big.stride(0),
                               ctypes.c_void_p(Hb.data_ptr()), 24, ctypes.c_void_p(Pb.data_ptr()),
                               None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == L.E_TOO_LARGE
    torch.cuda.synchronize()
    assert bool((Pb == 7.0).all())
