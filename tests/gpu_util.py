"""Helpers shared by the GPU tests (device checks, tolerances)."""
import os

import numpy as np
import pytest


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from symmetric_nmf_clustering_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libsymnmf.so is not built: the HIP path must be present on a GPU box")
    return torch


def to_dev(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def S_to_dev(S, torch):
    from symmetric_nmf_clustering_amd import api
    n = S.shape[0]
    out = api.alloc_S(n)
    out.copy_(torch.from_numpy(np.ascontiguousarray(S, dtype=np.float32)))
    return out


def s_close(got, ref, rel=1e-4, floor_frac=1e-3):
    """|dS| <= rel * max(|S_ref|, floor_frac * max|S_ref|) element-wise (the
    per-element relative bound with a floor for entries near zero)."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    floor = floor_frac * np.abs(ref).max()
    bound = rel * np.maximum(np.abs(ref), floor)
    err = np.abs(got - ref)
    return bool(np.all(err <= bound)), float((err / np.maximum(np.abs(ref), floor)).max())
