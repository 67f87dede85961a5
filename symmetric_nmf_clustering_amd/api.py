"""Python binding of libsymnmf (argument marshalling only).

Each function takes and returns torch tensors on the current HIP device and
passes raw device pointers, sizes and torch's current stream to the C ABI of
include/symnmf.h. Every step of the path runs in the library's kernels; torch
only supplies device memory and the stream.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _lib as L

_KINDS = {"abscorr": L.ABSCORR, "corr": L.ABSCORR, "tpdm": L.TPDM}
_SOLVERS = {"auto": L.AUTO, "full": L.FULL, "block_svrg": L.BLOCK_SVRG, "svrg": L.BLOCK_SVRG}
_INITS = {"uniform": L.INIT_UNIFORM, "scale_matched": L.INIT_SCALE_MATCHED, "caller": L.INIT_CALLER}


def _stream_ptr() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require_cuda(t: torch.Tensor, name: str, dtype=torch.float32):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a HIP device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")


def _S_layout(S: torch.Tensor):
    _require_cuda(S, "S")
    if S.dim() != 2 or S.shape[0] != S.shape[1] or S.stride(1) != 1:
        raise ValueError("S must be an n x n row-major view (unit column stride)")
    n = S.shape[0]
    lds = S.stride(0)
    if lds % 4 or S.data_ptr() % 16:
        raise ValueError("S needs a leading dimension that is a multiple of 4 and 16-byte "
                         "alignment; use alloc_S(n) or pad_S(S)")
    return n, lds


def workspace(nbytes: int, device=None) -> torch.Tensor:
    """A caller-owned workspace buffer (torch allocations are 256-byte aligned)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8,
                       device=device or torch.device("cuda"))


def workspace_bytes(op: int, n: int, k_or_p: int, T: int = 0, params: Optional[L.FitParams] = None) -> int:
    lib = L.load()
    b = lib.symnmf_workspace_bytes(op, n, k_or_p, T, ctypes.byref(params) if params else None)
    if b == 0:
        raise ValueError("invalid sizes for workspace query")
    return int(b)


def alloc_S(n: int, device=None) -> torch.Tensor:
    """An uninitialised n x n fp32 view with leading dimension round_up(n, 4)."""
    lds = (n + 3) // 4 * 4
    buf = torch.empty((n, lds), dtype=torch.float32, device=device or torch.device("cuda"))
    return buf[:, :n]


def pad_S(S: torch.Tensor) -> torch.Tensor:
    out = alloc_S(S.shape[0], S.device)
    out.copy_(S)
    return out


# ---------------------------------------------------------------------------
def build_S(X: torch.Tensor, kind: str = "abscorr", tail_frac: float = 0.05,
            out: Optional[torch.Tensor] = None):
    """S (n x n fp32) from a T x n returns window X. Returns (S, ||S||_F^2)."""
    _require_cuda(X, "X")
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be T x n row-major")
    T, n = X.shape
    S = alloc_S(n, X.device) if out is None else out
    n_s, lds = _S_layout(S)
    if n_s != n:
        raise ValueError("out has the wrong size")
    lib = L.load()
    ws = workspace(workspace_bytes(L.OP_BUILD_S, n, 1, T), X.device)
    fro = ctypes.c_double(0.0)
    st = lib.symnmf_build_S(_KINDS[kind], _ptr(X), T, n, X.stride(0), float(tail_frac), _ptr(S),
                            lds, ctypes.byref(fro), _ptr(ws), ws.numel(), ctypes.c_void_p(_stream_ptr()))
    L.check(st, "symnmf_build_S")
    return S, fro.value


def spectral_probe(S: torch.Tensor, p: int = 64, max_iters: int = 300, tol: float = 1e-6,
                   seed: int = 0):
    """Top-p eigenvalues of S by magnitude (sign kept). Returns (eigvals, iters, converged)."""
    n, lds = _S_layout(S)
    lib = L.load()
    ws = workspace(workspace_bytes(L.OP_PROBE, n, p), S.device)
    ev = (ctypes.c_double * p)()
    its = ctypes.c_int32(0)
    st = lib.symnmf_spectral_probe(_ptr(S), n, lds, p, max_iters, float(tol), int(seed), ev,
                                   ctypes.byref(its), _ptr(ws), ws.numel(),
                                   ctypes.c_void_p(_stream_ptr()))
    L.check(st, "symnmf_spectral_probe")
    return np.array(ev[:], dtype=np.float64), int(its.value), st == L.OK


def sh(S: torch.Tensor, H: torch.Tensor):
    """One S.H pass: returns (P = S H, tr(H^T S H))."""
    n, lds = _S_layout(S)
    _require_cuda(H, "H")
    if H.dim() != 2 or H.shape[0] != n or not H.is_contiguous():
        raise ValueError("H must be a contiguous n x k tensor")
    k = H.shape[1]
    P = torch.empty_like(H)
    lib = L.load()
    ws = workspace(workspace_bytes(L.OP_SH, n, k), S.device)
    tr = ctypes.c_double(0.0)
    st = lib.symnmf_sh(_ptr(S), n, lds, _ptr(H), k, _ptr(P), ctypes.byref(tr), _ptr(ws),
                       ws.numel(), ctypes.c_void_p(_stream_ptr()))
    L.check(st, "symnmf_sh")
    return P, tr.value


def sh_noalloc(S: torch.Tensor, H: torch.Tensor, out: Optional[torch.Tensor] = None,
               tr_out: Optional[torch.Tensor] = None):
    """The S.H pass on the library's static scratch (no workspace, no device
    allocation inside the call): returns (P, tr) with tr a one-element float64
    device tensor. ``out`` and ``tr_out`` let the caller own every buffer."""
    n, lds = _S_layout(S)
    _require_cuda(H, "H")
    if H.dim() != 2 or H.shape[0] != n or not H.is_contiguous():
        raise ValueError("H must be a contiguous n x k tensor")
    k = H.shape[1]
    P = torch.empty_like(H) if out is None else out
    tr = torch.empty(1, dtype=torch.float64, device=S.device) if tr_out is None else tr_out
    st = L.load().symnmf_sh_noalloc(_ptr(S), n, lds, _ptr(H), k, _ptr(P), _ptr(tr),
                                    ctypes.c_void_p(_stream_ptr()))
    L.check(st, "symnmf_sh_noalloc")
    return P, tr


def sh_sym(S: torch.Tensor, H: torch.Tensor):
    """The S.H pass from the upper triangle of a symmetric S (each block on or
    above the diagonal read once, bf16 matrix cores with split operands):
    returns (P = S H, tr(H^T S H)); k <= 32."""
    n, lds = _S_layout(S)
    _require_cuda(H, "H")
    if H.dim() != 2 or H.shape[0] != n or not H.is_contiguous() or H.dtype != torch.float32:
        raise ValueError("H must be a contiguous float32 n x k tensor")
    k = H.shape[1]
    P = torch.empty_like(H)
    lib = L.load()
    ws = workspace(workspace_bytes(L.OP_SH_SYM, n, k), S.device)
    tr = ctypes.c_double(0.0)
    st = lib.symnmf_sh_sym(_ptr(S), n, lds, _ptr(H), k, _ptr(P), ctypes.byref(tr), _ptr(ws),
                           ws.numel(), ctypes.c_void_p(_stream_ptr()))
    L.check(st, "symnmf_sh_sym")
    return P, tr.value


def sq(S: torch.Tensor, Q: torch.Tensor) -> torch.Tensor:
    """The probe's product Y = S Q on the bf16 matrix cores (three-part split
    operands, fp32 accumulation)."""
    n, lds = _S_layout(S)
    _require_cuda(Q, "Q")
    if Q.dim() != 2 or Q.shape[0] != n or not Q.is_contiguous() or Q.dtype != torch.float32:
        raise ValueError("Q must be a contiguous float32 n x w tensor")
    w = Q.shape[1]
    Y = torch.empty_like(Q)
    lib = L.load()
    ws = workspace(workspace_bytes(L.OP_SQ, n, w), S.device)
    st = lib.symnmf_sq(_ptr(S), n, lds, _ptr(Q), w, _ptr(Y), _ptr(ws), ws.numel(),
                       ctypes.c_void_p(_stream_ptr()))
    L.check(st, "symnmf_sq")
    return Y


@dataclass
class FitState:
    """The AdaptGrow controller state at a returned H: pass it back with that H
    and G (``fit(..., H0=H, G0=G, state=...)``) to continue the run exactly."""
    iter: int
    blocks: int
    anchor_iter: int
    f_prev_valid: int
    f_anchor: float
    f_prev: float
    H_anchor: torch.Tensor
    P_anchor: torch.Tensor


@dataclass
class FitResult:
    H: torch.Tensor
    G: Optional[torch.Tensor]
    report: dict
    f_trace: np.ndarray
    status: int
    state: Optional[FitState] = None

    @property
    def converged(self) -> bool:
        return bool(self.report["converged"])


def fit_params(**kw) -> L.FitParams:
    lib = L.load()
    p = L.FitParams()
    lib.symnmf_fit_params_default(ctypes.byref(p))
    for key, val in kw.items():
        if key == "solver" and isinstance(val, str):
            val = _SOLVERS[val]
        if key == "init" and isinstance(val, str):
            val = _INITS[val]
        if key == "sh_pass" and isinstance(val, str):
            val = {"rows": L.SH_ROWS, "upper": L.SH_UPPER}[val]
        if not hasattr(p, key):
            raise TypeError(f"unknown fit parameter {key}")
        setattr(p, key, val)
    return p


def fit(S: torch.Tensor, k: int, *, eigvals=None, H0: Optional[torch.Tensor] = None,
        G0: Optional[torch.Tensor] = None, return_G: bool = False,
        trace_cap: Optional[int] = None, ws: Optional[torch.Tensor] = None,
        state: Optional[FitState] = None, return_state: bool = False, **params) -> FitResult:
    """SymNMF fit S ~ H H^T with projected AdaGrad / Block-SVRG AdaptGrow.

    ``params`` are the fields of symnmf_fit_params (solver, max_iters, lr, eps,
    block_rows, init, phi0, gap_threshold, tol_rel, stall_tol, init_scale,
    seed, check_every, rms_decay, sh_pass, obj_floor, start_iter). H0 sets
    init='caller'; G0 sets resume=1. ``state`` (a previous result's state,
    with its H as H0 and G as G0) restores the controller and sets start_iter;
    ``return_state`` asks for the state of the returned H."""
    n, lds = _S_layout(S)
    if H0 is not None:
        if params.setdefault("init", L.INIT_CALLER) not in (L.INIT_CALLER, "caller"):
            raise ValueError("H0 given with an init other than 'caller'")
    if G0 is not None:
        params["resume"] = 1
    if state is not None:
        if G0 is None:
            raise ValueError("resuming from a state needs G0")
        params["start_iter"] = state.iter
    p = fit_params(**params)
    H = torch.empty((n, k), dtype=torch.float32, device=S.device)
    if H0 is not None:
        _require_cuda(H0, "H0")
        H.copy_(H0)
    G = None
    if return_G or G0 is not None:
        G = torch.empty((n, k), dtype=torch.float32, device=S.device)
        if G0 is not None:
            G.copy_(G0)
    cap = p.max_iters if trace_cap is None else int(trace_cap)
    trace = (ctypes.c_double * max(cap, 1))()
    ev = None
    n_eig = 0
    if eigvals is not None:
        eig = np.ascontiguousarray(eigvals, dtype=np.float64)
        ev = eig.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
        n_eig = eig.size
    rep = L.FitReport()
    lib = L.load()
    need = workspace_bytes(L.OP_FIT, n, k, 0, p)
    if ws is None or ws.numel() < need:
        ws = workspace(need, S.device)
    cst = None
    Ha_out = Pa_out = None
    if state is not None or return_state:
        Ha_out = torch.empty((n, k), dtype=torch.float32, device=S.device)
        Pa_out = torch.empty((n, k), dtype=torch.float32, device=S.device)
        cst = L.FitState()
        if state is not None:
            for name in ("iter", "blocks", "anchor_iter", "f_prev_valid", "f_anchor", "f_prev"):
                setattr(cst, name, getattr(state, name))
            Ha_out.copy_(state.H_anchor)
            Pa_out.copy_(state.P_anchor)
        cst.H_anchor = Ha_out.data_ptr()
        cst.P_anchor = Pa_out.data_ptr()
    st = lib.symnmf_fit(_ptr(S), n, lds, k, ctypes.byref(p), ev, n_eig, _ptr(H), _ptr(G),
                        trace if cap > 0 else None, cap, ctypes.byref(rep),
                        ctypes.byref(cst) if cst is not None else None, _ptr(ws), ws.numel(),
                        ctypes.c_void_p(_stream_ptr()))
    L.check(st, "symnmf_fit")
    r = rep.as_dict()
    ncopy = min(cap, r["iterations"] + (1 if r["converged"] else 0))
    out_state = None
    if cst is not None:
        out_state = FitState(cst.iter, cst.blocks, cst.anchor_iter, cst.f_prev_valid,
                             cst.f_anchor, cst.f_prev, Ha_out, Pa_out)
    return FitResult(H, G, r, np.array(trace[:ncopy], dtype=np.float64), st, out_state)


def labels(H: torch.Tensor) -> torch.Tensor:
    """Row-wise argmax of H (lowest index on ties) as int32."""
    _require_cuda(H, "H")
    if H.dim() != 2 or not H.is_contiguous():
        raise ValueError("H must be a contiguous n x k tensor")
    n, k = H.shape
    out = torch.empty(n, dtype=torch.int32, device=H.device)
    st = L.load().symnmf_labels(_ptr(H), n, k, _ptr(out), ctypes.c_void_p(_stream_ptr()))
    L.check(st, "symnmf_labels")
    return out


@dataclass
class KmeansResult:
    labels: torch.Tensor
    centroids: Optional[torch.Tensor]
    iterations: int
    converged: bool
    objective: float
    status: int


def spherical_kmeans(S: torch.Tensor, k: int, *, max_iters: int = 100, seed: int = 0,
                     return_centroids: bool = False) -> KmeansResult:
    """Spherical k-means on the L2-normalised rows of S (the hard-clustering
    baseline). Returns labels (n int32), optionally the centroids (n x k, column
    j = centroid j), the number of centroid updates, whether the last
    assignment moved no row, and sum_i <x_i, c_label(i)>."""
    n, lds = _S_layout(S)
    lab = torch.empty(n, dtype=torch.int32, device=S.device)
    C = torch.empty((n, k), dtype=torch.float32, device=S.device) if return_centroids else None
    ws = workspace(workspace_bytes(L.OP_KMEANS, n, k), S.device)
    it = ctypes.c_int32(0)
    conv = ctypes.c_int32(0)
    obj = ctypes.c_double(0.0)
    st = L.load().symnmf_spherical_kmeans(_ptr(S), n, lds, k, max_iters, seed, _ptr(lab), _ptr(C),
                                          ctypes.byref(it), ctypes.byref(conv), ctypes.byref(obj),
                                          _ptr(ws), ws.numel(), ctypes.c_void_p(_stream_ptr()))
    L.check(st, "symnmf_spherical_kmeans")
    return KmeansResult(lab, C, it.value, bool(conv.value), obj.value, st)


# ---- kernel timing ---------------------------------------------------------
def profile_enable(on: bool = True):
    L.load().symnmf_profile_enable(1 if on else 0)


def profile_reset():
    L.load().symnmf_profile_reset()


def profile_read(which: int):
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    by = ctypes.c_double(0.0)
    L.check(L.load().symnmf_profile_read(which, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(by)),
            "symnmf_profile_read")
    return {"launches": int(n.value), "ms": ms.value, "bytes": by.value}
