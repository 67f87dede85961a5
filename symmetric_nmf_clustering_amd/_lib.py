"""ctypes loader for libsymnmf.so and mirrors of the C structs in include/symnmf.h.

The library is loaded on first use. If it has not been built the loader raises:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SYMNMF_LIB", os.path.join(_HERE, "lib", "libsymnmf.so"))

OK = 0
W_NOT_CONVERGED = 1
E_INVALID = -1
E_WORKSPACE = -2
E_HIP = -3
E_NONFINITE = -4
E_DEGENERATE = -5
E_TOO_LARGE = -6

ABSCORR, TPDM = 0, 1
AUTO, FULL, BLOCK_SVRG = 0, 1, 2
INIT_UNIFORM, INIT_SCALE_MATCHED, INIT_CALLER = 0, 1, 2
SH_ROWS, SH_UPPER = 0, 1
OP_BUILD_S, OP_PROBE, OP_FIT, OP_SH, OP_KMEANS, OP_SQ, OP_SH_SYM = 0, 1, 2, 3, 4, 5, 6
(PROF_SH_FULL, PROF_SH_SAMPLED, PROF_SH_PROBE, PROF_BUILD_GRAM, PROF_UPDATE,
 PROF_SH_KMEANS, PROF_SH_SYM) = 0, 1, 2, 3, 4, 5, 6
PROF_NAMES = {
    PROF_SH_FULL: "sh_full", PROF_SH_SAMPLED: "sh_sampled", PROF_SH_PROBE: "sh_probe",
    PROF_BUILD_GRAM: "build_gram", PROF_UPDATE: "update", PROF_SH_KMEANS: "sh_kmeans",
    PROF_SH_SYM: "sh_sym",
}


class FitParams(ctypes.Structure):
    _fields_ = [
        ("solver", ctypes.c_int32),
        ("max_iters", ctypes.c_int32),
        ("lr", ctypes.c_double),
        ("eps", ctypes.c_double),
        ("block_rows", ctypes.c_int32),
        ("init", ctypes.c_int32),
        ("phi0", ctypes.c_double),
        ("gap_threshold", ctypes.c_double),
        ("tol_rel", ctypes.c_double),
        ("stall_tol", ctypes.c_double),
        ("init_scale", ctypes.c_double),
        ("seed", ctypes.c_uint64),
        ("check_every", ctypes.c_int32),
        ("resume", ctypes.c_int32),
        ("rms_decay", ctypes.c_double),
        ("sh_pass", ctypes.c_int32),
        ("obj_floor", ctypes.c_double),
        ("start_iter", ctypes.c_int32),
    ]


class FitState(ctypes.Structure):
    """symnmf_fit_state: the controller state at a returned H (resumption)."""
    _fields_ = [
        ("iter", ctypes.c_int32),
        ("blocks", ctypes.c_int32),
        ("anchor_iter", ctypes.c_int32),
        ("f_prev_valid", ctypes.c_int32),
        ("f_anchor", ctypes.c_double),
        ("f_prev", ctypes.c_double),
        ("H_anchor", ctypes.c_void_p),
        ("P_anchor", ctypes.c_void_p),
    ]


class FitReport(ctypes.Structure):
    _fields_ = [
        ("iterations", ctypes.c_int32),
        ("converged", ctypes.c_int32),
        ("start_branch", ctypes.c_int32),
        ("final_branch", ctypes.c_int32),
        ("blocks_final", ctypes.c_int32),
        ("n_blocks", ctypes.c_int32),
        ("doublings", ctypes.c_int32),
        ("zero_rows", ctypes.c_int32),
        ("f_last_iter", ctypes.c_int32),
        ("anchors", ctypes.c_int32),
        ("gamma", ctypes.c_double),
        ("lr_used", ctypes.c_double),
        ("init_scale_used", ctypes.c_double),
        ("f_last", ctypes.c_double),
        ("S_fro2", ctypes.c_double),
        ("S_mean", ctypes.c_double),
        ("seconds", ctypes.c_double),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


# (name, restype, argtypes) for every symbol include/symnmf.h declares
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_D = ctypes.c_double
SIGNATURES = [
    ("symnmf_abi_version", ctypes.c_int, []),
    ("symnmf_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("symnmf_fit_params_default", None, [ctypes.POINTER(FitParams)]),
    ("symnmf_workspace_bytes", ctypes.c_size_t,
     [ctypes.c_int, _I64, _I32, _I64, ctypes.POINTER(FitParams)]),
    ("symnmf_build_S", ctypes.c_int,
     [ctypes.c_int, _P, _I64, _I64, _I64, ctypes.c_float, _P, _I64,
      ctypes.POINTER(_D), _P, ctypes.c_size_t, _P]),
    ("symnmf_spectral_probe", ctypes.c_int,
     [_P, _I64, _I64, _I32, _I32, _D, ctypes.c_uint64, ctypes.POINTER(_D),
      ctypes.POINTER(_I32), _P, ctypes.c_size_t, _P]),
    ("symnmf_sh", ctypes.c_int,
     [_P, _I64, _I64, _P, _I32, _P, ctypes.POINTER(_D), _P, ctypes.c_size_t, _P]),
    ("symnmf_sh_noalloc", ctypes.c_int, [_P, _I64, _I64, _P, _I32, _P, _P, _P]),
    ("symnmf_sh_sym", ctypes.c_int,
     [_P, _I64, _I64, _P, _I32, _P, ctypes.POINTER(_D), _P, ctypes.c_size_t, _P]),
    ("symnmf_sq", ctypes.c_int,
     [_P, _I64, _I64, _P, _I32, _P, _P, ctypes.c_size_t, _P]),
    ("symnmf_fit", ctypes.c_int,
     [_P, _I64, _I64, _I32, ctypes.POINTER(FitParams), ctypes.POINTER(_D), _I32,
      _P, _P, ctypes.POINTER(_D), _I32, ctypes.POINTER(FitReport), ctypes.POINTER(FitState),
      _P, ctypes.c_size_t, _P]),
    ("symnmf_labels", ctypes.c_int, [_P, _I64, _I32, _P, _P]),
    ("symnmf_spherical_kmeans", ctypes.c_int,
     [_P, _I64, _I64, _I32, _I32, ctypes.c_uint64, _P, _P, ctypes.POINTER(_I32),
      ctypes.POINTER(_I32), ctypes.POINTER(_D), _P, ctypes.c_size_t, _P]),
    ("symnmf_profile_enable", None, [ctypes.c_int]),
    ("symnmf_profile_reset", None, []),
    ("symnmf_profile_read", ctypes.c_int,
     [ctypes.c_int, ctypes.POINTER(_I64), ctypes.POINTER(_D), ctypes.POINTER(_D)]),
]

_lib = None
_lock = threading.Lock()


class SymNMFError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = status_string(status) if _lib is not None else str(status)
        super().__init__(f"{where}: {msg} (status {status})")


def load(path: str | None = None):
    """Load libsymnmf.so (once). Raises if it is missing: build it first with
    ``python -m symmetric_nmf_clustering_amd.csrc.build``."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"libsymnmf.so not found at {p}; build it with "
                "`python -m symmetric_nmf_clustering_amd.csrc.build`")
        lib = ctypes.CDLL(p)
        for name, res, args in SIGNATURES:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().symnmf_status_string(int(status)).decode()


def check(status: int, where: str, allow_warning: bool = True) -> int:
    if status < 0 or (status > 0 and not allow_warning):
        raise SymNMFError(status, where)
    return status
