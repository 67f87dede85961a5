"""MI355X (gfx950) SymNMF clustering hot path.

The library (libsymnmf.so, HIP kernels behind the C ABI of include/symnmf.h)
builds the dependence matrix S from a returns window, probes its spectrum,
fits S ~ H H^T with projected AdaGrad / Block-SVRG AdaptGrow and returns
argmax labels. ``api`` is the thin Python binding; ``synth`` draws seeded
synthetic inputs.
"""
from . import _lib  # noqa: F401

__all__ = ["api", "synth", "metrics", "rolling"]


def __getattr__(name):
    if name in ("api", "synth", "metrics", "rolling"):
        import importlib

        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
