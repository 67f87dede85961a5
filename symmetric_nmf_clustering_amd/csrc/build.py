"""Builds libsymnmf.so for gfx950 with hipcc (in-tree, next to the package).

Usage: python -m symmetric_nmf_clustering_amd.csrc.build [--verbose]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
OUT_DIR = os.path.join(PKG, "lib")
OUT = os.path.join(OUT_DIR, "libsymnmf.so")
SOURCES = ["symnmf.cpp", "k_sh.hip", "k_fit.hip", "k_build.hip", "k_kmeans.hip", "k_sq.hip",
           "k_sym.hip", "noalloc.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return cand


def build(verbose: bool = False) -> str:
    """Compiles every source to an object in parallel (one hipcc per file, in
    _build/ at the repository root), then links libsymnmf.so."""
    os.makedirs(OUT_DIR, exist_ok=True)
    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, src + ".o")
        objs.append(obj)
        cmd = [hipcc(), *compile_flags, "-c", "-I", os.path.join(ROOT, "include"), "-I", HERE,
               os.path.join(HERE, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
    failed = []
    for src, pr in procs:
        out, err = pr.communicate()
        if pr.returncode != 0:
            failed.append(src)
            sys.stderr.write(out + err)
        elif verbose and err.strip():
            sys.stderr.write(err)
    if failed:
        raise RuntimeError("hipcc failed on " + ", ".join(failed))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed linking libsymnmf.so")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
