"""Kernel-level measurement helper for hardware counters.

Builds the dense |corr| S of a synthetic returns window on the device, then runs
``--passes`` full S.H passes through the C ABI (``symnmf_sh``: the same kernel
and launch configuration the fit uses for its full-batch steps) and a plain
element-wise kernel that reads ``--copy-mib`` MiB and writes as many. Under
``rocprofv3 --pmc FETCH_SIZE`` (or ``WRITE_SIZE``) that kernel's per-dispatch
counter value gives the factor that turns the counter into bytes; the S.H dispatches then give the
HBM traffic of one pass. Prints one JSON line with HIP-event timings.

Usage: python -m symmetric_nmf_clustering_amd.profile_passes [--n 100000] [--k 24]
"""
from __future__ import annotations

import argparse
import json
import sys


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--n", type=int, default=100000)
    ap.add_argument("--k", type=int, default=24)
    ap.add_argument("--T", type=int, default=252)
    ap.add_argument("--passes", type=int, default=4)
    ap.add_argument("--copy-mib", type=int, default=4096)
    args = ap.parse_args(argv)

    import numpy as np
    import torch

    from . import _lib, api, synth

    torch.cuda.set_device(0)
    w = synth.student_factor(n=args.n, k=args.k, T=args.T, seed=2,
                             min_size=min(64, args.n // args.k))
    X = torch.from_numpy(w.X).cuda()
    S, _ = api.build_S(X, "abscorr")
    H = torch.from_numpy(synth.random_factor(args.n, args.k, seed=0, scale=0.1)).cuda()
    api.profile_reset()
    api.profile_enable(True)
    for _ in range(args.passes):
        api.sh(S, H)
    torch.cuda.synchronize()
    api.profile_enable(False)
    sh = api.profile_read(_lib.PROF_SH_FULL)
    # calibration: an element-wise kernel that reads copy_mib MiB and writes
    # copy_mib MiB (a contiguous copy_() would go to a DMA engine instead)
    nfl = args.copy_mib * (1 << 20) // 4
    a = torch.ones(nfl, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        torch.mul(a, 1.0, out=b)
    e1.record()
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / 3
    ms = sh["ms"] / max(1, sh["launches"])
    out = {"n": args.n, "k": args.k, "passes": sh["launches"], "sh_avg_ms": ms,
           "sh_GBs": sh["bytes"] / max(1, sh["launches"]) / (ms * 1e-3) / 1e9,
           "copy_bytes_each_way": nfl * 4, "copy_avg_ms": copy_ms,
           "copy_GBs_read_plus_write": 2 * nfl * 4 / (copy_ms * 1e-3) / 1e9}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    sys.exit(main())
