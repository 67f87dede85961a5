"""Kernel-level measurement helper for hardware counters.

Builds the dense |corr| S of a synthetic returns window on the device, then runs
``--passes`` full S.H passes through the C ABI (``symnmf_sh``: the same kernel
and launch configuration the fit uses for its full-batch steps; with ``--op sq``
the probe's product ``symnmf_sq`` on a signed n x k basis instead) and a plain
element-wise kernel that reads ``--copy-mib`` MiB and writes as many. Under
``rocprofv3 --pmc FETCH_SIZE`` (or ``WRITE_SIZE``) that kernel's per-dispatch
counter value gives the factor that turns the counter into bytes; the S.H dispatches then give the
HBM traffic of one pass. ``--op sym`` runs the upper-triangle pass (``symnmf_sh_sym``)
instead. Prints one JSON line with HIP-event timings.

Usage: python -m symmetric_nmf_clustering_amd.profile_passes [--n 100000] [--k 24]

``summarize`` turns the two counter runs into the per-launch HBM traffic record
(no GPU needed):

    python -m symmetric_nmf_clustering_amd.profile_passes summarize \
        --fetch-csv F.csv --fetch-json F.json --write-csv W.csv --write-json W.json --out OUT.json \
        [--op sh|sym]

where F/W are rocprofv3's ``*_counter_collection.csv`` of the FETCH_SIZE and
WRITE_SIZE runs and the JSON files hold this module's printed line of each run.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys

COPY_REPS = 3
# the full S.H pass: contiguous row splits (row mode 0)
FULL_PASS = re.compile(r"sh_panel_kernel<(\d+), (\d+), (\d+), (true|false), 0>")
# the upper-triangle pass
SYM_PASS = re.compile(r"sym_kernel<(\d+), (true|false)>")
KERNELS = {
    # op: (dispatch name pattern, source file, algorithmic bytes per launch)
    "sh": (FULL_PASS, "k_sh.hip", lambda n, k: 4.0 * n * n + 8.0 * n * k),
    "sym": (SYM_PASS, "k_sym.hip", lambda n, k: 2.0 * n * (n + 1) + 8.0 * n * k),
}
CALIBRATION = "MulFunctor"


def _counter_rows(path, counter):
    with open(path, newline="") as f:
        return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]


def _last_json(path):
    lines = [ln for ln in open(path).read().splitlines() if ln.startswith("{")]
    return json.loads(lines[-1])


def summarize(argv):
    ap = argparse.ArgumentParser(prog="profile_passes summarize")
    ap.add_argument("--fetch-csv", required=True)
    ap.add_argument("--fetch-json", required=True)
    ap.add_argument("--write-csv", required=True)
    ap.add_argument("--write-json", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--op", choices=sorted(KERNELS), default="sh")
    args = ap.parse_args(argv)
    pattern, src_name, algo_bytes = KERNELS[args.op]
    rec = {}
    for counter, cpath, jpath in (("FETCH_SIZE", args.fetch_csv, args.fetch_json),
                                  ("WRITE_SIZE", args.write_csv, args.write_json)):
        rows = _counter_rows(cpath, counter)
        run = _last_json(jpath)
        sh = [r for r in rows if pattern.search(r["Kernel_Name"])]
        cal = [r for r in rows if CALIBRATION in r["Kernel_Name"]]
        if not sh or not cal:
            raise SystemExit(f"{cpath}: no {args.op} or calibration dispatches")
        names = {pattern.search(r["Kernel_Name"]).group(0) for r in sh}
        if len(names) != 1:
            raise SystemExit(f"{cpath}: several full-pass kernels {sorted(names)}")
        cal_bytes = run["copy_bytes_each_way"] * run["copy_reps"]
        factor = cal_bytes / (sum(float(r["Counter_Value"]) for r in cal) * 1024.0)
        kib = sum(float(r["Counter_Value"]) for r in sh) / len(sh)
        key = counter.lower()
        rec[key + "_kib_per_launch"] = kib
        rec[key + "_factor"] = factor
        rec[key + "_launches"] = len(sh)
        rec[key + "_calibration_dispatches"] = len(cal)
        rec["kernel"] = names.pop()
        rec["n"], rec["k"] = run["n"], run["k"]
    rec["calibration_kernel"] = ("torch element-wise multiply (MulFunctor), "
                                 f"{COPY_REPS} x {run['copy_bytes_each_way']} bytes read and written")
    rec["traffic_bytes_per_launch"] = (rec["fetch_size_kib_per_launch"] * 1024.0 * rec["fetch_size_factor"]
                                       + rec["write_size_kib_per_launch"] * 1024.0 * rec["write_size_factor"])
    n, k = rec["n"], rec["k"]
    rec["algorithmic_bytes_per_launch"] = algo_bytes(n, k)
    src = os.path.join("symmetric_nmf_clustering_amd", "csrc", src_name)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    rec["source"] = src
    rec["source_sha256"] = hashlib.sha256(open(os.path.join(root, src), "rb").read()).hexdigest()
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def main(argv=None):
    argv = sys.argv[1:] if argv is None else argv
    if argv and argv[0] == "summarize":
        return summarize(argv[1:])
    ap = argparse.ArgumentParser()
    ap.add_argument("--n", type=int, default=100000)
    ap.add_argument("--k", type=int, default=24)
    ap.add_argument("--T", type=int, default=252)
    ap.add_argument("--passes", type=int, default=4)
    ap.add_argument("--copy-mib", type=int, default=4096)
    ap.add_argument("--op", choices=("sh", "sq", "sym"), default="sh")
    args = ap.parse_args(argv)

    import numpy as np
    import torch

    from . import _lib, api, synth

    torch.cuda.set_device(0)
    w = synth.student_factor(n=args.n, k=args.k, T=args.T, seed=2,
                             min_size=min(64, args.n // args.k))
    X = torch.from_numpy(w.X).cuda()
    S, _ = api.build_S(X, "abscorr")
    if args.op in ("sh", "sym"):
        H = torch.from_numpy(synth.random_factor(args.n, args.k, seed=0, scale=0.1)).cuda()
    else:
        rng = np.random.default_rng(0)
        H = torch.from_numpy((rng.standard_normal((args.n, args.k)) / np.sqrt(args.n))
                             .astype(np.float32)).cuda()
    api.profile_reset()
    api.profile_enable(True)
    for _ in range(args.passes):
        if args.op == "sh":
            api.sh(S, H)
        elif args.op == "sym":
            api.sh_sym(S, H)
        else:
            api.sq(S, H)
    torch.cuda.synchronize()
    api.profile_enable(False)
    sh = api.profile_read({"sh": _lib.PROF_SH_FULL, "sym": _lib.PROF_SH_SYM,
                           "sq": _lib.PROF_SH_PROBE}[args.op])
    # calibration: an element-wise kernel that reads copy_mib MiB and writes
    # copy_mib MiB (a contiguous copy_() would go to a DMA engine instead)
    nfl = args.copy_mib * (1 << 20) // 4
    a = torch.ones(nfl, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(COPY_REPS):
        torch.mul(a, 1.0, out=b)
    e1.record()
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / COPY_REPS
    ms = sh["ms"] / max(1, sh["launches"])
    out = {"n": args.n, "k": args.k, "op": args.op, "passes": sh["launches"], "sh_avg_ms": ms,
           "sh_GBs": sh["bytes"] / max(1, sh["launches"]) / (ms * 1e-3) / 1e9,
           "copy_bytes_each_way": nfl * 4, "copy_reps": COPY_REPS, "copy_avg_ms": copy_ms,
           "copy_GBs_read_plus_write": 2 * nfl * 4 / (copy_ms * 1e-3) / 1e9}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    sys.exit(main())
