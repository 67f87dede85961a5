#!/usr/bin/env python3
"""Benchmark of the SymNMF clustering hot path on one MI355X.

One timed step is one whole job on one synthetic returns window resident in
HBM: build |corr| S (n x n fp32) with the MFMA Gram, run the spectral probe
(top 64 eigenvalues), fit S ~ H H^T with the AdaptGrow-selected solver to
convergence, and take the argmax labels. ``value`` is the number of SymNMF
iterations completed per second of whole-job time. The full-batch steps and
anchors take S H from the upper triangle of S (``--sh-pass upper``, the
default for k <= 32; ``rows`` streams all of S). The dominant kernel's achieved
HBM bandwidth is measured live with HIP events on the launch stream (the
library's kernel timing) over the timed region; a full-batch run with the
row-panel pass is timed beside it for reference.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="tfactor_n100000_k24")
    ap.add_argument("--solver", default="auto", choices=["auto", "full", "block_svrg"])
    ap.add_argument("--sh-pass", default="upper", choices=["upper", "rows"],
                    help="S.H product of the full-batch steps and anchors: the upper-triangle "
                         "pass (half the bytes of S, k <= 32) or full row panels")
    ap.add_argument("--probe-p", type=int, default=64)
    ap.add_argument("--probe-iters", type=int, default=300)
    ap.add_argument("--max-iters", type=int, default=2000)
    ap.add_argument("--full-iters", type=int, default=40,
                    help="full-batch steps timed after the jobs (reported separately)")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="rows of S.H the CPU oracle computes for its baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time the oracle baseline spends on its timed sample")
    ap.add_argument("--seeds", type=int, default=3,
                    help="seeds of the untimed time-to-convergence sweep (|corr| and TPDM); 0 skips it")
    ap.add_argument("--no-cold-warm", action="store_true",
                    help="skip the untimed cold/warm-start comparison on the next day's window")
    return ap.parse_args()


def cpu_baseline(w, k, rows, seconds=10.0):
    """The CPU oracle timed on a bounded sample of one full-batch iteration:
    the S.H product on `rows` rows of S (the oracle builds those rows itself,
    untimed) plus the gradient and AdaGrad update on all n x k entries; scaled
    to iterations per second of the whole n x n problem. Each part repeats
    until its share of `seconds` of CPU time is spent (at least 3 times)."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        cores = os.cpu_count() or 1
    n = w.n
    rows = min(rows, n)
    S_rows = oracle.abs_corr_rows(w.X, np.arange(rows))
    mean_est = float(S_rows.mean())
    H = oracle.init_uniform(n, k, oracle.init_scale_matched(mean_est, k), 0)
    lr = oracle.default_lr(mean_est, k)
    def repeat(fn, budget):
        reps, t0 = 0, time.perf_counter()
        while reps < 3 or time.perf_counter() - t0 < budget:
            fn()
            reps += 1
        return (time.perf_counter() - t0) / reps, reps

    rows_idx = np.arange(rows)
    P_rows, _ = oracle.sh_product(S_rows, H, rows=rows_idx)
    t_sh, reps_sh = repeat(lambda: oracle.sh_product(S_rows, H, rows=rows_idx), 0.8 * seconds)
    P = np.zeros((n, k))
    P[:rows] = P_rows
    G = np.zeros_like(H)

    def rest():
        K = H.T @ H
        g = 4.0 * (H @ K - P)
        oracle.adagrad_step(H, G, g, lr)
        return float((H * P).sum()) + float((K * K).sum())

    t_rest, reps_rest = repeat(rest, 0.2 * seconds)
    per_iter = t_sh * (n / rows) + t_rest
    return {"value": 1.0 / per_iter, "unit": "iters/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"S.H on {rows} of {n} rows (fp64 numpy matmul, x{n / rows:.1f}; "
                       f"{reps_sh} repetitions, {reps_sh * t_sh:.1f} s) plus the full n x k "
                       f"gradient/AdaGrad update ({reps_rest} repetitions, {reps_rest * t_rest:.1f} s)"),
            "seconds_per_iter": per_iter}


def cold_warm(args, w, X, S, res_t, api, synth, metrics, sh_pass):
    """Untimed: the window one day on (the same returns moved by a day, one new
    day of the recipe), fitted cold (the pages' protocol: the same seeded
    initialisation for every window) and warm (from the timed jobs' H of the
    current window, fresh accumulator), both with AdaptGrow from that window's
    probe, to convergence."""
    import numpy as np
    import torch
    nxt = synth.student_factor_next(n=w.n, k=w.k, T=w.T, seed=w.seed, shift=1)
    X.copy_(torch.from_numpy(nxt.X))
    api.build_S(X, "abscorr", out=S)
    ev, pits, _ = api.spectral_probe(S, p=args.probe_p, max_iters=args.probe_iters, tol=1e-6,
                                     seed=0)
    out = {"window": "the timed window moved by one day (student_factor_next, shift 1)",
           "probe_iters": pits}
    H_t = res_t.H.clone()
    labels = {}
    for name, kw in (("cold", {}), ("warm", {"H0": H_t})):
        torch.cuda.synchronize()
        t = time.perf_counter()
        r = api.fit(S, w.k, solver=args.solver, eigvals=ev, max_iters=args.max_iters,
                    tol_rel=1e-6, seed=0, sh_pass=sh_pass, **kw)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t
        lab = api.labels(r.H).cpu().numpy()
        labels[name] = lab
        rep = r.report
        out[name] = {"fit_s": dt, "fit_iterations": rep["iterations"],
                     "converged": bool(rep["converged"]),
                     "start_branch": "full" if rep["start_branch"] == 0 else "block_svrg",
                     "doublings": rep["doublings"], "f_last": rep["f_last"],
                     "ari_vs_planted": metrics.adjusted_rand_index(lab, w.labels)}
        print(f"[bench] next window {name}: {rep['iterations']} it in {dt:.2f} s, "
              f"converged={rep['converged']}", file=sys.stderr, flush=True)
    out["ari_cold_vs_warm"] = metrics.adjusted_rand_index(labels["cold"], labels["warm"])
    X.copy_(torch.from_numpy(w.X))
    return out


def measured_traffic(name):
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter
    summary, if the kernel source is the one those counters were taken on
    (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    try:
        rec = json.load(open(path))
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (OSError, KeyError, ValueError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return rec["traffic_bytes_per_launch"]


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU (the path is not sharded across GPUs); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    from symmetric_nmf_clustering_amd import _lib, api, metrics, synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    w = synth.workload(args.workload)
    n, k, T = w.n, w.k, w.T
    X = torch.from_numpy(w.X).to(dev)
    S = api.alloc_S(n, dev)

    sh_pass = args.sh_pass if k <= 32 else "rows"

    def job(kind="abscorr", seed=0):
        ph = {}
        torch.cuda.synchronize()
        t = time.perf_counter()
        _, fro = api.build_S(X, kind, out=S)
        torch.cuda.synchronize()
        ph["build_ms"] = (time.perf_counter() - t) * 1e3
        t = time.perf_counter()
        ev, pits, pconv = api.spectral_probe(S, p=args.probe_p, max_iters=args.probe_iters,
                                             tol=1e-6, seed=seed)
        ph["probe_ms"] = (time.perf_counter() - t) * 1e3
        ph["probe_iters"] = pits
        ph["probe_converged"] = bool(pconv)
        t = time.perf_counter()
        res = api.fit(S, k, solver=args.solver, eigvals=ev, max_iters=args.max_iters,
                      tol_rel=1e-6, seed=seed, sh_pass=sh_pass)
        torch.cuda.synchronize()
        ph["fit_s"] = time.perf_counter() - t
        t = time.perf_counter()
        lab = api.labels(res.H)
        torch.cuda.synchronize()
        ph["labels_ms"] = (time.perf_counter() - t) * 1e3
        print(f"[bench] job: build {ph['build_ms']:.1f} ms, probe {ph['probe_ms']:.0f} ms "
              f"({pits} it), fit {ph['fit_s']:.2f} s ({res.report['iterations']} it, "
              f"converged={res.report['converged']}), labels {ph['labels_ms']:.2f} ms",
              file=sys.stderr, flush=True)
        return res, lab, ev, ph, fro

    for _ in range(args.warmup):
        job()

    api.profile_reset()
    api.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    iters = 0
    phases = []
    for _ in range(args.steps):
        res, lab, ev, ph, fro = job()
        iters += res.report["iterations"]
        phases.append(ph)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    api.profile_enable(False)
    prof = {_lib.PROF_NAMES[i]: api.profile_read(i) for i in _lib.PROF_NAMES}

    rep = res.report
    ari = metrics.adjusted_rand_index(lab.cpu().numpy(), w.labels)

    # full-batch rate on the same S (every step one S.H pass), reported beside
    api.profile_reset()
    api.profile_enable(True)
    torch.cuda.synchronize()
    tf = time.perf_counter()
    full = api.fit(S, k, solver="full", max_iters=args.full_iters, tol_rel=0.0, seed=0,
                   sh_pass=sh_pass)
    torch.cuda.synchronize()
    tf = time.perf_counter() - tf
    api.profile_enable(False)
    prof_fb = {n_: api.profile_read(i) for i, n_ in ((_lib.PROF_SH_FULL, "sh_full"),
                                                     (_lib.PROF_SH_SYM, "sh_sym"))}
    # the row-panel pass on the same S, as a reference beside the upper pass
    api.profile_reset()
    api.profile_enable(True)
    torch.cuda.synchronize()
    tr_ = time.perf_counter()
    api.fit(S, k, solver="full", max_iters=args.full_iters, tol_rel=0.0, seed=0, sh_pass="rows")
    torch.cuda.synchronize()
    tr_ = time.perf_counter() - tr_
    api.profile_enable(False)
    prof_rows = api.profile_read(_lib.PROF_SH_FULL)

    def rate(d):
        ms = d["ms"] / max(1, d["launches"])
        by = d["bytes"] / max(1, d["launches"])
        return ms, by, by / (ms * 1e-3) / 1e9

    if sh_pass == "upper":
        dom = prof["sh_sym"] if prof["sh_sym"]["launches"] else prof_fb["sh_sym"]
        dom_name = "sym_kernel (upper-triangle S.H pass)"
        traffic_file = "sym_n100000_k24_traffic.json"
    else:
        dom = prof["sh_full"] if prof["sh_full"]["launches"] else prof_rows
        dom_name = "sh_panel_kernel (full S.H pass)"
        traffic_file = "sh_panel_n100000_k24_traffic.json"
    sh_ms, sh_bytes, achieved = rate(dom)
    rows_ms, rows_bytes, rows_gbs = rate(prof_rows)
    kernels = {}
    for name, d in list(prof.items()) + [("sh_full_rows_reference_run", prof_rows)]:
        if d["launches"]:
            ms = d["ms"] / d["launches"]
            kernels[name] = {"launches": d["launches"], "avg_ms": ms,
                             "GBs": d["bytes"] / d["launches"] / (ms * 1e-3) / 1e9}

    out = {
        "metric": "SymNMF iters/sec + S·H HBM GB/s (% of peak) at n=100k, k=24, fp32",
        "value": iters / elapsed,
        "unit": "iters/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "n": n, "k": k, "T": T, "S": "abscorr",
                   "solver": args.solver, "probe_p": args.probe_p, "tol_rel": 1e-6,
                   "sh_pass": sh_pass, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (measured_traffic(traffic_file)
                                 if args.workload == "tfactor_n100000_k24" else None),
                     "kernel": dom_name, "avg_ms": sh_ms, "bytes_per_launch": sh_bytes,
                     "rows_pass": {"kernel": "sh_panel_kernel", "avg_ms": rows_ms,
                                   "achieved": rows_gbs, "frac": rows_gbs / HBM_PEAK_GBS,
                                   "bytes_per_launch": rows_bytes,
                                   "traffic": (measured_traffic("sh_panel_n100000_k24_traffic.json")
                                               if args.workload == "tfactor_n100000_k24" else None)}},
        "job": {"fit_iterations": rep["iterations"], "converged": bool(rep["converged"]),
                "start_branch": "full" if rep["start_branch"] == 0 else "block_svrg",
                "final_branch": "full" if rep["final_branch"] == 0 else "block_svrg",
                "gamma_k1": rep["gamma"], "doublings": rep["doublings"],
                "anchors": rep["anchors"], "f_last": rep["f_last"],
                "time_to_convergence_s": float(np.median([p["fit_s"] for p in phases])),
                "build_ms": float(np.median([p["build_ms"] for p in phases])),
                "probe_ms": float(np.median([p["probe_ms"] for p in phases])),
                "probe_iters": phases[-1]["probe_iters"],
                "labels_ms": float(np.median([p["labels_ms"] for p in phases])),
                "fit_iters_per_s": rep["iterations"] / float(np.median([p["fit_s"] for p in phases])),
                "ari_vs_planted": ari, "lambda_top3": [float(x) for x in ev[:3]],
                "lambda_k_k1_k2": [float(ev[k - 1]), float(ev[k]), float(ev[k + 1])]},
        "full_batch": {"iters_per_s": args.full_iters / tf, "steps": args.full_iters,
                       "sh_pass": sh_pass,
                       "rows_pass_iters_per_s": args.full_iters / tr_},
        "kernels": kernels,
    }
    if args.seeds > 0:
        # time to convergence across seeds (init and probe start), |corr| and
        # TPDM on the same returns: the form of the pages' own figures. Not
        # part of the timed region; the timed jobs above are |corr| seed 0.
        sweep = {}
        for kind in ("abscorr", "tpdm"):
            runs = []
            for sd in range(args.seeds):
                if kind == "abscorr" and sd == 0:
                    r0, lab0, ph0 = rep, lab, phases[-1]
                else:
                    rr, lab0, _, ph0, _ = job(kind, sd)
                    r0 = rr.report
                runs.append({"seed": sd, "build_ms": ph0["build_ms"], "probe_ms": ph0["probe_ms"],
                             "probe_iters": ph0["probe_iters"], "fit_s": ph0["fit_s"],
                             "fit_iterations": r0["iterations"], "converged": bool(r0["converged"]),
                             "start_branch": "full" if r0["start_branch"] == 0 else "block_svrg",
                             "blocks_final": r0["blocks_final"],
                             "doublings": r0["doublings"], "gamma_k1": r0["gamma"],
                             "ari_vs_planted": metrics.adjusted_rand_index(lab0.cpu().numpy(), w.labels)})
            fs = [r["fit_s"] for r in runs]
            sweep[kind] = {"runs": runs, "fit_s_mean": float(np.mean(fs)),
                           "fit_s_min_max": [float(min(fs)), float(max(fs))],
                           "probe_plus_fit_s_mean": float(np.mean([r["fit_s"] + r["probe_ms"] / 1e3
                                                                   for r in runs]))}
        out["seeds"] = sweep
    if not args.no_cold_warm:
        out["cold_warm"] = cold_warm(args, w, X, S, res, api, synth, metrics, sh_pass)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, k, args.cpu_rows, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
