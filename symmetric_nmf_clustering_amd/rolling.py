"""Re-clustering through time: rolling windows with stability monitoring.

P1 ("GPU-Accelerated Clustering for Financial Instruments at Scale"), sections
"The temporal setup", "Tracking stability through time with the Rand index"
and the tail/body discussion after it: every window of a return stream gets its
own S (|corr| and TPDM), its own SymNMF fit with k fixed, and hard labels; the
labels of window t are compared with those of window t - delta by the adjusted
Rand index; a 3-sigma limit calibrated on calm windows turns a dip into an
alert; and the mean dependence between the stressed sectors, read off each S,
shows a co-crash that leaves the labels unchanged.

Every window runs on the device through the C ABI: ``symnmf_build_S`` into one
reused S buffer, ``symnmf_fit`` (full-batch AdaGrad, a fixed number of steps,
warm-started from the previous window's H unless ``warm_start`` is off),
``symnmf_labels``, and one S.H pass against the 0/1 membership columns of the
monitored groups, whose m x m block sums are the cross-sector dependence. The
host keeps the labels (n int32 per window) and computes the ARI series.

Readings (the pages leave these open):
* warm start: the rolling workload asks for it, the pages fit each window
  independently from the same seed; both are offered (``warm_start``). With a
  warm start the AdaGrad accumulator starts at zero in every window, and the
  first window, which has nothing to start from, is fitted from the seeded init
  to convergence (relative change below ``first_tol``, at most
  ``first_max_iters`` steps): otherwise the first windows of the series would be
  compared against a fit that had only ``iters`` steps.
* boundary instruments: rows of H whose second-largest loading is at least
  half the largest (the pages count instruments that the soft factorization
  keeps split across two clusters but give no rule).
* cross-sector dependence: the mean of S_ij over pairs i, j in different
  monitored groups, raw and scaled to S_ij / sqrt(S_ii S_jj) (the raw TPDM is
  of order 1/n, the scaled one is comparable with |corr|, whose diagonal is 1).
* calm windows: window t is calm when ARI(t - delta, t) exists, fewer than half
  of its days come after the membership switch and it holds no stressed day.
* the limit is the calm mean minus three sample standard deviations.

Usage: python -m symmetric_nmf_clustering_amd.rolling [--workload rolling_n20000_k24]
"""
from __future__ import annotations

import argparse
import json
import sys
import time

import numpy as np

KINDS = ("abscorr", "tpdm")


def calm_mask(W: int, T: int, delta: int, switch_day: int, stress_first: int,
              stress_last: int) -> np.ndarray:
    t = np.arange(W)
    after = np.maximum(0, t + T - switch_day)
    holds_stress = (t + T - 1 >= stress_first) & (t <= stress_last)
    return (t >= delta) & (2 * after < T) & ~holds_stress


def three_sigma(values: np.ndarray, calm: np.ndarray):
    """(limit, mean, sd, flags) of the calm-calibrated 3-sigma lower limit."""
    v = np.asarray(values, dtype=np.float64)
    c = v[calm]
    if c.size < 2:
        raise ValueError("need at least two calm windows to calibrate the limit")
    mean = float(np.mean(c))
    sd = float(np.std(c, ddof=1))
    limit = mean - 3.0 * sd
    flags = np.zeros(v.size, dtype=bool)
    ok = ~np.isnan(v)
    flags[ok] = v[ok] < limit
    return limit, mean, sd, flags


def boundary_share(H: np.ndarray, ratio: float = 0.5) -> float:
    """Share of rows whose second-largest loading is at least ``ratio`` times
    their largest (an all-zero row does not count)."""
    top2 = np.sort(np.asarray(H), axis=1)[:, -2:]
    return float(np.mean((top2[:, 1] > 0) & (top2[:, 0] >= ratio * top2[:, 1])))


def run(stream, *, T: int, windows: int, k: int, iters: int = 100, delta: int = 50,
        kinds=KINDS, warm_start: bool = True, seed: int = 0, tail_frac: float = 0.05,
        monitor_groups=None, keep_H: bool = False, first_max_iters: int = 2000,
        first_tol: float = 1e-6, kmeans: bool = False, kmeans_iters: int = 100,
        boundary_ratio: float = 0.5, S_windows=None) -> dict:
    """Run the rolling workload on ``cuda:0``; returns a dict of per-kind results.

    ``stream`` is a ``synth.Stream`` (host); its returns are copied to the device
    once and every window is a view of that copy. With ``kmeans`` every window
    also gets the spherical k-means baseline on the same S (seeded the same in
    every window), its agreement with the SymNMF labels, and the share of
    boundary instruments in H. ``S_windows`` (optional, one n x n host array per
    kind and window: ``S_windows[kind][t]``) supplies the dependence matrices
    instead of building them from the returns (a caller's own estimator)."""
    import torch

    from . import api, metrics

    if stream.days < T + windows - 1:
        raise ValueError("stream too short for the requested windows")
    n = stream.n
    dev = torch.device("cuda", 0)
    Xd = torch.from_numpy(stream.X).to(dev)
    S = api.alloc_S(n, dev)
    groups = list(stream.stress_groups if monitor_groups is None else monitor_groups)
    member = np.stack([(stream.labels_after == g) for g in groups], axis=1).astype(np.float32)
    Ind = torch.from_numpy(np.ascontiguousarray(member)).to(dev)
    sizes = member.sum(axis=0).astype(np.float64)
    calm = calm_mask(windows, T, delta, stream.switch_day, stream.stress_first, stream.stress_last)
    out = {"n": n, "k": k, "T": T, "windows": windows, "iters": iters, "delta": delta,
           "warm_start": warm_start, "monitor_groups": groups, "calm": calm, "kinds": {}}
    for kind in kinds:
        labs = np.empty((windows, n), dtype=np.int32)
        f_first = np.empty(windows)
        f_last = np.empty(windows)
        block = np.empty((windows, len(groups), len(groups)))
        block_n = np.empty((windows, len(groups), len(groups)))
        first_iters = 0
        first_conv = False
        t_build = np.empty(windows)
        t_fit = np.empty(windows)
        t_mon = np.empty(windows)
        t_km = np.zeros(windows)
        km_ari = np.full(windows, np.nan)
        km_iters = np.zeros(windows, dtype=np.int32)
        boundary = np.empty(windows)
        Hs = []
        H = None
        torch.cuda.synchronize()
        for t in range(windows):
            c0 = time.perf_counter()
            if S_windows is None:
                api.build_S(Xd[t:t + T], kind, tail_frac, out=S)
            else:
                S.copy_(torch.from_numpy(np.ascontiguousarray(S_windows[kind][t], dtype=np.float32)))
            torch.cuda.synchronize()
            c1 = time.perf_counter()
            if warm_start and H is not None:
                res = api.fit(S, k, solver="full", max_iters=iters, tol_rel=0.0, H0=H)
            elif warm_start:
                res = api.fit(S, k, solver="full", max_iters=first_max_iters, tol_rel=first_tol,
                              seed=seed)
                first_iters = res.report["iterations"]
                first_conv = bool(res.report["converged"])
            else:
                res = api.fit(S, k, solver="full", max_iters=iters, tol_rel=0.0, seed=seed)
            H = res.H
            torch.cuda.synchronize()
            c2 = time.perf_counter()
            labs[t] = api.labels(H).cpu().numpy()
            # diagonal of S (n strided elements) for the scaled block means
            dg = S.diagonal().double().clamp_min(1e-300).rsqrt()
            P, _ = api.sh(S, Ind)
            Pn, _ = api.sh(S, (Ind.double() * dg[:, None]).float().contiguous())
            Pm = P.cpu().numpy().astype(np.float64)
            Pnm = Pn.cpu().numpy().astype(np.float64)
            d_host = dg.cpu().numpy()
            Hh = H.cpu().numpy()
            c3 = time.perf_counter()
            boundary[t] = boundary_share(Hh, boundary_ratio)
            if kmeans:
                km = api.spherical_kmeans(S, k, max_iters=kmeans_iters, seed=seed)
                km_lab = km.labels.cpu().numpy()
                t_km[t] = time.perf_counter() - c3
                km_iters[t] = km.iterations
                km_ari[t] = metrics.adjusted_rand_index(km_lab, labs[t])
            block[t] = (member.astype(np.float64).T @ Pm) / np.outer(sizes, sizes)
            block_n[t] = ((member.astype(np.float64) * d_host[:, None]).T @ Pnm) / np.outer(sizes, sizes)
            f_first[t] = res.f_trace[0]
            f_last[t] = res.f_trace[-1]
            t_build[t], t_fit[t], t_mon[t] = c1 - c0, c2 - c1, c3 - c2
            if keep_H:
                Hs.append(Hh)
        drift = np.full(windows, np.nan)
        for t in range(delta, windows):
            drift[t] = metrics.adjusted_rand_index(labs[t - delta], labs[t])
        if calm.sum() >= 2:
            limit, mean, sd, flags = three_sigma(drift, calm)
        else:  # too few windows to calibrate (e.g. a run shorter than delta)
            limit = mean = sd = float("nan")
            flags = np.zeros(windows, dtype=bool)
        m = len(groups)
        off = ~np.eye(m, dtype=bool)
        pair_w = np.outer(sizes, sizes)[off]
        cross = (block[:, off] * pair_w).sum(axis=1) / pair_w.sum()
        cross_n = (block_n[:, off] * pair_w).sum(axis=1) / pair_w.sum()
        planted_before = np.array([metrics.adjusted_rand_index(stream.labels_before, l) for l in labs])
        planted_after = np.array([metrics.adjusted_rand_index(stream.labels_after, l) for l in labs])
        r = {"labels": labs, "f_first": f_first, "f_last": f_last, "block_means": block,
             "block_means_scaled": block_n, "cross_dependence": cross,
             "cross_dependence_scaled": cross_n, "first_window_iters": first_iters,
             "first_window_converged": first_conv,
             "ari_drift": drift, "limit": limit, "calm_mean": mean,
             "calm_sd": sd, "flags": flags, "ari_vs_before": planted_before,
             "ari_vs_after": planted_after, "build_s": t_build, "fit_s": t_fit,
             "monitor_s": t_mon, "boundary_fraction": boundary}
        if kmeans:
            r.update({"kmeans_s": t_km, "kmeans_iters": km_iters, "kmeans_vs_symnmf_ari": km_ari})
        if keep_H:
            r["H"] = Hs
        out["kinds"][kind] = r
    return out


def _num(x):
    x = float(x)
    return x if np.isfinite(x) else None


def summary(res: dict, stream) -> dict:
    """A JSON-able digest: timings, the drift dip and its alert, the co-crash."""
    T, W = res["T"], res["windows"]
    t = np.arange(W)
    holds_stress = (t + T - 1 >= stream.stress_first) & (t <= stream.stress_last)
    d = {"n": res["n"], "k": res["k"], "T": T, "windows": W, "iters": res["iters"],
         "delta": res["delta"], "warm_start": res["warm_start"],
         "calm_windows": int(res["calm"].sum()), "kinds": {}}
    for kind, r in res["kinds"].items():
        per = r["build_s"] + r["fit_s"] + r["monitor_s"]
        flagged = np.flatnonzero(r["flags"])
        dr = r["ari_drift"]
        d["kinds"][kind] = {
            "window_ms_mean": 1e3 * float(per.mean()),
            "build_ms_mean": 1e3 * float(r["build_s"].mean()),
            "fit_ms_mean": 1e3 * float(r["fit_s"].mean()),
            "total_s": float(per.sum()),
            "calm_ari_mean": _num(r["calm_mean"]), "calm_ari_sd": _num(r["calm_sd"]),
            "limit": _num(r["limit"]),
            "min_drift": _num(np.nanmin(dr)) if np.isfinite(dr).any() else None,
            "min_drift_window": int(np.nanargmin(dr)) if np.isfinite(dr).any() else None,
            "flagged_windows": int(flagged.size),
            "first_flag": int(flagged[0]) if flagged.size else None,
            "first_window_iters": int(r["first_window_iters"]),
            "cross_dependence_calm": _num(r["cross_dependence"][~holds_stress].mean())
            if (~holds_stress).any() else None,
            "cross_dependence_stress_peak": float(r["cross_dependence"][holds_stress].max())
            if holds_stress.any() else None,
            "cross_dependence_scaled_calm": _num(r["cross_dependence_scaled"][~holds_stress].mean())
            if (~holds_stress).any() else None,
            "cross_dependence_scaled_stress_peak":
                float(r["cross_dependence_scaled"][holds_stress].max()) if holds_stress.any() else None,
            "ari_vs_planted_first_window": float(r["ari_vs_before"][0]),
            "ari_vs_planted_last_window": float(r["ari_vs_after"][-1]),
            "boundary_fraction_mean": float(r["boundary_fraction"].mean()),
        }
        if "kmeans_s" in r:
            d["kinds"][kind].update({
                "kmeans_ms_mean": 1e3 * float(r["kmeans_s"].mean()),
                "kmeans_iters_mean": float(r["kmeans_iters"].mean()),
                "kmeans_vs_symnmf_ari_mean": float(np.nanmean(r["kmeans_vs_symnmf_ari"])),
            })
    return d


def main(argv=None):
    from . import synth

    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="rolling_n20000_k24", choices=sorted(synth.ROLLING))
    ap.add_argument("--windows", type=int, default=None)
    ap.add_argument("--cold", action="store_true", help="fit every window from the seeded init")
    ap.add_argument("--save", default=None, help="write the per-window series to this .npz")
    ap.add_argument("--no-kmeans", action="store_true", help="skip the spherical k-means baseline")
    args = ap.parse_args(argv)
    cfg = synth.ROLLING[args.workload]
    stream = synth.rolling_stream(**cfg["stream"])
    W = cfg["windows"] if args.windows is None else args.windows
    res = run(stream, T=cfg["T"], windows=W, k=cfg["stream"]["k"], iters=cfg["iters"],
              delta=cfg["delta"], warm_start=not args.cold, kmeans=not args.no_kmeans)
    if args.save:
        arrays = {f"{kind}_{key}": np.asarray(val) for kind, r in res["kinds"].items()
                  for key, val in r.items() if key not in ("labels", "H")}
        np.savez(args.save, calm=res["calm"], **arrays)
    print(json.dumps({"workload": args.workload, **summary(res, stream)}), flush=True)


if __name__ == "__main__":
    sys.exit(main())
