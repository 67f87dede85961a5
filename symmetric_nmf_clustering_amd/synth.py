"""Seeded synthetic return windows with planted groups.

This module only draws inputs: a T x n window of daily returns X (day-major,
float32) and the planted group label of every instrument. It holds none of the
clustering method's arithmetic, so both the HIP path and the CPU oracle may take
their inputs from it.

The pages ("GPU-Accelerated Clustering for Financial Instruments at Scale",
sections "The temporal setup" and "Choosing the rank k") describe a synthetic
return stream with planted groups of planted rank 24 and a joint tail-stress
episode, but do not print the generator. The recipes below are the workload
definitions this library is measured on:

* ``gaussian_blocks``: n instruments in k equal groups, r = a*f_g + b*e with
  f, e iid N(0, 1) (n=1024, k=8, T=256, a=0.6, b=0.8, seed 0).
* ``student_factor``: k groups of size 64 + Multinomial(n - 64k, 1/k), group
  membership by a seeded permutation, per-instrument loading l ~ U(0.3, 0.9),
  r = l*f_g + sqrt(1 - l^2)*e with f and e Student-t (df 4) divided by sqrt(2)
  so they have unit variance.
* ``student_factor_stress``: the same, plus a joint crash: on 10 contiguous
  days starting at a seeded day, every member of the first 4 groups of a
  seeded group permutation receives an extra -5 (five unit standard
  deviations).

* ``rolling_stream``: a D-day stream for rolling windows (the pages' "The
  temporal setup": instruments change planted group, and several groups share
  a tail-stress episode without changing group). Returns as in
  ``student_factor``, day by day under the membership of that day: a seeded
  fraction of instruments moves to another group from ``switch_day`` on, and
  on days ``stress_first``..``stress_last`` (inclusive) every member of a
  seeded set of groups receives an extra ``shock``.

Draw order (numpy ``default_rng(seed)``) is fixed and documented per function,
so a recipe is reproducible from its name, sizes and seed alone.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Window:
    """One synthetic window: returns X (T x n, float32, day-major) and labels."""

    X: np.ndarray
    labels: np.ndarray
    k: int
    recipe: str
    seed: int
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return self.X.shape[0]

    @property
    def n(self) -> int:
        return self.X.shape[1]


def _t4_unit(rng: np.random.Generator, shape) -> np.ndarray:
    # Student-t with 4 degrees of freedom has variance 4/(4-2) = 2.
    return rng.standard_t(4, size=shape) / np.sqrt(2.0)


def gaussian_blocks(n: int = 1024, k: int = 8, T: int = 256, a: float = 0.6,
                    b: float = 0.8, seed: int = 0) -> Window:
    """Equal groups, Gaussian factors and noise.

    Draw order: group permutation (n), factors F (T x k), noise E (T x n).
    """
    if n % k:
        raise ValueError("gaussian_blocks needs n divisible by k")
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n)
    labels = np.empty(n, dtype=np.int32)
    labels[perm] = np.repeat(np.arange(k, dtype=np.int32), n // k)
    F = rng.standard_normal((T, k))
    E = rng.standard_normal((T, n))
    X = a * F[:, labels] + b * E
    return Window(np.ascontiguousarray(X, dtype=np.float32), labels, k, "gaussian_blocks", seed,
                  {"a": a, "b": b})


def _student_groups(rng, n, k, min_size):
    if n < min_size * k:
        raise ValueError("n too small for k groups of the minimum size")
    sizes = min_size + rng.multinomial(n - min_size * k, np.full(k, 1.0 / k))
    perm = rng.permutation(n)
    labels = np.empty(n, dtype=np.int32)
    labels[perm] = np.repeat(np.arange(k, dtype=np.int32), sizes)
    return sizes, labels


def student_factor(n: int = 8192, k: int = 24, T: int = 252, seed: int = 1,
                   min_size: int = 64) -> Window:
    """Student-t planted-factor returns.

    Draw order: group sizes (multinomial), membership permutation (n),
    loadings l (n), factors F (T x k), noise E (T x n).
    """
    rng = np.random.default_rng(seed)
    sizes, labels = _student_groups(rng, n, k, min_size)
    load = rng.uniform(0.3, 0.9, size=n)
    F = _t4_unit(rng, (T, k))
    E = _t4_unit(rng, (T, n))
    X = load * F[:, labels] + np.sqrt(1.0 - load * load) * E
    return Window(np.ascontiguousarray(X, dtype=np.float32), labels, k, "student_factor", seed,
                  {"sizes": sizes.tolist()})


def student_factor_next(n: int = 8192, k: int = 24, T: int = 252, seed: int = 1,
                        shift: int = 1, min_size: int = 64) -> Window:
    """The ``student_factor`` window moved ``shift`` days on: days shift ..
    T - 1 of ``student_factor(n, k, T, seed)`` followed by ``shift`` new days of
    the same recipe (same groups and loadings), for warm-start comparisons
    between consecutive windows.

    Draw order: ``student_factor``'s draws (to recover the groups and
    loadings), then from ``default_rng([seed, 2])``, day by day, the new day's
    factors (k) and noise (n), so the days after the window do not depend on
    ``shift``.
    """
    base = student_factor(n, k, T, seed, min_size)
    rng0 = np.random.default_rng(seed)
    _student_groups(rng0, n, k, min_size)
    load = rng0.uniform(0.3, 0.9, size=n)
    rng = np.random.default_rng([seed, 2])
    new = np.empty((shift, n))
    for d in range(shift):
        f = _t4_unit(rng, k)
        e = _t4_unit(rng, n)
        new[d] = load * f[base.labels] + np.sqrt(1.0 - load * load) * e
    X = np.concatenate([base.X[shift:].astype(np.float64), new], axis=0)
    return Window(np.ascontiguousarray(X, dtype=np.float32), base.labels, k, "student_factor_next",
                  seed, {"sizes": base.meta["sizes"], "shift": shift})


def student_factor_stress(n: int = 8192, k: int = 24, T: int = 252,
                          seed: int = 1, min_size: int = 64,
                          stress_groups: int = 4, stress_days: int = 10,
                          shock: float = -5.0) -> Window:
    """``student_factor`` plus a joint tail-stress episode.

    The draws of ``student_factor`` come first (same seed gives the same
    calm returns), then: a permutation of the k groups (the first
    ``stress_groups`` are stressed) and the first stressed day, uniform on
    [0, T - stress_days].
    """
    base = student_factor(n, k, T, seed, min_size)
    rng = np.random.default_rng([seed, 1])
    gperm = rng.permutation(k)
    groups = np.sort(gperm[:stress_groups])
    day0 = int(rng.integers(0, T - stress_days + 1))
    X = base.X.astype(np.float64)
    members = np.isin(base.labels, groups)
    X[day0:day0 + stress_days, members] += shock
    meta = dict(base.meta)
    meta.update({"stress_groups": groups.tolist(), "stress_day0": day0,
                 "stress_days": stress_days, "shock": shock})
    return Window(np.ascontiguousarray(X, dtype=np.float32), base.labels, k,
                  "student_factor_stress", seed, meta)


@dataclass
class Stream:
    """A D x n day-major return stream (float32) and its planted structure."""

    X: np.ndarray
    labels_before: np.ndarray   # membership before switch_day
    labels_after: np.ndarray    # membership from switch_day on
    switched: np.ndarray        # indices of the instruments that moved
    k: int
    switch_day: int
    stress_groups: list
    stress_first: int
    stress_last: int            # inclusive
    seed: int
    meta: dict = field(default_factory=dict)

    @property
    def days(self) -> int:
        return self.X.shape[0]

    @property
    def n(self) -> int:
        return self.X.shape[1]

    def window(self, t: int, T: int) -> np.ndarray:
        """Days t .. t + T - 1 (a view)."""
        if t < 0 or t + T > self.days:
            raise ValueError("window outside the stream")
        return self.X[t:t + T]


def rolling_stream(n: int = 20000, k: int = 24, days: int = 501, switch_day: int = 300,
                   switch_frac: float = 0.05, stress_groups: int = 3, stress_first: int = 420,
                   stress_last: int = 430, shock: float = -5.0, seed: int = 5,
                   min_size: int = 64) -> Stream:
    """Student-t planted-factor stream with a membership switch and a co-crash.

    Draw order: group sizes (multinomial), membership permutation (n),
    loadings l (n), a permutation of the instruments (the first
    round(switch_frac n) switch), for each switcher an offset in 1..k-1 (its new
    group is (old + offset) mod k), a permutation of the k groups (the first
    ``stress_groups`` are stressed), factors F (days x k), noise E (days x n).
    The stressed groups are taken in the membership from ``switch_day`` on.
    """
    if not (0 <= switch_day <= days and 0 <= stress_first <= stress_last < days):
        raise ValueError("event days outside the stream")
    rng = np.random.default_rng(seed)
    _, before = _student_groups(rng, n, k, min_size)
    load = rng.uniform(0.3, 0.9, size=n)
    nsw = int(round(switch_frac * n))
    switched = np.sort(rng.permutation(n)[:nsw])
    offs = rng.integers(1, k, size=nsw)
    after = before.copy()
    after[switched] = (before[switched] + offs) % k
    gperm = rng.permutation(k)
    groups = np.sort(gperm[:stress_groups])
    F = _t4_unit(rng, (days, k))
    E = _t4_unit(rng, (days, n))
    X = np.empty((days, n), dtype=np.float64)
    cut = switch_day
    scale = np.sqrt(1.0 - load * load)
    X[:cut] = load * F[:cut][:, before] + scale * E[:cut]
    X[cut:] = load * F[cut:][:, after] + scale * E[cut:]
    members = np.isin(after, groups)
    X[stress_first:stress_last + 1, members] += shock
    return Stream(np.ascontiguousarray(X, dtype=np.float32), before.astype(np.int32),
                  after.astype(np.int32), switched, k, switch_day, groups.tolist(), stress_first,
                  stress_last, seed, {"switch_frac": switch_frac, "shock": shock,
                                      "min_size": min_size})


# Named workloads: (recipe, kwargs).  The sizes are the ones the library is
# measured and parity-tested on.
WORKLOADS = {
    "blocks_n1024_k8": (gaussian_blocks, dict(n=1024, k=8, T=256, seed=0)),
    "tfactor_n8192_k24": (student_factor, dict(n=8192, k=24, T=252, seed=1)),
    "tstress_n8192_k24": (student_factor_stress,
                          dict(n=8192, k=24, T=252, seed=1)),
    "tfactor_n100000_k24": (student_factor,
                            dict(n=100000, k=24, T=252, seed=2)),
}

# The rolling workload: a 501-day stream read as 250 windows of 252 days.
ROLLING = {
    "rolling_n20000_k24": dict(stream=dict(n=20000, k=24, days=501, switch_day=300,
                                           switch_frac=0.05, stress_groups=3, stress_first=420,
                                           stress_last=430, seed=5),
                               T=252, windows=250, iters=100, delta=50),
}


def workload(name: str, **overrides) -> Window:
    fn, kw = WORKLOADS[name]
    kw = dict(kw)
    kw.update(overrides)
    return fn(**kw)


def random_symmetric_nonneg(n: int, seed: int, dtype=np.float32) -> np.ndarray:
    """A seeded dense symmetric nonnegative matrix (uniform [0, 1) entries),
    for kernel tests that need an S without a returns window."""
    rng = np.random.default_rng(seed)
    A = rng.random((n, n))
    S = np.triu(A) + np.triu(A, 1).T
    return S.astype(dtype)


def random_factor(n: int, k: int, seed: int, scale: float = 1.0,
                  dtype=np.float32) -> np.ndarray:
    """A seeded nonnegative n x k factor, uniform on [0, scale)."""
    rng = np.random.default_rng(seed)
    return (scale * rng.random((n, k))).astype(dtype)
