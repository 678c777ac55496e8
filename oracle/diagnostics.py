"""Oracle: drift diagnostics over the active rows.

Test infrastructure only (see the package docstring).

Definitions follow the "Diagnostics" table of the page "WS2 Cross-Config Logprob Drift
Contract" (every metric over active response/action tokens only):

* ratio0      = exp(dlogp) per token, reduced as the arithmetic mean over active rows;
* clipfrac0   = mean indicator that ratio0 is outside the clip range [1-eps_low, 1+eps_high]
                (the closed interval is inside; outside is strict);
* approx_kl0  = masked mean of exp(dlogp) - 1 - dlogp, evaluated as expm1(d) - d, which is
                the same quantity without cancellation;
* mean_abs_dlogp, and the max of |dlogp|;
* p95 / p99 of |dlogp| by the nearest-rank rule: the ceil(q*n)-th smallest value;
* mismatch_kl = forward mismatch KL of the "Attention Debug Matrix" Metrics section: the
                k1 estimator of KL(rollout || train) from rollout-sampled tokens, the mean
                of log pi_rollout(y) - log pi_train(y) = mean of -dlogp. (approx_kl0 is the
                k3 estimator of the same KL, the metric that page calls mismatch_k3_kl.)

Per-sequence / per-rank views ("Diagnostics" table, per-rank versions when distributed)
are the same statistics over contiguous row segments given by offsets.

Sums use ``math.fsum`` (correctly rounded). Percentiles come from a full sort. The
worst-token row is the smallest row index attaining the maximum (the B1 acceptance list asks
for worst-token metadata; ties go to the first row).
"""
from __future__ import annotations

import math

import numpy as np


def nearest_rank(n: int, q_num: int, q_den: int) -> int:
    """1-based nearest rank ceil(q*n) for q = q_num/q_den, in exact integer arithmetic,
    clamped to [1, n]."""
    k = (q_num * n + q_den - 1) // q_den
    return max(1, min(n, k))


def diagnostics(d, active, eps_low=0.2, eps_high=0.2):
    """d: dlogp per row (any float dtype; it is widened exactly to float64).
    active: 0/1 per row. Returns a dict of the statistics plus a status string
    ("OK", "ENOACTIVE" when no row is active, "ENONFINITE" when an active dlogp is not
    finite; in the latter case the sums and order statistics are not meaningful)."""
    d = np.asarray(d)
    act = np.asarray(active) != 0
    rows = np.nonzero(act)[0]
    vals = [float(v) for v in d[rows].astype(np.float64)]
    n = len(vals)
    out = {"n_active": n, "n_clip_low": 0, "n_clip_high": 0, "n_nonfinite": 0,
           "argmax_row": -1, "ratio0": math.nan, "clipfrac0": math.nan,
           "approx_kl0": math.nan, "mean_abs_dlogp": math.nan, "mean_dlogp": math.nan,
           "p95_abs_dlogp": math.nan, "p99_abs_dlogp": math.nan,
           "max_abs_dlogp": math.nan, "mismatch_kl": math.nan, "status": "OK"}
    if n == 0:
        out["status"] = "ENOACTIVE"
        return out
    nonfinite = sum(1 for v in vals if not math.isfinite(v))
    out["n_nonfinite"] = nonfinite
    if nonfinite:
        out["status"] = "ENONFINITE"
        return out
    lo_edge = 1.0 - eps_low
    hi_edge = 1.0 + eps_high
    n_lo = 0
    n_hi = 0
    for v in vals:
        ratio = math.exp(v)
        if ratio < lo_edge:
            n_lo += 1
        elif ratio > hi_edge:
            n_hi += 1
    out["n_clip_low"] = n_lo
    out["n_clip_high"] = n_hi
    out["ratio0"] = math.fsum(math.exp(v) for v in vals) / n
    out["approx_kl0"] = math.fsum(math.expm1(v) - v for v in vals) / n
    out["clipfrac0"] = (n_lo + n_hi) / n
    out["mean_abs_dlogp"] = math.fsum(abs(v) for v in vals) / n
    out["mean_dlogp"] = math.fsum(vals) / n
    out["mismatch_kl"] = math.fsum(-v for v in vals) / n
    a = sorted(abs(v) for v in vals)
    out["p95_abs_dlogp"] = a[nearest_rank(n, 95, 100) - 1]
    out["p99_abs_dlogp"] = a[nearest_rank(n, 99, 100) - 1]
    out["max_abs_dlogp"] = a[n - 1]
    mx = a[n - 1]
    for r, v in zip(rows, vals):
        if abs(v) == mx:
            out["argmax_row"] = int(r)
            break
    return out


def segment_diagnostics(d, active, offsets, eps_low=0.2, eps_high=0.2):
    """Statistics of each segment [offsets[s], offsets[s+1]) of the rows (cu_seqlens for
    sequences, b*L for batch rows, or one range per rank). argmax_row is the global row
    index. A segment whose bounds are not 0 <= lo <= hi <= N gets status "EMASK"."""
    d = np.asarray(d)
    active = np.asarray(active)
    N = len(d)
    out = []
    for s in range(len(offsets) - 1):
        lo, hi = int(offsets[s]), int(offsets[s + 1])
        if not 0 <= lo <= hi <= N:
            bad = diagnostics(d[:0], active[:0], eps_low, eps_high)
            bad["status"] = "EMASK"
            out.append(bad)
            continue
        st = diagnostics(d[lo:hi], active[lo:hi], eps_low, eps_high)
        if st["argmax_row"] >= 0:
            st["argmax_row"] += lo
        out.append(st)
    return out
