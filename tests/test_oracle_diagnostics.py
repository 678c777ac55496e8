"""Pins of the oracle's diagnostics (CPU only): closed forms, invariants, nearest-rank
brute force and numpy's inverted-CDF percentile, and hand-worked fixtures."""
import json
import math
import os

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(99)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_identical_sides_closed_form():
    """Zero-update expectation ("WS2 Cross-Config Logprob Drift Contract", Primary
    Failure Signal): with train == rollout, dlogp is exactly 0, ratio0 = 1 and
    approx_kl0 = 0; nothing is clipped and every percentile of |dlogp| is 0."""
    d = np.zeros(1000, np.float32)
    act = (RNG.random(1000) < 0.7).astype(np.uint8)
    s = oracle.diagnostics(d, act)
    assert s["status"] == "OK"
    assert s["n_active"] == int(act.sum())
    assert s["ratio0"] == 1.0 and s["approx_kl0"] == 0.0 and s["clipfrac0"] == 0.0
    assert s["p95_abs_dlogp"] == s["p99_abs_dlogp"] == s["max_abs_dlogp"] == 0.0
    assert s["mean_abs_dlogp"] == 0.0
    assert s["argmax_row"] == int(np.nonzero(act)[0][0])


def test_kl_identity_and_nonnegativity():
    for scale in (1e-4, 1e-2, 0.5):
        d = (RNG.standard_normal(5000) * scale).astype(np.float32)
        s = oracle.diagnostics(d, np.ones(5000, np.uint8))
        # approx_kl0 = mean(exp(d)) - 1 - mean(d), algebraically
        assert abs(s["approx_kl0"] - (s["ratio0"] - 1.0 - s["mean_dlogp"])) <= 1e-12
        assert s["approx_kl0"] >= 0.0
        # the second-order term: mean(d^2)/2 for small d
        if scale <= 1e-2:
            m2 = float(np.mean(d.astype(np.float64) ** 2)) / 2
            assert abs(s["approx_kl0"] - m2) <= 0.05 * m2


def test_clip_counts_hand_built():
    d = np.array([math.log(1.25), math.log(0.75), math.log(1.1), math.log(0.9), 0.0,
                  -0.3, 0.25], np.float64)
    s = oracle.diagnostics(d, np.ones(len(d), np.uint8), 0.2, 0.2)
    assert s["n_clip_high"] == 2 and s["n_clip_low"] == 2
    assert s["clipfrac0"] == 4 / 7
    s2 = oracle.diagnostics(d, np.ones(len(d), np.uint8), 0.3, 0.1)
    # exp: 1.25, 0.75, 1.1, 0.9, 1, 0.7408, 1.284 -> low (<0.7): none; high (>1.1): 1.25, 1.284
    assert s2["n_clip_low"] == 0 and s2["n_clip_high"] == 2


def test_clip_edges_at_float32_neighbours():
    """The float32 dlogp values on either side of ln(1.2) and ln(0.8)."""
    for edge, side in ((math.log(1.2), "hi"), (math.log(0.8), "lo")):
        f = np.float32(edge)
        below = np.nextafter(f, np.float32(-10))
        above = np.nextafter(f, np.float32(10))
        vals = np.array([below, f, above], np.float32)
        for v in vals:
            s = oracle.diagnostics(np.array([v]), np.ones(1, np.uint8))
            r = math.exp(float(v))
            if side == "hi":
                assert s["n_clip_high"] == (1 if r > 1.2 else 0)
            else:
                assert s["n_clip_low"] == (1 if r < 0.8 else 0)
        # the two neighbours straddle the edge
        assert (math.exp(float(below)) < (1.2 if side == "hi" else 0.8)) and \
               (math.exp(float(above)) > (1.2 if side == "hi" else 0.8))


def _brute_nearest_rank(a, q_num, q_den):
    """Smallest value v of the sample such that at least q*n of the sample is <= v."""
    n = len(a)
    for v in sorted(a):
        if q_den * sum(1 for x in a if x <= v) >= q_num * n:
            return v
    raise AssertionError


@pytest.mark.parametrize("n", [1, 2, 3, 19, 20, 21, 99, 100, 101, 1000, 4097])
def test_percentiles_brute_force_and_numpy(n):
    d = (RNG.standard_normal(n) * 1e-3).astype(np.float32)
    if n > 5:
        d[3] = d[7]  # a tie
    s = oracle.diagnostics(d, np.ones(n, np.uint8))
    a = [abs(float(v)) for v in d]
    if n <= 1000:
        assert s["p95_abs_dlogp"] == _brute_nearest_rank(a, 95, 100)
        assert s["p99_abs_dlogp"] == _brute_nearest_rank(a, 99, 100)
    absd = np.abs(d.astype(np.float64))
    assert s["p95_abs_dlogp"] == float(np.percentile(absd, 95, method="inverted_cdf"))
    assert s["p99_abs_dlogp"] == float(np.percentile(absd, 99, method="inverted_cdf"))
    assert s["max_abs_dlogp"] == float(absd.max())


def test_nearest_rank_integer_arithmetic():
    for n in range(1, 5000):
        assert oracle.nearest_rank(n, 95, 100) == max(1, math.ceil(95 * n / 100))
        assert oracle.nearest_rank(n, 99, 100) == max(1, math.ceil(99 * n / 100))
    assert oracle.nearest_rank(20, 95, 100) == 19
    assert oracle.nearest_rank(100, 99, 100) == 99
    assert oracle.nearest_rank(7, 1, 1) == 7


def test_argmax_ties_and_inactive_rows():
    d = np.array([0.1, -0.5, 0.2, 0.5, 9.0, -0.5], np.float32)
    act = np.array([1, 1, 1, 1, 0, 1], np.uint8)
    s = oracle.diagnostics(d, act)
    assert s["argmax_row"] == 1                 # first of the tied |d| = 0.5 rows
    assert s["max_abs_dlogp"] == 0.5            # row 4 (9.0) is not active
    assert s["n_active"] == 5


def test_statuses():
    assert oracle.diagnostics(np.zeros(4), np.zeros(4, np.uint8))["status"] == "ENOACTIVE"
    s = oracle.diagnostics(np.array([0.0, np.nan, 1.0]), np.ones(3, np.uint8))
    assert s["status"] == "ENONFINITE" and s["n_nonfinite"] == 1
    s = oracle.diagnostics(np.array([0.0, np.nan, 1.0]), np.array([1, 0, 1], np.uint8))
    assert s["status"] == "OK"


def _eval(expr):
    return eval(expr, {"__builtins__": {}}, {"exp": math.exp, "log": math.log,
                                              "expm1": math.expm1, "e": math.e})


def test_golden_worked_examples():
    with open(os.path.join(GOLDEN, "diagnostics_worked.json")) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 3
    for c in cases:
        d = np.array([_eval(v) for v in c["dlogp"]], np.float64)
        act = np.array(c["active"], np.uint8)
        s = oracle.diagnostics(d, act, c["eps_low"], c["eps_high"])
        for k, v in c["expect"].items():
            want = _eval(v) if isinstance(v, str) else v
            if isinstance(want, int) and not isinstance(want, bool):
                assert s[k] == want, (c["name"], k)
            else:
                assert abs(s[k] - want) <= 1e-15 * max(1.0, abs(want)), (c["name"], k, s[k], want)


def test_mismatch_kl_and_k3_equal_the_exact_forward_kl():
    """Tokens drawn in exact proportion to a rational rollout law q, scored by a train law p:
    the k1 mean of -dlogp and the k3 mean of exp(d) - 1 - d both equal KL(q || p) exactly
    (E_q[p/q] = 1), the library routine scipy.stats.entropy(q, p) being the reference."""
    from scipy.stats import entropy as kl
    rng = np.random.default_rng(3)
    counts = rng.integers(1, 40, size=23)
    q = counts / counts.sum()
    p = rng.dirichlet(np.ones(23))
    d = np.repeat(np.log(p) - np.log(q), counts)            # dlogp = train - rollout
    st = oracle.diagnostics(d, np.ones(len(d), np.uint8))
    want = float(kl(q, p))
    assert abs(st["mismatch_kl"] - want) <= 1e-12
    assert abs(st["approx_kl0"] - want) <= 1e-12
    # the reverse direction is a different number: the estimator is not symmetric by accident
    assert abs(float(kl(p, q)) - want) > 1e-3


def test_mismatch_kl_closed_forms():
    act = np.ones(5, np.uint8)
    st = oracle.diagnostics(np.full(5, -0.25), act)
    assert st["mismatch_kl"] == 0.25 and abs(st["approx_kl0"] - (math.exp(-0.25) - 0.75)) < 1e-16
    assert oracle.diagnostics(np.zeros(5), act)["mismatch_kl"] == 0.0
    assert math.isnan(oracle.diagnostics(np.zeros(5), np.zeros(5))["mismatch_kl"])


def test_segment_diagnostics_match_slices_and_the_whole():
    rng = np.random.default_rng(8)
    N = 3000
    d = (rng.standard_t(3, N) * 1e-2).astype(np.float32)
    act = (rng.random(N) < 0.8).astype(np.uint8)
    offsets = np.array([0, 0, 17, 1000, 1001, 2500, 3000])
    segs = oracle.segment_diagnostics(d, act, offsets)
    assert segs[0]["status"] == "ENOACTIVE" and segs[0]["n_active"] == 0   # empty segment
    assert sum(s["n_active"] for s in segs) == int(act.sum())
    for s, (lo, hi) in zip(segs, zip(offsets[:-1], offsets[1:])):
        if s["n_active"] == 0:
            continue
        a = np.abs(d[lo:hi][act[lo:hi] == 1].astype(np.float64))
        assert s["max_abs_dlogp"] == a.max()
        r = s["argmax_row"]
        assert lo <= r < hi and act[r] == 1 and abs(float(d[r])) == a.max()
        srt = np.sort(a)
        assert s["p99_abs_dlogp"] == srt[math.ceil(0.99 * len(a) - 1e-9) - 1]
    whole = oracle.segment_diagnostics(d, act, np.array([0, N]))[0]
    ref = oracle.diagnostics(d, act)
    for k in ref:
        assert (whole[k] == ref[k]) or (isinstance(ref[k], float) and math.isnan(ref[k])), k
    bad = oracle.segment_diagnostics(d, act, np.array([0, 10, 5, N]))
    assert bad[1]["status"] == "EMASK" and bad[0]["status"] == "OK"
    assert oracle.segment_diagnostics(d, act, np.array([0, N + 1]))[0]["status"] == "EMASK"
