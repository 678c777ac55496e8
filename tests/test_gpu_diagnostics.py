"""GPU parity of drift_diagnostics against the oracle on the SAME dlogp array: counts,
p95/p99/max and the worst row bit-exact, means to 1e-5 relative."""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import assert_gate_b, assert_stats_exact, make_small, run_library, status_name

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _gpu_stats(d, act, eps_lo=0.2, eps_hi=0.2, logprob_ws=None):
    from train_rollout_logprob_amd import binding as B
    dd = torch.as_tensor(np.asarray(d, np.float32), device="cuda")
    aa = torch.as_tensor(np.asarray(act, np.uint8), device="cuda")
    st, s = B.diagnostics(dd, aa, eps_lo, eps_hi, logprob_ws=logprob_ws)
    return status_name(st), s


def _check(d, act, eps_lo=0.2, eps_hi=0.2):
    d = np.asarray(d, np.float32)
    st, got = _gpu_stats(d, act, eps_lo, eps_hi)
    want = oracle.diagnostics(d, act, eps_lo, eps_hi)
    assert st == want["status"], (st, want["status"])
    if want["status"] == "OK":
        assert_stats_exact(got, want)
    return got, want


@pytest.mark.parametrize("n", [1, 2, 3, 100, 4095, 4096, 4097, 12288, 65536, 65537, 100003, 300001])
def test_random_arrays(n):
    rng = np.random.default_rng(n)
    d = (rng.standard_normal(n) * 5e-3).astype(np.float32)
    act = (rng.random(n) < 0.8).astype(np.uint8)
    act[0] = 1
    _check(d, act)


def test_heavy_tails_ties_and_zeros():
    rng = np.random.default_rng(3)
    n = 50000
    d = (rng.standard_t(2, n) * 1e-3).astype(np.float32)
    d[::7] = 0.0
    d[::11] = -d[5]                   # many ties of one magnitude
    d[123] = 0.9                      # clipped high
    d[456] = -0.5                     # clipped low
    act = np.ones(n, np.uint8)
    act[::13] = 0
    got, want = _check(d, act)
    assert got["n_clip_high"] >= 1 and got["n_clip_low"] >= 1


def test_all_equal_values():
    d = np.full(10000, 3e-4, np.float32)
    got, want = _check(d, np.ones(10000, np.uint8))
    assert got["p95_abs_dlogp"] == got["max_abs_dlogp"] == np.float32(3e-4)
    assert got["argmax_row"] == 0


def test_clip_edges_and_asymmetric_range():
    edge_hi = np.float32(math.log(1.2))
    edge_lo = np.float32(math.log(0.8))
    vals = [np.nextafter(edge_hi, np.float32(0)), edge_hi, np.nextafter(edge_hi, np.float32(1)),
            np.nextafter(edge_lo, np.float32(0)), edge_lo, np.nextafter(edge_lo, np.float32(-1)),
            0.25, -0.3, 0.1]
    d = np.array(vals, np.float32)
    _check(d, np.ones(len(d), np.uint8))
    _check(d, np.ones(len(d), np.uint8), 0.3, 0.1)


def test_statuses():
    st, s = _gpu_stats(np.zeros(10, np.float32), np.zeros(10, np.uint8))
    assert st == "ENOACTIVE" and s["n_active"] == 0 and s["argmax_row"] == -1
    assert math.isnan(s["ratio0"]) and math.isnan(s["p95_abs_dlogp"])
    d = np.array([0.0, np.nan, 1.0], np.float32)
    st, s = _gpu_stats(d, np.ones(3, np.uint8))
    assert st == "ENONFINITE" and s["n_nonfinite"] == 1
    st, s = _gpu_stats(d, np.array([1, 0, 1], np.uint8))
    assert st == "OK"


def test_zero_update_closed_form_on_gpu_pipeline():
    """train == rollout through the whole path: d = 0, ratio0 = 1, approx_kl0 = 0,
    clipfrac0 = 0, every percentile 0."""
    case = make_small(dict(name="qwen8b", B=2, L=64))
    got = run_library(case, rollout=case.train)
    from train_rollout_logprob_amd import binding as B
    st, s = B.diagnostics(got["d_dev"], got["a_dev"], logprob_ws=got["ws"])
    assert status_name(st) == "OK"
    assert s["n_active"] == case.n_active()
    assert s["ratio0"] == 1.0 and s["approx_kl0"] == 0.0 and s["clipfrac0"] == 0.0
    assert s["p95_abs_dlogp"] == s["p99_abs_dlogp"] == s["max_abs_dlogp"] == 0.0


@pytest.mark.parametrize("key", ["tiny", "qwen8b_small", "packed_small"])
def test_pipeline_gate_a_and_gate_b(key):
    """Gate A: diagnostics of the GPU's dlogp array equal the oracle's diagnostics of the
    same array (exact counts and order statistics). Gate B (end to end): every GPU mean
    (ratio0, approx_kl0, mean |d|, mean d, mismatch_kl) against the oracle's means of its
    own fp64 dlogp, to 1e-5 relative; counts, clip counts and order statistics as far as
    the per-token tolerance decides them."""
    from helpers import run_oracle, small_variants
    case = make_small(small_variants()[key])
    got = run_library(case)
    from train_rollout_logprob_amd import binding as B
    st, s = B.diagnostics(got["d_dev"], got["a_dev"], case.eps_low, case.eps_high,
                          logprob_ws=got["ws"])
    assert status_name(st) == "OK"
    want_a = oracle.diagnostics(got["dlogp"], got["active"], case.eps_low, case.eps_high)
    assert_stats_exact(s, want_a)
    ref = run_oracle(case)
    want_b = oracle.diagnostics(ref["dlogp"], ref["active"], case.eps_low, case.eps_high)
    print(f"[gate B] {key}: " + ", ".join(
        f"{k} rel={abs(s[k] - want_b[k]) / abs(want_b[k]):.2e}"
        for k in ("ratio0", "approx_kl0", "mean_abs_dlogp")), flush=True)
    act = ref["active"] == 1
    assert_gate_b(s, want_b, ref["dlogp"][act], case.eps_low, case.eps_high)


@pytest.mark.parametrize("n", [4099, 100003])
def test_unaligned_views_take_the_scalar_loads(n):
    """dlogp and active as views one element in (4-byte but not 16-byte aligned): the
    select reads the rows one by one instead of four at a time; same statistics."""
    from train_rollout_logprob_amd import binding as B
    rng = np.random.default_rng(n + 1)
    d = (rng.standard_normal(n + 1) * 5e-3).astype(np.float32)
    act = (rng.random(n + 1) < 0.7).astype(np.uint8)
    dd = torch.as_tensor(d, device="cuda")[1:]
    aa = torch.as_tensor(act, device="cuda")[1:]
    assert dd.data_ptr() % 16 != 0 and aa.data_ptr() % 4 != 0
    st, got = B.diagnostics(dd, aa, 0.2, 0.2)
    want = oracle.diagnostics(d[1:], act[1:], 0.2, 0.2)
    assert status_name(st) == want["status"] == "OK"
    assert_stats_exact(got, want)


def test_statuses_and_ties_above_the_single_block_size():
    """Batches above 65536 rows take one launch per digit: no active row, a non-finite
    dlogp, and all-equal magnitudes behave as in the single-block selection."""
    n = 70001
    st, s = _gpu_stats(np.zeros(n, np.float32), np.zeros(n, np.uint8))
    assert st == "ENOACTIVE" and s["n_active"] == 0 and math.isnan(s["p99_abs_dlogp"])
    d = np.full(n, -2.5e-4, np.float32)
    d[::3] = 2.5e-4
    got, want = _check(d, np.ones(n, np.uint8))
    assert got["p95_abs_dlogp"] == got["max_abs_dlogp"] == np.float32(2.5e-4)
    assert got["argmax_row"] == 0
    d[777] = np.inf
    st, s = _gpu_stats(d, np.ones(n, np.uint8))
    assert st == "ENONFINITE" and s["n_nonfinite"] == 1
