"""GPU parity of drift_segment_diagnostics (per-sequence / per-batch-row / per-rank views
of the "Diagnostics" table) against the oracle's per-segment diagnostics of the SAME dlogp
array: counts, p95/p99/max and the worst row bit-exact, means (and the forward mismatch
KL) to 1e-5 relative."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_stats_exact, device_inputs, make_small, run_library, status_name
from train_rollout_logprob_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _segments(d, act, offsets, eps_lo=0.2, eps_hi=0.2, logprob_ws=None):
    from train_rollout_logprob_amd import binding as B
    dd = torch.as_tensor(np.asarray(d, np.float32), device="cuda")
    aa = torch.as_tensor(np.asarray(act, np.uint8), device="cuda")
    oo = torch.as_tensor(np.asarray(offsets, np.int32), device="cuda")
    return B.segment_diagnostics(dd, aa, oo, eps_lo, eps_hi, logprob_ws=logprob_ws)


def _check(d, act, offsets, eps_lo=0.2, eps_hi=0.2):
    d = np.asarray(d, np.float32)
    got = _segments(d, act, offsets, eps_lo, eps_hi)
    want = oracle.segment_diagnostics(d, act, offsets, eps_lo, eps_hi)
    assert len(got) == len(want)
    for s, (g, w) in enumerate(zip(got, want)):
        assert status_name(g["status"]) == w["status"], (s, g["status"], w["status"])
        if w["status"] == "OK":
            assert_stats_exact(g, w)
        assert g["n_active"] == w["n_active"]
    return got, want


def test_random_segments_with_empty_and_tiny_ones():
    rng = np.random.default_rng(41)
    N = 20000
    d = (rng.standard_t(2, N) * 3e-3).astype(np.float32)
    act = (rng.random(N) < 0.85).astype(np.uint8)
    cuts = np.sort(rng.choice(np.arange(1, N), 60, replace=False))
    offsets = np.concatenate([[0, 0, 1, 2], cuts, [N, N]])
    print(f"[case] segments random N={N} S={len(offsets) - 1}", flush=True)
    _check(d, act, offsets)


def test_heavy_ties_and_one_big_segment():
    rng = np.random.default_rng(5)
    N = 100003
    d = rng.choice(np.array([0.0, 1e-3, -1e-3, 2.5e-2, -0.7], np.float32), N)
    act = np.ones(N, np.uint8)
    print("[case] segments ties N=100003", flush=True)
    _check(d, act, np.array([0, N]))
    _check(d, act, np.array([0, 50000, 50001, N]), eps_lo=0.1, eps_hi=0.3)


def test_statuses_per_segment():
    from train_rollout_logprob_amd import binding as B
    rng = np.random.default_rng(2)
    N = 5000
    d = (rng.standard_normal(N) * 1e-3).astype(np.float32)
    act = np.ones(N, np.uint8)
    d[1234] = np.nan
    act[3000:4000] = 0
    got, want = _check(d, act, np.array([0, 1000, 2000, 3000, 4000, N]))
    assert status_name(got[1]["status"]) == "ENONFINITE" and got[1]["n_nonfinite"] == 1
    assert status_name(got[3]["status"]) == "ENOACTIVE"
    assert status_name(got[0]["status"]) == "OK"
    # bounds outside [0, N] or decreasing offsets: EMASK for that segment only
    bad = _segments(d, act, np.array([0, 100, 50, N + 7]))
    assert [status_name(s["status"]) for s in bad] == ["OK", "EMASK", "EMASK"]


def test_per_sequence_and_per_row_on_scored_batches():
    """Segments of real pipelines: packed sequences by cu_seqlens and left-padded batch rows
    by b*L, on the GPU's own dlogp; the logprob status is folded into every segment."""
    for spec, seg in ((dict(name="packed", nseq=7, len_lo=30, len_hi=400, V=3001), "cu"),
                      (dict(name="qwen8b", B=3, L=96), "rows")):
        case = make_small(spec)
        got = run_library(case)
        offs = case.cu_seqlens if seg == "cu" else np.arange(case.B + 1) * case.L
        print(f"[case] segments {spec['name']} by {seg}: S={len(offs) - 1}", flush=True)
        g, w = _check(got["dlogp"], got["active"], offs, case.eps_low, case.eps_high)
        assert sum(s["n_active"] for s in g) == int(got["active"].sum())
        # the same offsets through the logprob workspace of a failed call
        bad = case.ids.copy()
        r0 = int(np.nonzero(got["active"])[0][0])
        bad[r0] = case.V + 1
        case.ids = bad
        failed = run_library(case)
        st = _segments(failed["dlogp"], failed["active"], offs, logprob_ws=failed["ws"])
        assert all(status_name(s["status"]) == "ETOKEN" for s in st)


def test_report_has_metrics_segments_and_metadata():
    from train_rollout_logprob_amd import binding as B
    case = make_small(dict(name="packed", nseq=4, len_lo=30, len_hi=200, V=3001))
    got = run_library(case)
    st, stats = B.diagnostics(got["d_dev"], got["a_dev"])
    segs = B.segment_diagnostics(got["d_dev"], got["a_dev"],
                                 torch.as_tensor(case.cu_seqlens, device="cuda"))
    rep = B.report(stats, segs, dtype=case.dtype, padding_side=case.layout,
                   parallelism="single GPU", cache_mode="none")
    import json
    text = json.dumps(rep)
    assert rep["metrics"]["mismatch_kl"] == -stats["mean_dlogp"]
    assert rep["mismatch_k3_kl"] == stats["approx_kl0"]
    assert len(rep["segments"]) == 4 and "build_fingerprint" in text
    assert rep["counts"]["n_active"] == sum(s["n_active"] for s in rep["segments"])


@pytest.mark.slow
def test_full_size_packed_per_sequence():
    """The packed fp32 workload (256 sequences, V=32000): per-sequence statistics of the
    GPU's dlogp against the oracle's, every segment."""
    from train_rollout_logprob_amd import binding as B
    case = synth.make_logits_case("packed", device="cuda")
    ids, att, act, cu = device_inputs(case)
    print(f"[case] full packed segments N={case.N}", flush=True)
    t, r, d, a, ws = B.selected_logprob(case.train, case.rollout, ids, att, act, case.layout,
                                        case.B, case.L, cu, check=True)
    segs = B.segment_diagnostics(d, a, cu, case.eps_low, case.eps_high, logprob_ws=ws)
    want = oracle.segment_diagnostics(d.cpu().numpy(), a.cpu().numpy(), case.cu_seqlens,
                                      case.eps_low, case.eps_high)
    for g, w in zip(segs, want):
        assert status_name(g["status"]) == w["status"]
        if w["status"] == "OK":
            assert_stats_exact(g, w)
    del case, t, r, d, a, ws
    torch.cuda.empty_cache()
