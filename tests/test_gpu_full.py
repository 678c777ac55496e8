"""Full-size workloads on the GPU, in the launch configuration the benchmark times (and the
Qwen3-8B-shaped batch once more with a soft-cap of 30 on both sides).

Every active row of each scoring workload is compared with the fp64 oracle (the oracle
runs in a pool of host worker processes started before this process touched the GPU):
per-token logp of both sides and dlogp within 2e-5. The diagnostics are checked twice:
Gate A, the library's statistics of its own dlogp array against the oracle's statistics
of the same array (counts, order statistics, argmax and clipfrac0 bit-exact, means to
1e-12 relative); and
Gate B, the library's statistics against the oracle's statistics of the oracle's own fp64
dlogp (means to 1e-5 relative; counts and order statistics as far as the per-token
tolerance decides them)."""
import numpy as np
import pytest
import torch

import oracle
from helpers import (LOGP_TOL, assert_gate_b, assert_stats_exact, device_inputs,
                     oracle_all_rows, oracle_pool, status_name)
from train_rollout_logprob_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


# soft-cap 30 on both sides: the folded log-sum-exp terms of the scoring kernel at full size
CHAIN = {"qwen8b_softcap": [("softcap", 30.0)]}


@pytest.mark.parametrize("name", ["tiny", "qwen8b", "packed", "large", "qwen8b_softcap"])
def test_full_size_every_active_row(name):
    from train_rollout_logprob_amd import binding as B
    pool = oracle_pool()
    if pool is None:
        pytest.skip("the oracle worker pool was not started (no GPU counted at start-up)")
    print(f"[case] full {name}: generating", flush=True)
    chain = CHAIN.get(name)
    tr = (chain, chain)
    case = synth.make_logits_case(name.split("_")[0], device="cuda")
    ids, att, act, cu = device_inputs(case)
    print(f"[case] full {name}: N={case.N} V={case.V} n_active={case.n_active()}", flush=True)
    step = B.ScoringStep(case.train, case.rollout, ids, att, act, case.layout, case.B, case.L,
                         cu, case.eps_low, case.eps_high, transforms=tr)
    st = step.run()
    assert status_name(st) == "OK"
    s = step.stats.as_dict()
    t, r, d, a = step.out
    a_h = a.cpu().numpy()
    want_active = oracle.active_rows(case.attention, case.action, case.N, case.layout,
                                     case.cu_seqlens).astype(np.uint8)
    assert np.array_equal(a_h, want_active)
    assert s["n_active"] == case.n_active()
    rows = np.nonzero(a_h)[0]
    th, rh, dh = (x.cpu().numpy() for x in (t, r, d))
    assert np.all(th[a_h == 0] == 0) and np.all(rh[a_h == 0] == 0) and np.all(dh[a_h == 0] == 0)
    print(f"[case] full {name}: oracle over {len(rows)} rows in {pool.workers} workers",
          flush=True)
    ot, orr, od = oracle_all_rows(pool, case, rows, tr)
    for name_, g, w in (("train", th, ot), ("rollout", rh, orr), ("dlogp", dh, od)):
        err = np.abs(g[rows].astype(np.float64) - w)
        print(f"[case] {name} {name_}: max err {err.max():.3e} (row {rows[int(err.argmax())]}) "
              f"over all {len(rows)} active rows", flush=True)
        assert float(err.max()) <= LOGP_TOL, name_
    # Gate A: the library's statistics of its own array
    assert_stats_exact(s, oracle.diagnostics(dh, a_h, case.eps_low, case.eps_high))
    # Gate B: against the oracle's statistics of its own fp64 dlogp
    d_oracle = np.zeros(case.N)
    d_oracle[rows] = od
    want_b = oracle.diagnostics(d_oracle, a_h, case.eps_low, case.eps_high)
    assert_gate_b(s, want_b, od, case.eps_low, case.eps_high)
    print(f"[case] {name}: gate B ratio0 {s['ratio0']:.12g} vs {want_b['ratio0']:.12g}, "
          f"approx_kl0 {s['approx_kl0']:.6g} vs {want_b['approx_kl0']:.6g}, "
          f"max|d| {s['max_abs_dlogp']:.6g} vs {want_b['max_abs_dlogp']:.6g}", flush=True)
    del step, case, t, r, d, a
    torch.cuda.empty_cache()
