"""Full-size workloads on the GPU, in the launch configuration the benchmark times:
sampled rows against the fp64 oracle (first, last and random active rows), and the
diagnostics of the whole GPU dlogp array against the oracle's diagnostics of the same
array (exact counts and order statistics)."""
import numpy as np
import pytest
import torch

import oracle
from helpers import LOGP_TOL, assert_stats_exact, device_inputs, status_name
from train_rollout_logprob_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


@pytest.mark.parametrize("name", ["tiny", "qwen8b", "packed", "large"])
def test_full_size_workload(name):
    from train_rollout_logprob_amd import binding as B
    print(f"[case] full {name}: generating", flush=True)
    case = synth.make_logits_case(name, device="cuda")
    ids, att, act, cu = device_inputs(case)
    print(f"[case] full {name}: N={case.N} V={case.V} n_active={case.n_active()}", flush=True)
    t, r, d, a, ws = B.selected_logprob(case.train, case.rollout, ids, att, act, case.layout,
                                        case.B, case.L, cu)
    st, s = B.diagnostics(d, a, case.eps_low, case.eps_high, logprob_ws=ws)
    assert status_name(st) == "OK"
    a_h = a.cpu().numpy()
    want_active = oracle.active_rows(case.attention, case.action, case.N, case.layout,
                                     case.cu_seqlens).astype(np.uint8)
    assert np.array_equal(a_h, want_active)
    assert s["n_active"] == case.n_active()
    rows = np.nonzero(a_h)[0]
    rng = np.random.default_rng(17)
    k = min(len(rows), 48)
    sample = np.unique(np.concatenate([rows[:2], rows[-2:], rng.choice(rows, k, replace=False)]))
    tr = synth.rows_to_host(case.train, sample)
    ro = synth.rows_to_host(case.rollout, sample)
    ot, orr, od = oracle.score_rows(tr, ro, case.dtype, case.ids[sample])
    th, rh, dh = (x.cpu().numpy().astype(np.float64)[sample] for x in (t, r, d))
    for name_, g, w in (("train", th, ot), ("rollout", rh, orr), ("dlogp", dh, od)):
        err = float(np.abs(g - w).max())
        print(f"[case] {name} {name_} max err {err:.3e} over {len(sample)} rows", flush=True)
        assert err <= LOGP_TOL, name_
    d_h = d.cpu().numpy()
    want = oracle.diagnostics(d_h, a_h, case.eps_low, case.eps_high)
    assert_stats_exact(s, want)
    del case, t, r, d, a, ws
    torch.cuda.empty_cache()
