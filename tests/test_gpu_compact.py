"""GPU parity of drift_active_rows (the ascending active-row list) against the oracle's
list, bit-exact: ragged and tile-multiple sizes, empty and full masks, non-0/1 bytes, the
entries past n left untouched, batches on both sides of 1024 tiles of 4096 rows (where the
tiles' offsets move from the scatter blocks to a scan launch), and the list of a scored
batch's `active` output."""
import numpy as np
import pytest
import torch

import oracle
from helpers import device_inputs
from train_rollout_logprob_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


@pytest.mark.parametrize("N", [0, 1, 4095, 4096, 4097, 100003, 270336,
                               4096 * 1024, 4096 * 1024 + 1, 16777216 + 4099])
@pytest.mark.parametrize("p", [0.0, 0.01, 0.5, 1.0])
def test_active_rows_match_the_oracle(N, p):
    from train_rollout_logprob_amd import binding as B
    print(f"[case] active_rows N={N} p={p}", flush=True)
    rng = np.random.default_rng(N * 7 + int(p * 100))
    a = (rng.random(N) < p).astype(np.uint8)
    if N > 3:
        a[a == 1] = rng.choice(np.array([1, 2, 255], np.uint8), int(a.sum()))  # nonzero = active
    act = torch.as_tensor(a, device="cuda")
    rows = torch.full((max(N, 1),), -7, dtype=torch.int32, device="cuda")
    rows, n, _ = B.active_rows(act, rows=rows)
    want = oracle.active_row_list(a)
    got = rows.cpu().numpy()
    assert int(n.item()) == len(want)
    assert np.array_equal(got[:len(want)], want.astype(np.int32))
    assert np.all(got[len(want):] == -7)


@pytest.mark.parametrize("name", ["tiny", "packed_small"])
def test_active_rows_of_a_scored_batch(name):
    from train_rollout_logprob_amd import binding as B
    spec = {"tiny": dict(name="tiny"),
            "packed_small": dict(name="packed", nseq=9, len_lo=40, len_hi=500, V=3001)}[name]
    case = synth.make_logits_case(**spec, device="cuda")
    ids, att, act, cu = device_inputs(case)
    _, _, _, a, _ = B.selected_logprob(case.train, case.rollout, ids, att, act, case.layout,
                                       case.B, case.L, cu)
    rows, n, _ = B.active_rows(a)
    want = oracle.active_row_list(oracle.active_rows(case.attention, case.action, case.N,
                                                     case.layout, case.cu_seqlens))
    assert int(n.item()) == len(want) == case.n_active()
    assert np.array_equal(rows.cpu().numpy()[:len(want)], want.astype(np.int32))
