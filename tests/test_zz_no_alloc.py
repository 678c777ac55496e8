"""drift_diagnostics_noalloc (no workspace argument, statistics written to device memory)
against drift_diagnostics on the same inputs, through the C ABI: bitwise the same
statistics on two calls in a row, the second with a smaller batch (the library's scratch
keeps the first call's contents), then an empty batch and a batch whose scoring call
recorded a logical-input error."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _same(got, want):
    assert set(got) == set(want)
    for k, w in want.items():
        g = got[k]
        if isinstance(w, float):
            assert np.float64(g).tobytes() == np.float64(w).tobytes(), (k, g, w)
        else:
            assert g == w, (k, g, w)


def _batch(n, seed, tail):
    rng = np.random.default_rng(seed)
    d = rng.standard_t(2, n) * tail if tail else rng.normal(0.0, 1e-3, n)
    a = (rng.random(n) < 0.8).astype(np.uint8)
    return (torch.as_tensor(d.astype(np.float32), device="cuda"),
            torch.as_tensor(a, device="cuda"))


def test_noalloc_matches_diagnostics_on_consecutive_calls():
    from train_rollout_logprob_amd import binding as B
    out = torch.empty(128, dtype=torch.uint8, device="cuda")
    # the larger batch takes the multi-block digit path, the smaller the single-block one
    for n, seed, tail in ((300001, 1, 0.05), (4099, 2, 0.0), (70001, 3, 0.3)):
        print(f"[case] noalloc n={n} seed={seed}", flush=True)
        d, a = _batch(n, seed, tail)
        st, want = B.diagnostics(d, a, 0.2, 0.2)
        assert st == B.DRIFT_OK and want["status"] == B.DRIFT_OK
        got, _ = B.diagnostics_noalloc(d, a, 0.2, 0.2, out=out)
        _same(got, want)
        # the same call again, now that the scratch holds this batch's own state
        got2, _ = B.diagnostics_noalloc(d, a, 0.2, 0.2, out=out)
        _same(got2, want)


def test_noalloc_empty_and_status_cases():
    from train_rollout_logprob_amd import binding as B
    d, a = _batch(1000, 4, 0.0)
    a.zero_()
    st, want = B.diagnostics(d, a, 0.2, 0.2)
    assert st == B.DRIFT_ENOACTIVE
    got, _ = B.diagnostics_noalloc(d, a, 0.2, 0.2)
    _same(got, want)
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    eb = torch.empty(0, dtype=torch.uint8, device="cuda")
    st, want = B.diagnostics(e, eb, 0.2, 0.2)
    got, _ = B.diagnostics_noalloc(e, eb, 0.2, 0.2)
    _same(got, want)
    # a scoring call whose action mask marks a padded row: its status outranks the stats'
    x = torch.randn((8, 64), device="cuda")
    ids = torch.zeros(8, dtype=torch.int32, device="cuda")
    att = torch.tensor([1, 1, 1, 0, 1, 1, 1, 1], dtype=torch.uint8, device="cuda")
    act = torch.tensor([0, 1, 1, 1, 0, 1, 1, 1], dtype=torch.uint8, device="cuda")
    t, r, dd, aa, ws = B.selected_logprob(x, x, ids, att, act, "right", 2, 4)
    st, want = B.diagnostics(dd, aa, 0.2, 0.2, logprob_ws=ws)
    assert st == B.DRIFT_EMASK
    got, _ = B.diagnostics_noalloc(dd, aa, 0.2, 0.2, logprob_ws=ws)
    _same(got, want)


def test_noalloc_rejects_batches_beyond_its_scratch():
    from train_rollout_logprob_amd import binding as B
    n = B.DRIFT_NOALLOC_MAX_ROWS + 1
    d = torch.zeros(n, dtype=torch.float32, device="cuda")
    a = torch.zeros(n, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.DriftError):
        B.diagnostics_noalloc(d, a, 0.2, 0.2)
