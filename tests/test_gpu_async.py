"""drift_diagnostics_async (no synchronization; statistics written by the device to device
memory or pinned host memory) against drift_diagnostics on the same inputs, through the C
ABI: bitwise the same statistics on both selection paths, for both kinds of output memory,
with a logprob status folded in; and the pipelined ScoringStep (submit / collect, the
diagnostics on a stream of their own) against its synchronizing run()."""
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


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _batch(n, seed, tail):
    rng = np.random.default_rng(seed)
    d = rng.standard_t(2, n) * tail if tail else rng.normal(0.0, 1e-3, n)
    a = (rng.random(n) < 0.8).astype(np.uint8)
    return (torch.as_tensor(d.astype(np.float32), device="cuda"),
            torch.as_tensor(a, device="cuda"))


@pytest.mark.parametrize("where", ["device", "pinned"])
def test_async_matches_diagnostics(where):
    from train_rollout_logprob_amd import binding as B
    import ctypes
    sz = ctypes.sizeof(B.drift_stats)
    if where == "device":
        out = torch.empty(sz, dtype=torch.uint8, device="cuda")
    else:
        out = torch.empty(sz, dtype=torch.uint8, pin_memory=True)
    # 300001 and 70001 rows take the multi-block digit path, 4099 the single-block one
    for n, seed, tail in ((300001, 1, 0.05), (4099, 2, 0.0), (70001, 3, 0.3), (1, 5, 0.0)):
        print(f"[case] async {where} n={n} seed={seed}", flush=True)
        d, a = _batch(n, seed, tail)
        a[0] = 1
        st, want = B.diagnostics(d, a, 0.2, 0.2)
        assert st == want["status"]
        out.fill_(0xAB)
        B.diagnostics_async(d, a, out, 0.2, 0.2)
        torch.cuda.synchronize()
        _same(B.stats_from(out), want)


def test_async_empty_and_status_cases():
    from train_rollout_logprob_amd import binding as B
    import ctypes
    out = torch.empty(ctypes.sizeof(B.drift_stats), dtype=torch.uint8, pin_memory=True)
    d, a = _batch(1000, 4, 0.0)
    a.zero_()
    st, want = B.diagnostics(d, a, 0.2, 0.2)
    assert st == B.DRIFT_ENOACTIVE
    B.diagnostics_async(d, a, out, 0.2, 0.2)
    torch.cuda.synchronize()
    _same(B.stats_from(out), want)
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    eb = torch.empty(0, dtype=torch.uint8, device="cuda")
    st, want = B.diagnostics(e, eb, 0.2, 0.2)
    B.diagnostics_async(e, eb, out, 0.2, 0.2)
    torch.cuda.synchronize()
    _same(B.stats_from(out), want)
    # a scoring call whose action mask marks a padded row: its status outranks the stats'
    x = torch.randn((8, 64), device="cuda")
    ids = torch.zeros(8, dtype=torch.int32, device="cuda")
    att = torch.tensor([1, 1, 1, 0, 1, 1, 1, 1], dtype=torch.uint8, device="cuda")
    act = torch.tensor([0, 1, 1, 1, 0, 1, 1, 1], dtype=torch.uint8, device="cuda")
    t, r, dd, aa, ws = B.selected_logprob(x, x, ids, att, act, "right", 2, 4)
    st, want = B.diagnostics(dd, aa, 0.2, 0.2, logprob_ws=ws)
    assert st == B.DRIFT_EMASK
    B.diagnostics_async(dd, aa, out, 0.2, 0.2, logprob_ws=ws)
    torch.cuda.synchronize()
    _same(B.stats_from(out), want)


def test_pipelined_steps_match_run():
    """Three steps submitted two deep (each collected after the next is launched) give the
    statistics of the synchronizing run(), bitwise, in every slot."""
    from helpers import make_small, device_inputs
    from train_rollout_logprob_amd import binding as B
    case = make_small(dict(name="large", B=4, L=64))
    ids, att, act, cu = device_inputs(case)
    step = B.ScoringStep(case.train, case.rollout, ids, att, act, case.layout, case.B, case.L,
                         cu, case.eps_low, case.eps_high, depth=2)
    assert step.run() == B.DRIFT_OK
    want = step.stats.as_dict()
    prev = step.submit()
    for _ in range(3):
        cur = step.submit()
        assert step.collect(prev) == B.DRIFT_OK
        _same(step.stats_of(prev).as_dict(), want)
        prev = cur
    assert step.collect(prev) == B.DRIFT_OK
    _same(step.stats_of(prev).as_dict(), want)
    with pytest.raises(RuntimeError):   # collected already
        step.collect(prev)
    a, b = step.submit(), step.submit()
    with pytest.raises(RuntimeError):   # a third outstanding step in two slots
        step.submit()
    for k in (a, b):
        assert step.collect(k) == B.DRIFT_OK
        _same(step.stats_of(k).as_dict(), want)


@pytest.mark.parametrize("overlap", [True, False], ids=["two_streams", "one_stream"])
@pytest.mark.parametrize("spec", [dict(name="qwen8b", B=3, L=96),
                                  dict(name="large", B=4, L=20000, V=8, prompt=4)],
                         ids=["qwen8b_small", "large_V8_80000_rows"])
def test_pipelined_steps_on_changing_inputs(spec, overlap):
    """Each step scores new logits (written in place on the step's stream after the previous
    submit) while the previous step's diagnostics run on the diagnostics stream (or after
    it on the step's own stream): every slot's statistics and per-row outputs are bitwise
    those of a synchronizing run() on the same logits; once with the single-block selection
    and once above 65536 rows."""
    from helpers import make_small, device_inputs
    from train_rollout_logprob_amd import binding as B
    print(f"[case] pipelined changing inputs {spec} overlap={overlap}", flush=True)
    case = make_small(spec)
    ids, att, act, cu = device_inputs(case)
    train = case.train.clone()
    gen = torch.Generator(device="cuda").manual_seed(11)
    variants = [(case.train.float() + torch.randn(train.shape, generator=gen, device="cuda")
                 * (0.02 * k)).to(train.dtype) for k in range(5)]
    mk = lambda: B.ScoringStep(train, case.rollout, ids, att, act, case.layout, case.B, case.L,
                               cu, case.eps_low, case.eps_high, overlap=overlap)
    ref, step = mk(), mk()
    assert step.overlap == overlap
    want = []
    for v in variants:
        train.copy_(v)
        assert ref.run() == B.DRIFT_OK
        want.append((ref.stats.as_dict(), [x.clone() for x in ref.out]))
    assert len({w[0]["max_abs_dlogp"] for w in want}) == len(variants)  # the steps differ
    prev = None
    for k, v in enumerate(variants):
        train.copy_(v)          # ordered after the previous step's scoring on this stream
        cur = step.submit()
        if prev is not None:
            assert step.collect(prev[0]) == B.DRIFT_OK
            _same(step.stats_of(prev[0]).as_dict(), want[prev[1]][0])
            for g, w in zip(step.out_of(prev[0]), want[prev[1]][1]):
                assert torch.equal(_bits(g), _bits(w))
        prev = (cur, k)
    assert step.collect(prev[0]) == B.DRIFT_OK
    _same(step.stats_of(prev[0]).as_dict(), want[prev[1]][0])
    if case.N > 65536:
        assert step.N > 65536
