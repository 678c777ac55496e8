"""GPU parity of drift_lmhead_logprob (fused hidden x W_vocab + log-softmax gather)
against the fp64 oracle, and the batch-composition bitwise control: the same rows
re-scored inside batches of 1, 7 and 64 rows give bitwise the full-batch result."""
import numpy as np
import pytest
import torch

import oracle
from helpers import LOGP_TOL, status_name
from train_rollout_logprob_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _oracle(case, rows, transforms=None):
    w64 = oracle.widen(_bits(case.weight), "bf16").reshape(case.H, case.V)
    return oracle.lmhead_logprob(_bits(case.hidden), w64, case.ids, rows=rows,
                                 transforms=transforms)


# The last two shapes span hundreds of tiles (more than one per compute unit) with ragged
# token and vocabulary edges, with an even (H=256: 4 stages of 64) and an odd (H=320: 5)
# number of K stages.
@pytest.mark.parametrize("T,H,V", [(300, 264, 1000), (128, 64, 128), (1, 8, 8), (77, 520, 4104),
                                   (2000, 256, 20008), (1537, 320, 20000)])
def test_parity_ragged_shapes(T, H, V):
    from train_rollout_logprob_amd import binding as B
    print(f"[case] lmhead T={T} H={H} V={V}", flush=True)
    case = synth.make_lmhead_case(device="cuda", T=T, H=H, V=V)
    ids = torch.as_tensor(case.ids, device="cuda")
    logp, ws = B.lmhead_logprob(case.hidden, case.weight, ids, check=True)
    want = _oracle(case, None)
    err = np.abs(logp.cpu().numpy().astype(np.float64) - want)
    print(f"[case] max err {err.max():.3e}", flush=True)
    assert err.max() <= LOGP_TOL
    # the weight as [V, H] (read in place when H % 64 == 0, else copied with K padding):
    # the same products in the same K order, so bitwise the [H, V] result
    w_vh = case.weight.t().contiguous()
    logp_vh, _ = B.lmhead_logprob(case.hidden, w_vh, ids, check=True, weight_layout="vh")
    assert torch.equal(logp_vh.view(torch.int32), logp.view(torch.int32))


def test_active_mask_and_token_errors():
    from train_rollout_logprob_amd import binding as B
    case = synth.make_lmhead_case(device="cuda", T=200, H=128, V=512)
    ids = torch.as_tensor(case.ids, device="cuda")
    act = torch.ones(200, dtype=torch.uint8, device="cuda")
    act[::3] = 0
    logp, ws = B.lmhead_logprob(case.hidden, case.weight, ids, act, check=True)
    base, _ = B.lmhead_logprob(case.hidden, case.weight, ids)
    a = act.cpu().numpy() == 1
    assert np.all(logp.cpu().numpy()[~a] == 0.0)
    assert np.array_equal(logp.cpu().numpy()[a], base.cpu().numpy()[a])
    bad = ids.clone()
    bad[5] = 512
    logp, ws = B.lmhead_logprob(case.hidden, case.weight, bad)
    st, row = B.drift_get_status(ws)
    assert status_name(st) == "ETOKEN" and row == 5
    assert np.isnan(logp[5].item())
    bad[5] = -100
    act[5] = 0                                       # an inactive row is never checked
    logp, ws = B.lmhead_logprob(case.hidden, case.weight, bad, act, check=True)


def test_batch_composition_control_is_bitwise_zero():
    """Rows scored in the full batch, then inside batches of 1, 7 and 64 rows at other
    positions (other rows drawn from the pool), are bitwise equal: dlogp == 0 exactly."""
    from train_rollout_logprob_amd import binding as B
    T, H, V = 2048, 1024, 16384
    case = synth.make_lmhead_case(device="cuda", T=T, H=H, V=V)
    ids = torch.as_tensor(case.ids, device="cuda")
    full, _ = B.lmhead_logprob(case.hidden, case.weight, ids, check=True)
    full = full.cpu().numpy()
    rng = np.random.default_rng(11)
    probe = [0, 5, 1000, T - 1]
    for bs in (1, 7, 64):
        for pr in probe:
            rows = rng.integers(0, T, bs)
            slot = int(rng.integers(0, bs))
            rows[slot] = pr
            idx = torch.as_tensor(rows, device="cuda")
            h = case.hidden.index_select(0, idx).contiguous()
            got, _ = B.lmhead_logprob(h, case.weight, ids.index_select(0, idx).contiguous(),
                                      check=True)
            g = np.float32(got[slot].item())
            assert g.view(np.uint32) == full[pr].view(np.uint32), (bs, pr, g, full[pr])


@pytest.mark.slow
def test_full_size_every_row_and_invariance():
    """T=16384, H=4096, V=151936 as timed: every row against the oracle (fp64 products of
    the bf16 inputs, in chunks of 2048 rows), the whole batch with the weight given as
    [V, H] bitwise equal to the [H, V] call, and four rows (including the first and the
    last) re-scored in batches of 1, 7 and 64."""
    from train_rollout_logprob_amd import binding as B
    case = synth.make_lmhead_case(device="cuda")
    ids = torch.as_tensor(case.ids, device="cuda")
    logp, ws = B.lmhead_logprob(case.hidden, case.weight, ids, check=True)
    full = logp.cpu().numpy()
    w64 = oracle.widen(_bits(case.weight), "bf16").reshape(case.H, case.V)
    hb = _bits(case.hidden)
    worst = 0.0
    for a in range(0, case.T, 2048):
        rows = np.arange(a, min(a + 2048, case.T))
        want = oracle.lmhead_logprob(hb, w64, case.ids, rows=rows)
        err = np.abs(full[rows].astype(np.float64) - want)
        worst = max(worst, float(err.max()))
        print(f"[case] lmhead full rows {a}..{rows[-1]}: max err {err.max():.3e}", flush=True)
        assert err.max() <= LOGP_TOL, (a, float(err.max()))
    print(f"[case] lmhead full max err {worst:.3e} over all {case.T} rows", flush=True)
    del w64
    rng = np.random.default_rng(12)
    w_vh = case.weight.t().contiguous()
    logp_vh, _ = B.lmhead_logprob(case.hidden, w_vh, ids, check=True, weight_layout="vh")
    assert torch.equal(logp_vh.view(torch.int32), logp.view(torch.int32))
    del w_vh, logp_vh
    probe = [0, 1234, 9999, case.T - 1]
    for bs in (1, 7, 64):
        for pr in probe:
            rr = rng.integers(0, case.T, bs)
            slot = int(rng.integers(0, bs))
            rr[slot] = pr
            idx = torch.as_tensor(rr, device="cuda")
            got, _ = B.lmhead_logprob(case.hidden.index_select(0, idx).contiguous(),
                                      case.weight, ids.index_select(0, idx).contiguous(),
                                      check=True)
            g = np.float32(got[slot].item())
            assert g.view(np.uint32) == full[pr].view(np.uint32), (bs, pr)


# chains on the head's logits (all fold: at most one soft-cap, |cap x later factors| <= 40)
HEAD_CHAINS = {
    "softcap30": [("softcap", 30.0)],
    "temp_softcap": [("temperature", 0.7), ("softcap", 15.0)],
    "scale_neg_softcap": [("scale", -1.5), ("softcap", 10.0), ("scale", 2.0)],
    # a multiplying chain only (on these scaled weights, a temperature above 1 keeps the
    # logits at a few units; the fp32 GEMM's own error grows with their size)
    "temperature": [("temperature", 2.0)],
}


@pytest.mark.parametrize("chain", list(HEAD_CHAINS))
@pytest.mark.parametrize("T,H,V", [(300, 264, 1000), (77, 520, 4104), (2000, 256, 20008)])
def test_chain_parity_ragged_shapes(T, H, V, chain):
    """drift_lmhead_logprob_chain against the oracle's head with the same chain, for both
    weight layouts (bitwise the same results), with ragged token and vocabulary edges."""
    from train_rollout_logprob_amd import binding as B
    print(f"[case] lmhead chain={chain} T={T} H={H} V={V}", flush=True)
    case = synth.make_lmhead_case(device="cuda", T=T, H=H, V=V)
    # logits of a few units, so that the caps bite
    case.weight.mul_(20.0)
    ids = torch.as_tensor(case.ids, device="cuda")
    tr = HEAD_CHAINS[chain]
    logp, ws = B.lmhead_logprob(case.hidden, case.weight, ids, check=True, transforms=tr)
    want = _oracle(case, None, tr)
    err = np.abs(logp.cpu().numpy().astype(np.float64) - want)
    print(f"[case] max err {err.max():.3e}", flush=True)
    assert err.max() <= LOGP_TOL
    w_vh = case.weight.t().contiguous()
    logp_vh, _ = B.lmhead_logprob(case.hidden, w_vh, ids, check=True, weight_layout="vh",
                                  transforms=tr)
    assert torch.equal(logp_vh.view(torch.int32), logp.view(torch.int32))


def test_identity_chain_is_bitwise_the_plain_head():
    from train_rollout_logprob_amd import binding as B
    case = synth.make_lmhead_case(device="cuda", T=300, H=264, V=1000)
    ids = torch.as_tensor(case.ids, device="cuda")
    plain, _ = B.lmhead_logprob(case.hidden, case.weight, ids, check=True)
    for tr in ([("scale", 1.0)], [("temperature", 1.0)]):
        got, _ = B.lmhead_logprob(case.hidden, case.weight, ids, check=True, transforms=tr)
        assert torch.equal(got.view(torch.int32), plain.view(torch.int32)), tr


def test_chain_refused_when_it_does_not_fold():
    from train_rollout_logprob_amd import binding as B
    case = synth.make_lmhead_case(device="cuda", T=16, H=64, V=256)
    ids = torch.as_tensor(case.ids, device="cuda")
    for tr in ([("softcap", 30.0), ("softcap", 20.0)], [("softcap", 50.0)]):
        with pytest.raises(B.DriftError):
            B.lmhead_logprob(case.hidden, case.weight, ids, transforms=tr)


def test_chain_batch_composition_control_is_bitwise_zero():
    """With a soft-cap on the logits, rows re-scored in batches of 1, 7 and 64 at other
    positions are bitwise equal to the full batch."""
    from train_rollout_logprob_amd import binding as B
    T, H, V = 2048, 1024, 16384
    case = synth.make_lmhead_case(device="cuda", T=T, H=H, V=V)
    case.weight.mul_(20.0)
    ids = torch.as_tensor(case.ids, device="cuda")
    tr = [("softcap", 30.0)]
    full, _ = B.lmhead_logprob(case.hidden, case.weight, ids, check=True, transforms=tr)
    full = full.cpu().numpy()
    rng = np.random.default_rng(13)
    for bs in (1, 7, 64):
        for pr in (0, 5, 1000, T - 1):
            rows = rng.integers(0, T, bs)
            slot = int(rng.integers(0, bs))
            rows[slot] = pr
            idx = torch.as_tensor(rows, device="cuda")
            got, _ = B.lmhead_logprob(case.hidden.index_select(0, idx).contiguous(),
                                      case.weight, ids.index_select(0, idx).contiguous(),
                                      check=True, transforms=tr)
            g = np.float32(got[slot].item())
            assert g.view(np.uint32) == full[pr].view(np.uint32), (bs, pr)


@pytest.mark.slow
def test_full_size_chain_every_row():
    """The timed head shape with a soft-cap of 10 on logits scaled to a few units (std 6.4):
    every row against the oracle, in chunks of 2048 rows."""
    from train_rollout_logprob_amd import binding as B
    case = synth.make_lmhead_case(device="cuda")
    case.weight.mul_(5.0)
    ids = torch.as_tensor(case.ids, device="cuda")
    tr = [("softcap", 10.0)]
    logp, ws = B.lmhead_logprob(case.hidden, case.weight, ids, check=True, transforms=tr)
    full = logp.cpu().numpy()
    w64 = oracle.widen(_bits(case.weight), "bf16").reshape(case.H, case.V)
    hb = _bits(case.hidden)
    worst = 0.0
    for a in range(0, case.T, 2048):
        rows = np.arange(a, min(a + 2048, case.T))
        want = oracle.lmhead_logprob(hb, w64, case.ids, rows=rows, transforms=tr)
        err = np.abs(full[rows].astype(np.float64) - want)
        worst = max(worst, float(err.max()))
        assert err.max() <= LOGP_TOL, (a, float(err.max()))
    print(f"[case] lmhead chain full max err {worst:.3e} over all {case.T} rows", flush=True)
