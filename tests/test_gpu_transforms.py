"""GPU parity of the vocab-padding mask and the per-side logit transform chains
("[WS2] Framework for ablation experiment", LogProb knobs rows 2 and 7) against the
fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import (LOGP_TOL, assert_logprob_parity, device_inputs, host_logits, make_small,
                     run_library, status_name)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _oracle(case, vocab_real=None, transforms=(None, None), ids=None):
    return oracle.selected_logprob(host_logits(case.train), host_logits(case.rollout), case.dtype,
                                   case.ids if ids is None else ids, case.attention, case.action,
                                   case.V, case.layout, case.B, case.L, case.cu_seqlens,
                                   vocab_real=vocab_real, transforms=transforms)


CHAINS = {
    "temperature": ([("temperature", 0.7)], [("temperature", 0.7)]),
    "scale": ([("scale", 1.3)], [("scale", 1.3)]),
    "softcap": ([("softcap", 15.0)], [("softcap", 15.0)]),
    "chain3": ([("scale", 2.0), ("softcap", 30.0), ("temperature", 1.5)],
               [("scale", 2.0), ("softcap", 30.0), ("temperature", 1.5)]),
    "per_side": (None, [("temperature", 0.9)]),
    "order_swapped": ([("scale", 3.0), ("softcap", 10.0)], [("softcap", 10.0), ("scale", 3.0)]),
    # saturating soft-cap: most logits end near +-5 (the folded form's g near 0 and 1)
    "softcap_saturating": ([("scale", 8.0), ("softcap", 5.0)], [("scale", 8.0), ("softcap", 5.0)]),
    # a cap above the folded form's bound, and two soft-cap steps: the step-by-step chain
    "softcap_wide": ([("softcap", 60.0)], [("softcap", 60.0)]),
    "two_softcaps": ([("softcap", 30.0), ("softcap", 20.0)], [("softcap", 25.0)]),
}


@pytest.mark.parametrize("spec", [dict(name="qwen8b", B=2, L=48), dict(name="packed", nseq=3,
                                  len_lo=40, len_hi=90, V=3001)], ids=["bf16", "f32_ragged"])
@pytest.mark.parametrize("chain", list(CHAINS))
def test_transform_chain_parity(spec, chain):
    case = make_small(spec)
    tr = CHAINS[chain]
    print(f"[case] {spec['name']} chain={chain}", flush=True)
    got = run_library(case, transforms=tr)
    want = _oracle(case, transforms=tr)
    assert status_name(got["status"]) == want["status"] == "OK"
    assert_logprob_parity(got, want)


def test_identity_chain_is_bitwise_the_plain_path():
    case = make_small(dict(name="qwen8b", B=2, L=48))
    plain = run_library(case)
    ident = run_library(case, transforms=([("scale", 1.0)], [("temperature", 1.0)]))
    for k in ("train_logp", "rollout_logp", "dlogp"):
        assert np.array_equal(plain[k].view(np.uint32), ident[k].view(np.uint32)), k


@pytest.mark.parametrize("dtype_spec", [dict(name="qwen8b", B=2, L=32, V=1000),
                                        dict(name="tiny", B=2, L=32, V=1003, prompt=8)])
def test_vocab_mask(dtype_spec):
    case = make_small(dtype_spec)
    Vr = case.V - 63
    ids = case.ids % Vr
    case.ids = ids.astype(np.int32)
    # make the padded columns large so that "include" and "mask" differ a lot
    case.train[:, Vr:] = 20.0
    case.rollout[:, Vr:] = 20.0
    got = run_library(case, vocab_real=Vr)
    want = _oracle(case, vocab_real=Vr)
    assert status_name(got["status"]) == want["status"] == "OK"
    assert_logprob_parity(got, want)
    both = run_library(case, vocab_real=Vr, transforms=([("softcap", 12.0)], None))
    want2 = _oracle(case, vocab_real=Vr, transforms=([("softcap", 12.0)], None))
    assert_logprob_parity(both, want2)
    # an active selected id inside the padded columns is a token error
    bad = case.ids.copy()
    r0 = int(np.nonzero(got["active"])[0][0])
    bad[r0] = Vr + 5
    case.ids = bad
    st = run_library(case, vocab_real=Vr)
    assert status_name(st["status"]) == _oracle(case, vocab_real=Vr)["status"] == "ETOKEN"
    assert st["first_bad"] == r0


def test_transforms_keep_batch_composition_invariance():
    from train_rollout_logprob_amd import binding as B
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    V = 151936
    pool = torch.randn((20, V), generator=g, device="cuda").mul_(3).to(torch.bfloat16)
    ids = torch.randint(0, V, (20,), generator=g, device="cuda", dtype=torch.int32)
    tr = ([("softcap", 30.0), ("temperature", 0.8)], [("temperature", 0.8)])
    ref = None
    for bs, slot in ((1, 0), (9, 4), (20, 13)):
        rows = torch.arange(bs, device="cuda") % 20
        rows[slot] = 3
        t, r, d, a, ws = B.selected_logprob(pool[rows], pool[rows], ids[rows], layout="right",
                                            batch=1, seq_len=bs, check=True, transforms=tr)
        v = np.array([t[slot].item(), r[slot].item(), d[slot].item()], np.float32)
        if ref is None:
            ref = v
        assert np.array_equal(v.view(np.uint32), ref.view(np.uint32)), bs


@pytest.mark.parametrize("chain", [[("softcap", 15.0)], [("scale", 2.0), ("softcap", 40.0)],
                                   [("softcap", 60.0)]], ids=["folded", "folded_scaled",
                                                              "step_by_step"])
def test_softcap_of_infinite_logits(chain):
    """A soft-cap maps +-inf logits to +-cap: rows with infinite logits (the selected one
    among them) stay finite and match the oracle; a NaN logit still fails the row closed
    (ENONFINITE) and leaves the other rows' values unchanged."""
    from train_rollout_logprob_amd import binding as B
    V, N = 3001, 5
    g = torch.Generator(device="cuda")
    g.manual_seed(21)
    x = torch.randn((N, V), generator=g, device="cuda") * 4
    ids = torch.tensor([7, 100, 3000, 0, 1234], dtype=torch.int32, device="cuda")
    x[0, 50:60] = math.inf
    x[1, :2500] = -math.inf
    x[2, 3000] = math.inf                   # the selected logit, in the ragged last group
    x[3, 0] = -math.inf                     # the selected logit
    tr = (chain, chain)
    t, r, d, a, ws = B.selected_logprob(x, x, ids, layout="right", batch=1, seq_len=N,
                                        check=True, transforms=tr)
    want = oracle.score_rows(x.cpu().numpy(), x.cpu().numpy(), "f32", ids.cpu().numpy(),
                             transforms=tr)[0]
    got = t.double().cpu().numpy()
    assert np.all(np.isfinite(want)) and np.abs(got - want).max() <= LOGP_TOL, (got, want)
    y = x.clone()
    y[4, 17] = math.nan
    t2, r2, d2, a2, ws2 = B.selected_logprob(y, y, ids, layout="right", batch=1, seq_len=N,
                                             transforms=tr)
    st, bad = B.drift_get_status(ws2)
    assert status_name(st) == "ENONFINITE" and bad == 4
    assert math.isnan(t2[4].item())
    assert np.array_equal(t2[:4].cpu().numpy().view(np.uint32), t[:4].cpu().numpy().view(np.uint32))
