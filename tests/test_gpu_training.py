"""GPU parity of the training-only state of the selected logprob ("[WS2] Framework for
ablation experiment", LogProb knobs row 11): per-row entropy and LSE from the scoring pass,
and drift_dlogits, against the fp64 oracle.

Tolerances. Entropy is the p-weighted mean of -log p_v, each term carrying the error of a
selected logprob, so it takes the logprob bound LOGP_TOL; the exported LSE likewise. A
dlogits element g * dz * ([v == y] - p_v) moves by |g dz| p_v times the error of z_v - LSE
(at most LOGP_TOL), plus the rounding of dz and of the product (2e-6 of |g| S, S the
product of the chain's multiplying factors, a bound of |dz|). Off the selected column that
is |value| * LOGP_TOL; on it |g| S LOGP_TOL. A bf16 output adds half a bf16 ulp (2^-8 of
the value)."""
import numpy as np
import pytest
import torch

import oracle
from helpers import (FULL_CHUNK_BYTES, LOGP_TOL, copy_rows, device_inputs, host_logits,
                     make_small, oracle_pool, run_library, status_name)
from train_rollout_logprob_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


SPECS = {
    "bf16_left": dict(name="qwen8b", B=2, L=48),
    "bf16_ragged_V": dict(name="qwen8b", B=2, L=32, V=1001),
    "f32_right": dict(name="tiny"),
    "f32_packed_ragged": dict(name="packed", nseq=3, len_lo=40, len_hi=90, V=3001),
    "bf16_V8": dict(name="large", B=2, L=16, V=8, prompt=4),
}
CHAINS = {
    "none": (None, None),
    "softcap_temp": ([("softcap", 20.0), ("temperature", 0.8)], [("temperature", 1.25)]),
    "scale_neg": ([("scale", -1.5)], None),
    # chains the folded form does not take (two soft-caps; a cap above 40): step by step,
    # and a folded side beside a step-by-step one
    "softcap_twice": ([("softcap", 30.0), ("softcap", 12.0)], [("softcap", 50.0)]),
    "mixed_forms": ([("softcap", 25.0)], [("softcap", 30.0), ("softcap", 20.0)]),
}


def _chain_gain(chain):
    s = 1.0
    for kind, v in (chain or ()):
        s *= abs(v) if kind == "scale" else 1.0 / v if kind == "temperature" else 1.0
    return s


def _rows(case, side):
    return host_logits(case.train if side == 0 else case.rollout)


def _forward(case, vocab_real=None, transforms=(None, None), entropy=True):
    N = case.N
    ent = tuple(torch.full((N,), -7.0, dtype=torch.float32, device="cuda") for _ in range(2))
    lse = tuple(torch.full((N,), -7.0, dtype=torch.float64, device="cuda") for _ in range(2))
    got = run_library(case, vocab_real=vocab_real, transforms=transforms,
                      entropy=ent if entropy else (None, None), lse=lse)
    got["ent"] = [e.cpu().numpy() for e in ent]
    got["lse"] = [l.cpu().numpy() for l in lse]
    got["lse_dev"] = lse
    return got


@pytest.mark.parametrize("chain", list(CHAINS))
@pytest.mark.parametrize("spec", list(SPECS))
def test_entropy_and_lse_parity(spec, chain):
    case = make_small(SPECS[spec])
    tr = CHAINS[chain]
    Vr = case.V - 5 if case.V > 64 else None
    if Vr is not None:
        case.ids = (case.ids % Vr).astype(np.int32)
    print(f"[case] entropy {spec} chain={chain} Vr={Vr}", flush=True)
    got = _forward(case, vocab_real=Vr, transforms=tr)
    assert status_name(got["status"]) == "OK"
    act = got["active"] == 1
    want_act = oracle.active_rows(case.attention, case.action, case.N, case.layout,
                                  case.cu_seqlens)
    assert np.array_equal(act, want_act.astype(bool))
    for side in (0, 1):
        rows = _rows(case, side)
        idx = np.nonzero(act)[0]
        H = oracle.entropy_rows(rows[idx], case.dtype, vocab_real=Vr, transform=tr[side])
        V_ = case.V if Vr is None else Vr
        L = np.array([oracle.logsumexp_row(oracle.apply_transforms(
            oracle.widen(rows[r, :V_], case.dtype), tr[side])) for r in idx])
        eh = np.abs(got["ent"][side][idx].astype(np.float64) - H)
        el = np.abs(got["lse"][side][idx] - L)
        assert eh.max() <= LOGP_TOL, (side, float(eh.max()))
        assert el.max() <= LOGP_TOL, (side, float(el.max()))
        assert np.all(got["ent"][side][~act] == 0) and np.all(got["lse"][side][~act] == 0)
    # the entropy variant of the kernel leaves the logprob outputs bitwise unchanged
    plain = run_library(case, vocab_real=Vr, transforms=tr)
    for k in ("train_logp", "rollout_logp", "dlogp"):
        assert np.array_equal(plain[k].view(np.uint32), got[k].view(np.uint32)), k


def test_entropy_rejected_rows_are_nan():
    case = make_small(SPECS["f32_right"])
    r0 = int(np.nonzero(case.action)[0][3])
    case.ids = case.ids.copy()
    case.ids[r0] = case.V + 3
    got = _forward(case)
    assert status_name(got["status"]) == "ETOKEN" and got["first_bad"] == r0
    for side in (0, 1):
        assert np.isnan(got["ent"][side][r0]) and np.isnan(got["lse"][side][r0])


def _dlogits_case(spec, chain, out_dtype, with_grad, vocab_real=True, pad=0):
    from train_rollout_logprob_amd import binding as B
    case = make_small(SPECS[spec])
    Vr = case.V - 7 if (vocab_real and case.V > 64) else None
    if Vr is not None:
        case.ids = (case.ids % Vr).astype(np.int32)
    tr = CHAINS[chain]
    got = _forward(case, vocab_real=Vr, transforms=tr, entropy=False)
    assert status_name(got["status"]) == "OK"
    ids, _, _, _ = device_inputs(case)
    g = None
    if with_grad:
        gen = torch.Generator(device="cuda")
        gen.manual_seed(5)
        g = torch.randn(case.N, generator=gen, device="cuda", dtype=torch.float32)
    outs = []
    for side in (0, 1):
        out = torch.full((case.N, case.V + pad), 3.0, dtype=out_dtype, device="cuda")
        B.dlogits(case.train, case.rollout, ids, side, got["lse_dev"][side], got["a_dev"],
                  grad_logp=g, out_dtype=out_dtype, out=out, vocab_real=Vr, transforms=tr)
        outs.append(out.float().cpu().numpy())
    return case, Vr, tr, got, (None if g is None else g.cpu().numpy()), outs


def _check_dlogits(case, Vr, tr, got, g, outs, out_dtype):
    act = got["active"]
    for side in (0, 1):
        want = oracle.dlogits_rows(_rows(case, side), case.dtype, case.ids, act, vocab_real=Vr,
                                   transform=tr[side], grad=g)
        o = outs[side][:, :case.V].astype(np.float64)
        gabs = np.ones(case.N) if g is None else np.abs(g.astype(np.float64))
        base = gabs * _chain_gain(tr[side])                    # bound of |g dz| per row
        # off the selected column |want| = |g dz| p_v, so its error is |want| * LOGP_TOL;
        # on it the error is |g dz| p_y LOGP_TOL <= base * LOGP_TOL
        tol = np.abs(want) * LOGP_TOL + base[:, None] * 2e-6
        on = act == 1
        rows_on = np.nonzero(on)[0]
        tol[rows_on, case.ids[rows_on].astype(np.int64)] += base[rows_on] * LOGP_TOL
        if out_dtype == torch.bfloat16:
            tol = tol + (np.abs(want) + tol) * 2.0 ** -8
        err = np.abs(o - want)
        worst = float((err - tol).max())
        assert worst <= 0.0, (side, worst, float(err.max()))
        assert np.all(o[act == 0] == 0)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("chain", list(CHAINS))
@pytest.mark.parametrize("spec", ["bf16_left", "f32_packed_ragged", "bf16_ragged_V", "bf16_V8"])
def test_dlogits_parity(spec, chain, out_dtype):
    print(f"[case] dlogits {spec} chain={chain} out={out_dtype}", flush=True)
    r = _dlogits_case(spec, chain, out_dtype, with_grad=(chain != "none"))
    _check_dlogits(*r, out_dtype)


def test_dlogits_strided_output_and_rejected_rows():
    """Columns past V in a wider output are left untouched; a rejected id gives NaN on
    [0, vocab_real) and 0 past it; inactive rows are 0."""
    from train_rollout_logprob_amd import binding as B
    case = make_small(SPECS["f32_right"])
    r0 = int(np.nonzero(case.action)[0][2])
    case.ids = case.ids.copy()
    Vr = case.V - 9
    case.ids = (case.ids % Vr).astype(np.int32)
    case.ids[r0] = Vr + 1
    got = _forward(case, vocab_real=Vr, entropy=False)
    assert status_name(got["status"]) == "ETOKEN"
    ids, _, _, _ = device_inputs(case)
    out = torch.full((case.N, case.V + 13), 3.0, dtype=torch.float32, device="cuda")
    B.dlogits(case.train, case.rollout, ids, 0, got["lse_dev"][0], got["a_dev"], out=out,
              vocab_real=Vr)
    o = out.cpu().numpy()
    assert np.all(o[:, case.V:] == 3.0)
    assert np.all(np.isnan(o[r0, :Vr])) and np.all(o[r0, Vr:case.V] == 0)
    assert np.all(o[got["active"] == 0, :case.V] == 0)
    want = oracle.dlogits_rows(_rows(case, 0), case.dtype, case.ids, got["active"],
                               vocab_real=Vr)
    ok = (got["active"] == 1) & (np.arange(case.N) != r0)
    assert np.abs(o[ok, :case.V] - want[ok]).max() <= LOGP_TOL


def test_dlogits_unaligned_rows_take_the_scalar_path():
    """A logits view whose rows start off a 16-byte boundary (one column in) gives bitwise
    the values of the aligned layout (vector path vs element path)."""
    from train_rollout_logprob_amd import binding as B
    case = make_small(SPECS["bf16_left"])
    N, V = case.N, case.V
    wide = torch.zeros((N, V + 1), dtype=case.train.dtype, device="cuda")
    wide[:, 1:] = case.train
    shifted = wide[:, 1:]
    got = _forward(case, entropy=False)
    ids, _, _, _ = device_inputs(case)
    a = B.dlogits(case.train, case.rollout, ids, 0, got["lse_dev"][0], got["a_dev"])
    b = B.dlogits(shifted, shifted, ids, 0, got["lse_dev"][0], got["a_dev"])
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.slow
def test_full_size_entropy_and_dlogits_every_row():
    """The full bf16 scoring workload (B=8, L=2048, V=151936) with entropy and LSE exported,
    then dlogits of the train side into bf16: every active row against the oracle, run in
    the host worker pool in chunks (entropy and LSE of both sides within 2e-5; every
    element of the gradient within the bound of the small shapes, with g = 1), and every
    inactive row of the gradient zero."""
    from train_rollout_logprob_amd import binding as B
    pool = oracle_pool()
    if pool is None:
        pytest.skip("the oracle worker pool was not started (no GPU counted at start-up)")
    case = synth.make_logits_case("qwen8b", device="cuda")
    ids, att, act, cu = device_inputs(case)
    N, V = case.N, case.V
    ent = tuple(torch.empty(N, dtype=torch.float32, device="cuda") for _ in range(2))
    lse = tuple(torch.empty(N, dtype=torch.float64, device="cuda") for _ in range(2))
    print(f"[case] full qwen8b entropy N={N}", flush=True)
    t, r, d, a, ws = B.selected_logprob(case.train, case.rollout, ids, att, act, case.layout,
                                        case.B, case.L, cu, check=True, entropy=ent, lse=lse)
    out = B.dlogits(case.train, case.rollout, ids, 0, lse[0], a, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    a_h = a.cpu().numpy()
    ent_h = [e.cpu().numpy().astype(np.float64) for e in ent]
    lse_h = [x.cpu().numpy() for x in lse]
    rows = np.nonzero(a_h)[0]
    per = max(1, FULL_CHUNK_BYTES // (2 * V * case.elem_bytes))
    worst = {"entropy": 0.0, "lse": 0.0, "dlogits": -np.inf}
    for a0 in range(0, len(rows), per):
        sel = rows[a0:a0 + per]
        idx = torch.as_tensor(sel, device="cuda")
        bt, br = pool.buffers(per, V, case.dtype)
        copy_rows(bt[:len(sel)], case.train, idx)
        copy_rows(br[:len(sel)], case.rollout, idx)
        et, er, lt, lr = pool.entropy(len(sel), V, case.dtype)
        for side, (e, l) in enumerate(((et, lt), (er, lr))):
            worst["entropy"] = max(worst["entropy"], float(np.abs(ent_h[side][sel] - e).max()))
            worst["lse"] = max(worst["lse"], float(np.abs(lse_h[side][sel] - l).max()))
        # side 1 of the buffer now holds the train side's gradient rows from the GPU
        copy_rows(br[:len(sel)], out, idx)
        # the small-shape bound with g = 1, S = 1: |want| LOGP_TOL + 2e-6, plus LOGP_TOL at
        # the selected column, then (|want| + that) * 2^-8 for the bf16 output
        ex, ey = pool.dlogits_excess(len(sel), V, case.dtype, "bf16", case.ids[sel],
                                     (LOGP_TOL + 2.0 ** -8 + LOGP_TOL * 2.0 ** -8))
        worst["dlogits"] = max(worst["dlogits"], float(ex.max()) - 2e-6 * (1 + 2.0 ** -8),
                               float(ey.max()) - (2e-6 + LOGP_TOL) * (1 + 2.0 ** -8))
        print(f"[case] full qwen8b rows {a0}..{a0 + len(sel) - 1} of {len(rows)}: {worst}",
              flush=True)
    assert worst["entropy"] <= LOGP_TOL and worst["lse"] <= LOGP_TOL
    assert worst["dlogits"] <= 0.0
    inactive = torch.as_tensor(np.nonzero(a_h == 0)[0], device="cuda")
    assert torch.count_nonzero(out.index_select(0, inactive)).item() == 0
    del case, t, r, d, a, ws, out
    torch.cuda.empty_cache()
