"""GPU parity of drift_selected_logprob against the fp64 oracle, edge cases, error
statuses, determinism and the batch-composition (C1) bitwise control."""
import math

import numpy as np
import pytest
import torch

from helpers import (LOGP_TOL, assert_logprob_parity, make_small, run_library, run_oracle,
                     small_variants, status_name)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


@pytest.mark.parametrize("key", list(small_variants().keys()))
def test_parity_small_variants(key):
    case = make_small(small_variants()[key])
    print(f"[case] {key} N={case.N} V={case.V} dtype={case.dtype} layout={case.layout}",
          flush=True)
    got = run_library(case)
    want = run_oracle(case)
    assert status_name(got["status"]) == want["status"] == "OK"
    assert_logprob_parity(got, want)
    assert int(got["active"].sum()) == case.n_active() > 0


def test_int64_ids_and_row_stride():
    case = make_small(dict(name="qwen8b", B=2, L=40, V=3000))
    base = run_library(case)
    # same logits inside wider rows (row_stride = V + 24)
    pad = 24
    wide_t = torch.full((case.N, case.V + pad), float("nan"), device="cuda",
                        dtype=case.train.dtype)
    wide_r = wide_t.clone()
    wide_t[:, : case.V] = case.train
    wide_r[:, : case.V] = case.rollout
    got = run_library(case, ids_dtype=torch.int64, train=wide_t[:, : case.V],
                      rollout=wide_r[:, : case.V])
    assert got["status"] == 0
    for k in ("train_logp", "rollout_logp", "dlogp", "active"):
        assert np.array_equal(got[k], base[k]), k   # bitwise: same rows, same tree


def test_identical_sides_give_exact_zero():
    case = make_small(dict(name="large", B=3, L=48))
    got = run_library(case, rollout=case.train)
    act = got["active"] == 1
    assert np.all(got["dlogp"][act] == 0.0)
    assert np.array_equal(got["train_logp"], got["rollout_logp"])


def test_uniform_logits_give_minus_log_V():
    for V, dt in ((151936, torch.bfloat16), (32000, torch.float32), (1, torch.float32),
                  (1001, torch.bfloat16)):
        N = 5
        x = torch.full((N, V), 2.5, device="cuda", dtype=dt)
        ids = torch.arange(N, device="cuda", dtype=torch.int32) % V
        from train_rollout_logprob_amd import binding as B
        t, r, d, a, ws = B.selected_logprob(x, x, ids, layout="right", batch=1, seq_len=N,
                                            check=True)
        assert torch.all(a == 1)
        err = (t.double() + math.log(V)).abs().max().item()
        assert err <= LOGP_TOL, (V, err)


def test_empty_and_all_inactive():
    from train_rollout_logprob_amd import binding as B
    x = torch.zeros((0, 64), device="cuda")
    ids = torch.zeros(0, dtype=torch.int32, device="cuda")
    t, r, d, a, ws = B.selected_logprob(x, x, ids, layout="right", batch=0, seq_len=1,
                                        check=True)
    assert t.numel() == 0
    case = make_small(dict(name="tiny", B=2, L=16, V=64, prompt=4))
    act = torch.zeros(case.N, dtype=torch.uint8, device="cuda")
    ids, att, _, _ = __import__("helpers").device_inputs(case)
    t, r, d, a, ws = B.selected_logprob(case.train, case.rollout, ids, att, act, "right", case.B,
                                        case.L, check=True)
    assert torch.all(a == 0) and torch.all(t == 0) and torch.all(d == 0)


def _status_of(case, **mut):
    import helpers
    from train_rollout_logprob_amd import binding as B
    ids, att, act, cu = helpers.device_inputs(case)
    tr, ro = mut.get("train", case.train), mut.get("rollout", case.rollout)
    ids = mut.get("ids", ids)
    att = mut.get("att", att)
    act = mut.get("act", act)
    cu = mut.get("cu", cu)
    layout = mut.get("layout", case.layout)
    t, r, d, a, ws = B.selected_logprob(tr, ro, ids, att, act, layout, case.B, case.L, cu)
    st, bad = B.drift_get_status(ws)
    return status_name(st), bad, (t, r, d, a)


def test_error_statuses_match_oracle():
    import oracle
    case = make_small(dict(name="tiny", B=2, L=32, V=300, prompt=8))
    ids, att, act, _ = __import__("helpers").device_inputs(case)
    act_rows = np.nonzero((case.attention != 0) & (case.action != 0))[0]
    r0 = int(act_rows[0])

    def expect(**mut):
        host = {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in mut.items()}
        o = oracle.selected_logprob(
            __import__("helpers").host_logits(mut.get("train", case.train)),
            __import__("helpers").host_logits(mut.get("rollout", case.rollout)), case.dtype,
            host.get("ids", case.ids), host.get("att", case.attention),
            host.get("act", case.action), case.V, mut.get("layout", case.layout), case.B,
            case.L)
        got, bad, outs = _status_of(case, **mut)
        assert got == o["status"], (list(mut), got, o["status"])
        return got, bad

    assert expect()[0] == "OK"
    hole = att.clone(); hole[3] = 0
    assert expect(att=hole) == ("EMASK", 3)             # row 3: a 0 followed by a 1
    assert expect(layout="left")[0] == "EMASK"
    pad_act = act.clone(); pad_act[case.N - 1] = 1      # action on a padded row
    assert expect(act=pad_act) == ("EMASK", case.N - 1)
    two = act.clone(); two[r0] = 2
    assert expect(act=two)[0] == "EMASK"
    oov = ids.clone(); oov[r0] = case.V
    st, bad = expect(ids=oov)
    assert (st, bad) == ("ETOKEN", r0)
    neg = ids.clone(); neg[r0] = -100
    assert expect(ids=neg)[0] == "ETOKEN"
    ign = ids.clone(); ign[0] = -100                    # row 0 is a prompt row
    assert expect(ids=ign)[0] == "OK"
    both = oov.clone()
    assert expect(ids=both, att=hole)[0] == "EMASK"
    xn = case.train.clone(); xn[r0, 7] = float("nan")
    assert expect(train=xn) == ("ENONFINITE", r0)
    xi = case.rollout.clone(); xi[r0, 7] = float("inf")
    assert expect(rollout=xi)[0] == "ENONFINITE"
    xs = case.train.clone(); xs[r0, int(case.ids[r0])] = float("-inf")
    assert expect(train=xs)[0] == "ENONFINITE"
    xo = case.train.clone(); xo[r0, (int(case.ids[r0]) + 1) % case.V] = float("-inf")
    assert expect(train=xo)[0] == "OK"
    xp = case.train.clone(); xp[0, :] = float("nan")    # inactive row: never read
    assert expect(train=xp)[0] == "OK"
    xa = case.train.clone(); xa[r0, :] = float("-inf")  # every logit -inf
    assert expect(train=xa)[0] == "ENONFINITE"


def test_oov_row_outputs_nan_and_others_unchanged():
    case = make_small(dict(name="tiny", B=2, L=32, V=300, prompt=8))
    base = run_library(case)
    ids, _, _, _ = __import__("helpers").device_inputs(case)
    r0 = int(np.nonzero(base["active"])[0][3])
    oov = ids.clone(); oov[r0] = 10 ** 6
    st, bad, (t, r, d, a) = _status_of(case, ids=oov)
    assert st == "ETOKEN" and bad == r0
    t = t.cpu().numpy()
    assert math.isnan(t[r0])
    keep = np.arange(case.N) != r0
    assert np.array_equal(t[keep], base["train_logp"][keep])


def test_negative_inf_entries_are_probability_zero():
    import oracle, helpers
    case = make_small(dict(name="packed", nseq=3, len_lo=40, len_hi=80, V=2000))
    tr = case.train.clone()
    ro = case.rollout.clone()
    tr[:, 100:700] = float("-inf")
    ro[:, 0:1999:3] = float("-inf")
    ids = case.ids.copy()
    ids[:] = 1999 if 1999 % 3 else 1998
    case.ids = ids
    got = run_library(case, train=tr, rollout=ro)
    want = run_oracle(case, train=tr, rollout=ro)
    assert status_name(got["status"]) == want["status"] == "OK"
    assert_logprob_parity(got, want)


def test_repeat_runs_are_bitwise_identical():
    case = make_small(dict(name="qwen8b", B=2, L=64))
    a = run_library(case)
    for _ in range(3):
        b = run_library(case)
        for k in ("train_logp", "rollout_logp", "dlogp", "active"):
            assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f32", 32000), ("bf16", 1001)])
def test_batch_composition_control_is_bitwise_zero(dtype, V):
    """The same rows re-scored at other positions, in batches of 1, 7 and 64, under both
    padding sides, give bitwise the same logp and dlogp (the batch-composition control of
    the Attention Debug Matrix page)."""
    from train_rollout_logprob_amd import binding as B
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    pool = 80
    base_t = (torch.randn((pool, V), generator=g, device="cuda") * 3).to(tdt)
    base_r = (base_t.float() + torch.randn((pool, V), generator=g, device="cuda") * 5e-3).to(tdt)
    ids_pool = torch.randint(0, V, (pool,), generator=g, device="cuda", dtype=torch.int32)
    probe = [0, 17, 42, pool - 1]
    ref = None
    rng = np.random.default_rng(5)
    for bs in (1, 7, 64):
        for side in ("right", "left"):
            # batch of `bs` sequences of length L=8; each probe row lands in a random slot
            L = 8
            N = bs * L
            rows = rng.integers(0, pool, N)
            slots = rng.choice(N, size=len(probe), replace=False) if N >= len(probe) else None
            results = []
            for j, pr in enumerate(probe):
                rr = rows.copy()
                slot = int(slots[j]) if slots is not None else 0
                rr[slot] = pr
                idx = torch.as_tensor(rr, device="cuda")
                t = base_t.index_select(0, idx)
                r = base_r.index_select(0, idx)
                ids = ids_pool.index_select(0, idx)
                att = torch.ones(N, dtype=torch.uint8, device="cuda")
                act = torch.ones(N, dtype=torch.uint8, device="cuda")
                # pad one row of every other sequence, away from the probe slot
                for b in range(0, bs, 2):
                    prow = b * L + (L - 1 if side == "right" else 0)
                    if prow != slot:
                        att[prow] = 0
                        act[prow] = 0
                tl, rl, dl, al, ws = B.selected_logprob(t, r, ids, att, act, side, bs, L,
                                                        check=True)
                results.append((tl[slot].item(), rl[slot].item(), dl[slot].item()))
            arr = np.array(results, dtype=np.float32)
            if ref is None:
                ref = arr
            assert np.array_equal(arr.view(np.uint32), ref.view(np.uint32)), (bs, side)
