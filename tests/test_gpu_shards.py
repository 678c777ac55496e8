"""Vocabulary-parallel scoring on one GPU ("[WS2] Framework for ablation experiment",
LogProb knobs rows 3-5 and 8; the tp-partition control of the "Attention Debug Matrix"
Metrics): the exact reduction against the fp64 oracle, and shard partials merged in global
shard order against the unsharded exact call, bitwise, for many splits of the vocabulary.

Each shard is emulated by a column view of the full logits: its rows are the shard's
columns only, exactly what one tensor-parallel rank holds."""
import numpy as np
import pytest
import torch

import oracle
from helpers import (LOGP_TOL, assert_logprob_parity, device_inputs, host_logits, make_small,
                     oracle_all_rows, oracle_pool, run_library, small_variants, status_name)
from train_rollout_logprob_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _bits(x):
    return np.asarray(x).view(np.uint32 if np.asarray(x).dtype == np.float32 else np.uint64)


def _sharded(case, bounds, vocab_real=None, transforms=(None, None), lse=True):
    """Shard partials of every [b_s, b_{s+1}) column view, gathered and merged."""
    from train_rollout_logprob_amd import binding as B
    ids, att, act, cu = device_inputs(case)
    tparts, rparts = [], []
    for s in range(len(bounds) - 1):
        lo, hi = int(bounds[s]), int(bounds[s + 1])
        tp, rp, ws = B.shard_partials(case.train[:, lo:hi], case.rollout[:, lo:hi], ids, lo,
                                      case.V, att, act, case.layout, case.B, case.L, cu,
                                      vocab_real=vocab_real, transforms=transforms)
        tparts.append(tp)
        rparts.append(rp)
    lses = tuple(torch.empty(case.N, dtype=torch.float64, device="cuda") for _ in range(2))
    t, r, d, a, ws = B.merge_shards(torch.cat(tparts), torch.cat(rparts), bounds, ids, case.V,
                                    case.N, att, act, case.layout, case.B, case.L, cu,
                                    vocab_real=vocab_real, lse=lses if lse else (None, None))
    st, bad = B.drift_get_status(ws)
    return {"train_logp": t.cpu().numpy(), "rollout_logp": r.cpu().numpy(),
            "dlogp": d.cpu().numpy(), "active": a.cpu().numpy(), "status": st,
            "first_bad": bad, "lse": [l.cpu().numpy() for l in lses]}


def _exact(case, vocab_real=None, transforms=(None, None)):
    lses = tuple(torch.empty(case.N, dtype=torch.float64, device="cuda") for _ in range(2))
    got = run_library(case, reduction="exact", vocab_real=vocab_real, transforms=transforms,
                      lse=lses)
    got["lse"] = [l.cpu().numpy() for l in lses]
    return got


def _assert_bitwise(a, b, what=""):
    for k in ("train_logp", "rollout_logp", "dlogp"):
        assert np.array_equal(_bits(a[k]), _bits(b[k])), (what, k)
    assert np.array_equal(a["active"], b["active"])
    for side in (0, 1):
        assert np.array_equal(_bits(a["lse"][side]), _bits(b["lse"][side])), (what, side)


def _partitions(V):
    eq = lambda S: [((V // S) // 8 * 8) * i for i in range(S)] + [V]
    parts = [[0, V], eq(2), eq(3), eq(4), eq(8), [0, 8, V], [0, V - (V % 8 or 8), V]]
    rng = np.random.default_rng(V)
    cuts = sorted(set((rng.integers(1, V // 8, 5) * 8).tolist()))
    parts.append([0, *cuts, V])
    parts.append([0, 0, cuts[0], cuts[0], V])          # empty shards
    return parts


@pytest.mark.parametrize("key", list(small_variants()))
def test_exact_reduction_parity(key):
    case = make_small(small_variants()[key])
    print(f"[case] exact parity {key}", flush=True)
    got = run_library(case, reduction="exact")
    want = oracle.selected_logprob(host_logits(case.train), host_logits(case.rollout),
                                   case.dtype, case.ids, case.attention, case.action, case.V,
                                   case.layout, case.B, case.L, case.cu_seqlens)
    assert status_name(got["status"]) == want["status"]
    assert_logprob_parity(got, want)


@pytest.mark.parametrize("spec", [dict(name="qwen8b", B=2, L=40),
                                  dict(name="packed", nseq=3, len_lo=30, len_hi=90, V=3001),
                                  dict(name="qwen8b", B=2, L=24, V=1001)],
                         ids=["bf16_151936", "f32_3001", "bf16_1001"])
def test_shard_merge_is_bitwise_the_unsharded_exact_result(spec):
    case = make_small(spec)
    ref = _exact(case)
    assert status_name(ref["status"]) == "OK"
    for bounds in _partitions(case.V):
        print(f"[case] shards {spec['name']} V={case.V} bounds={bounds}", flush=True)
        got = _sharded(case, bounds)
        assert status_name(got["status"]) == "OK"
        _assert_bitwise(got, ref, bounds)


def test_shards_with_vocab_mask_and_transforms():
    case = make_small(dict(name="qwen8b", B=2, L=32, V=4096))
    Vr = 4000
    case.ids = (case.ids % Vr).astype(np.int32)
    tr = ([("softcap", 25.0), ("temperature", 0.8)], [("scale", 1.1)])
    ref = _exact(case, vocab_real=Vr, transforms=tr)
    want = oracle.selected_logprob(host_logits(case.train), host_logits(case.rollout),
                                   case.dtype, case.ids, case.attention, case.action, case.V,
                                   case.layout, case.B, case.L, vocab_real=Vr, transforms=tr)
    assert status_name(ref["status"]) == want["status"] == "OK"
    assert_logprob_parity(ref, want)
    for bounds in ([0, 2048, 4096], [0, 1000 // 8 * 8, 3992, 4096], [0, 4000, 4096],
                   [0, 8, 16, 24, 4096]):
        got = _sharded(case, bounds, vocab_real=Vr, transforms=tr)
        _assert_bitwise(got, ref, bounds)


def test_sharded_rows_against_the_sharded_oracle():
    case = make_small(dict(name="packed", nseq=3, len_lo=20, len_hi=60, V=3001))
    bounds = [0, 1000, 2000, 3001]
    got = _sharded(case, bounds)
    rows = np.nonzero(got["active"])[0]
    tr = synth.rows_to_host(case.train, rows)
    ro = synth.rows_to_host(case.rollout, rows)
    t, r, d = oracle.sharded_score_rows(tr, ro, case.dtype, case.ids[rows], bounds)
    for g, w in ((got["train_logp"][rows], t), (got["rollout_logp"][rows], r),
                 (got["dlogp"][rows], d)):
        assert np.abs(g.astype(np.float64) - w).max() <= LOGP_TOL


def test_exact_reduction_keeps_batch_composition_invariance():
    from train_rollout_logprob_amd import binding as B
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    V = 151936
    pool = torch.randn((16, V), generator=g, device="cuda").mul_(3).to(torch.bfloat16)
    ids = torch.randint(0, V, (16,), generator=g, device="cuda", dtype=torch.int32)
    ref = None
    for bs, slot in ((1, 0), (7, 5), (16, 11)):
        rows = torch.arange(bs, device="cuda") % 16
        rows[slot] = 2
        t, r, d, a, ws = B.selected_logprob(pool[rows], pool[rows], ids[rows], layout="right",
                                            batch=1, seq_len=bs, check=True, reduction="exact")
        v = np.array([t[slot].item(), d[slot].item()], np.float32)
        if ref is None:
            ref = v
        assert np.array_equal(v.view(np.uint32), ref.view(np.uint32)), bs


def test_shard_statuses():
    from train_rollout_logprob_amd import binding as B
    case = make_small(dict(name="qwen8b", B=2, L=24, V=1024))
    # a NaN logit in one shard fails closed after the merge, at that row
    r0 = int(np.nonzero(case.action)[0][4])
    case.train[r0, 700] = float("nan")
    got = _sharded(case, [0, 512, 1024])
    assert status_name(got["status"]) == "ENONFINITE" and got["first_bad"] == r0
    assert status_name(_exact(case)["status"]) == "ENONFINITE"
    case.train[r0, 700] = 0.0
    # partials made with shifted ownership (shard starts disagree with the merge bounds)
    case.ids = case.ids.copy()
    case.ids[r0] = 300
    ids, att, act, cu = device_inputs(case)
    tp0, rp0, _ = B.shard_partials(case.train[:, :512], case.rollout[:, :512], ids, 0, case.V,
                                   att, act, case.layout, case.B, case.L, cu)
    tp1, rp1, _ = B.shard_partials(case.train[:, 512:], case.rollout[:, 512:], ids, 512,
                                   case.V, att, act, case.layout, case.B, case.L, cu)
    t, r, d, a, ws = B.merge_shards(torch.cat([tp0, tp1]), torch.cat([rp0, rp1]), [0, 256, 1024],
                                    ids, case.V, case.N, att, act, case.layout, case.B, case.L)
    st, bad = B.drift_get_status(ws)
    assert status_name(st) == "EMASK"
    assert bad == r0 or bad < r0
    # a selected id out of range is a token error in the shard calls and in the merge
    case.ids[r0] = case.V + 2
    got = _sharded(case, [0, 512, 1024])
    assert status_name(got["status"]) == "ETOKEN" and got["first_bad"] == r0


def test_exact_lse_feeds_dlogits():
    from train_rollout_logprob_amd import binding as B
    case = make_small(dict(name="qwen8b", B=2, L=24, V=2048))
    ids, att, act, cu = device_inputs(case)
    lse = tuple(torch.empty(case.N, dtype=torch.float64, device="cuda") for _ in range(2))
    t, r, d, a, ws = B.selected_logprob(case.train, case.rollout, ids, att, act, case.layout,
                                        case.B, case.L, check=True, lse=lse, reduction="exact")
    g = B.dlogits(case.train, case.rollout, ids, 0, lse[0], a)
    want = oracle.dlogits_rows(host_logits(case.train), case.dtype, case.ids, a.cpu().numpy())
    assert np.abs(g.cpu().numpy() - want).max() <= LOGP_TOL


@pytest.mark.slow
def test_full_size_eight_shards_bitwise():
    """The full bf16 scoring workload (B=8, L=2048, V=151936) split into 8 tensor-parallel
    vocabulary shards of 18992 columns: every row bitwise equal to the unsharded exact
    result, and every active row against the oracle (run in the host worker pool)."""
    pool = oracle_pool()
    if pool is None:
        pytest.skip("the oracle worker pool was not started (no GPU counted at start-up)")
    case = synth.make_logits_case("qwen8b", device="cuda")
    print(f"[case] full qwen8b 8 shards N={case.N}", flush=True)
    ref = _exact(case)
    assert status_name(ref["status"]) == "OK"
    got = _sharded(case, [i * 18992 for i in range(8)] + [case.V])
    _assert_bitwise(got, ref, "8 shards")
    rows = np.nonzero(ref["active"])[0]
    t, r, d = oracle_all_rows(pool, case, rows)
    for k, w in (("train_logp", t), ("rollout_logp", r), ("dlogp", d)):
        err = float(np.abs(ref[k][rows].astype(np.float64) - w).max())
        print(f"[case] full qwen8b exact {k} max err {err:.3e} over {len(rows)} rows", flush=True)
        assert err <= LOGP_TOL
    del case
    torch.cuda.empty_cache()
