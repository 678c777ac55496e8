"""Degenerate inputs of the newer entry points on the GPU: empty batches, a single vocabulary
column, probability-zero columns, the exact mode's exponent limit, and segments without
rows, each against the closed form or the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import LOGP_TOL, status_name

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def B_():
    from train_rollout_logprob_amd import binding as B
    return B


@pytest.mark.parametrize("reduction", ["tree", "exact"])
def test_empty_batch_every_entry_point(reduction):
    B = B_()
    x = torch.zeros((0, 64), device="cuda", dtype=torch.bfloat16)
    ids = torch.zeros(0, dtype=torch.int32, device="cuda")
    lse = tuple(torch.zeros(0, dtype=torch.float64, device="cuda") for _ in range(2))
    t, r, d, a, ws = B.selected_logprob(x, x, ids, layout="right", batch=0, seq_len=1,
                                        check=True, reduction=reduction, lse=lse)
    assert t.numel() == 0
    g = B.dlogits(x, x, ids, 0, lse[0], a)
    assert g.shape == (0, 64)
    segs = B.segment_diagnostics(d, a, torch.zeros(2, dtype=torch.int32, device="cuda"))
    assert len(segs) == 1 and status_name(segs[0]["status"]) == "ENOACTIVE"
    tp, rp, _ = B.shard_partials(x[:, :32], x[:, :32], ids, 0, 64, layout="right", batch=0,
                                 seq_len=1)
    tp2, rp2, _ = B.shard_partials(x[:, 32:], x[:, 32:], ids, 32, 64, layout="right", batch=0,
                                   seq_len=1)
    t2, r2, d2, a2, ws2 = B.merge_shards(torch.cat([tp, tp2]), torch.cat([rp, rp2]), [0, 32, 64],
                                         ids, 64, 0, layout="right", batch=0, seq_len=1)
    assert t2.numel() == 0 and status_name(B.drift_get_status(ws2)[0]) == "OK"


@pytest.mark.parametrize("reduction", ["tree", "exact"])
def test_single_column_and_uniform_rows(reduction):
    """V = 1: the only column is the selected one, logp = 0, entropy = 0, dlogits = 0;
    uniform rows give -ln V for several V, in both reductions."""
    B = B_()
    for V, dt in ((1, torch.float32), (1, torch.bfloat16), (7, torch.float32),
                  (4096, torch.bfloat16), (151936, torch.bfloat16)):
        N = 6
        x = torch.full((N, V), -3.25, device="cuda", dtype=dt)
        ids = torch.arange(N, device="cuda", dtype=torch.int32) % V
        lse = tuple(torch.empty(N, dtype=torch.float64, device="cuda") for _ in range(2))
        ent = tuple(torch.empty(N, dtype=torch.float32, device="cuda") for _ in range(2))
        kw = dict(lse=lse) if reduction == "exact" else dict(lse=lse, entropy=ent)
        t, r, d, a, ws = B.selected_logprob(x, x, ids, layout="right", batch=1, seq_len=N,
                                            check=True, reduction=reduction, **kw)
        err = (t.double() + math.log(V)).abs().max().item()
        assert err <= LOGP_TOL, (V, err)
        assert torch.all(d == 0)                                 # identical sides
        assert (lse[0] - (-3.25 + math.log(V))).abs().max().item() <= LOGP_TOL
        if reduction == "tree":
            assert (ent[0].double() - math.log(V)).abs().max().item() <= LOGP_TOL
        g = B.dlogits(x, x, ids, 0, lse[0], a).double().cpu().numpy()
        want = -np.full((N, V), 1.0 / V)
        want[np.arange(N), np.arange(N) % V] += 1.0
        assert np.abs(g - want).max() <= LOGP_TOL


@pytest.mark.parametrize("reduction", ["tree", "exact"])
def test_probability_zero_columns(reduction):
    """-inf logits add nothing: a row whose only finite logit is the selected one has
    logp = 0 on both sides; -inf elsewhere keeps the oracle's value."""
    B = B_()
    V, N = 3000, 4
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    x = torch.randn((N, V), generator=g, device="cuda")
    ids = torch.tensor([5, 2999, 0, 1500], dtype=torch.int32, device="cuda")
    x[0, :] = -math.inf
    x[0, 5] = 1.5
    x[1, :2000] = -math.inf
    t, r, d, a, ws = B.selected_logprob(x, x, ids, layout="right", batch=1, seq_len=N,
                                        check=True, reduction=reduction)
    want = oracle.score_rows(x.cpu().numpy(), x.cpu().numpy(), "f32", ids.cpu().numpy())[0]
    assert abs(t[0].item()) <= LOGP_TOL
    assert np.abs(t.double().cpu().numpy() - want).max() <= LOGP_TOL


def test_exact_mode_exponent_limit_fails_closed():
    """The exact mode takes group exponents up to 2^24 (|logit| < 1.16e7) and fails closed
    beyond; the tree mode takes them (any finite fp32 exponent)."""
    B = B_()
    V, N = 512, 2
    x = torch.zeros((N, V), device="cuda")
    ids = torch.zeros(N, dtype=torch.int32, device="cuda")
    x[1, 100] = 2.0e7
    for red, want in (("tree", "OK"), ("exact", "ENONFINITE")):
        t, r, d, a, ws = B.selected_logprob(x, x, ids, layout="right", batch=1, seq_len=N,
                                            reduction=red)
        st, bad = B.drift_get_status(ws)
        assert status_name(st) == want, red
        if want != "OK":
            assert bad == 1 and math.isnan(t[1].item()) and t[0].item() == t[0].item()
    x[1, 100] = 1.0e7                                            # below the limit: fine
    t, r, d, a, ws = B.selected_logprob(x, x, ids, layout="right", batch=1, seq_len=N,
                                        reduction="exact", check=True)
    assert abs(t[1].item() - (0.0 - 1.0e7)) <= 1.0                # x_y - LSE = 0 - 1e7


def test_segments_without_rows_or_active_rows():
    B = B_()
    d = torch.randn(100, device="cuda") * 1e-3
    a = torch.zeros(100, dtype=torch.uint8, device="cuda")
    a[40:60] = 1
    offs = torch.tensor([0, 0, 40, 60, 60, 100], dtype=torch.int32, device="cuda")
    segs = B.segment_diagnostics(d, a, offs)
    assert [status_name(s["status"]) for s in segs] == ["ENOACTIVE", "ENOACTIVE", "OK",
                                                         "ENOACTIVE", "ENOACTIVE"]
    want = oracle.diagnostics(d.cpu().numpy()[40:60], np.ones(20, np.uint8))
    assert segs[2]["n_active"] == 20 and segs[2]["p99_abs_dlogp"] == np.float32(
        want["p99_abs_dlogp"])
    assert segs[2]["argmax_row"] == 40 + want["argmax_row"]
    assert B.segment_diagnostics(d, a, torch.zeros(1, dtype=torch.int32, device="cuda")) == []


def test_batch_beyond_one_dispatch():
    """A batch larger than one dispatch holds (2^32 - 1 work-items: 8388607 rows of 512
    threads for fp32 scoring, 16777215 rows of 256 threads for dlogits) is covered by
    consecutive launches over row ranges. Rows on both sides of each boundary, the last
    rows and random rows against the oracle; every row's `active`; Gate A of the whole
    dlogp array; dlogits rows on both sides of its boundary."""
    B = B_()
    N, V = 16777215 + 129, 8
    splits = (8388607, 16777215)
    print(f"[case] fp32 N={N} V={V}: scoring launches split at {splits}", flush=True)
    rng = np.random.default_rng(41)
    ids = rng.integers(0, V, N).astype(np.int32)
    act = (rng.random(N) < 0.9).astype(np.uint8)
    gen = torch.Generator(device="cuda").manual_seed(41)
    ro = torch.randn((N, V), generator=gen, device="cuda") * 2.0
    tr = ro + torch.randn((N, V), generator=gen, device="cuda") * 1e-3
    ids_d = torch.as_tensor(ids, device="cuda")
    act_d = torch.as_tensor(act, device="cuda")
    lse_t = torch.empty(N, dtype=torch.float64, device="cuda")
    lse_r = torch.empty(N, dtype=torch.float64, device="cuda")
    t, r, d, a, ws = B.selected_logprob(tr, ro, ids_d, None, act_d, "right", N, 1, check=True,
                                        lse=(lse_t, lse_r))
    a_h = a.cpu().numpy()
    assert np.array_equal(a_h, act)
    near = np.concatenate([np.arange(s - 3, s + 3) for s in splits] + [np.arange(N - 4, N)])
    rows = np.unique(np.concatenate([near, rng.integers(0, N, 500)]))
    rows = rows[act[rows] == 1]
    idx = torch.as_tensor(rows, device="cuda")
    ot, orr, od = oracle.score_rows(tr.index_select(0, idx).cpu().numpy(),
                                    ro.index_select(0, idx).cpu().numpy(), "f32", ids[rows])
    for g, w in ((t, ot), (r, orr), (d, od)):
        err = np.abs(g.index_select(0, idx).cpu().numpy().astype(np.float64) - w)
        assert float(err.max()) <= LOGP_TOL
    d_h = d.cpu().numpy()
    st, s = B.diagnostics(d, a, 0.2, 0.2, logprob_ws=ws)
    assert status_name(st) == "OK"
    from helpers import assert_stats_exact
    assert_stats_exact(s, oracle.diagnostics(d_h, a_h, 0.2, 0.2))
    del d, r, lse_r
    g = torch.empty((N, V), dtype=torch.float32, device="cuda")
    B.dlogits(tr, ro, ids_d, 0, lse_t, a, out=g)
    drows = np.arange(splits[1] - 3, splits[1] + 3)
    idx = torch.as_tensor(drows, device="cuda")
    want = oracle.dlogits_rows(tr.index_select(0, idx).cpu().numpy(), "f32", ids[drows],
                               act[drows])
    got = g.index_select(0, idx).cpu().numpy().astype(np.float64)
    assert np.abs(got - want).max() <= 2e-5
    torch.cuda.empty_cache()


def test_exact_batch_beyond_one_dispatch():
    """The exact reduction on short rows runs one wave per row, four rows per block, so one
    dispatch covers 67108860 rows; a larger batch takes consecutive launches. Sampled rows
    and the rows on both sides of the boundary against the oracle, and the boundary rows,
    the last rows and a few random rows bitwise equal to the same rows scored as a batch of
    their own (the exact result does not depend on the batch or the launch a row falls in)."""
    B = B_()
    split = 67108860
    N, V = split + 37, 8
    print(f"[case] exact fp32 N={N} V={V}: launches split at {split}", flush=True)
    rng = np.random.default_rng(43)
    ids = rng.integers(0, V, N).astype(np.int32)
    act = (rng.random(N) < 0.9).astype(np.uint8)
    gen = torch.Generator(device="cuda").manual_seed(43)
    ro = torch.randn((N, V), generator=gen, device="cuda") * 2.0
    tr = ro + torch.randn((N, V), generator=gen, device="cuda") * 1e-3
    ids_d = torch.as_tensor(ids, device="cuda")
    act_d = torch.as_tensor(act, device="cuda")
    t, r, d, a, _ = B.selected_logprob(tr, ro, ids_d, None, act_d, "right", N, 1, check=True,
                                       reduction="exact")
    assert torch.equal(a, act_d)
    near = np.concatenate([np.arange(split - 5, split + 5), np.arange(N - 4, N)])
    rows = np.unique(np.concatenate([near, rng.integers(0, N, 300)]))
    rows = rows[act[rows] == 1]
    idx = torch.as_tensor(rows, device="cuda")
    ot, orr, od = oracle.score_rows(tr.index_select(0, idx).cpu().numpy(),
                                    ro.index_select(0, idx).cpu().numpy(), "f32", ids[rows])
    for g, w in ((t, ot), (r, orr), (d, od)):
        err = np.abs(g.index_select(0, idx).cpu().numpy().astype(np.float64) - w)
        assert float(err.max()) <= LOGP_TOL
    n = len(rows)
    t2, r2, d2, a2, _ = B.selected_logprob(tr.index_select(0, idx), ro.index_select(0, idx),
                                           ids_d.index_select(0, idx), None,
                                           act_d.index_select(0, idx), "right", n, 1,
                                           check=True, reduction="exact")
    for g, w in ((t, t2), (r, r2), (d, d2)):
        assert torch.equal(g.index_select(0, idx).view(torch.int32), w.view(torch.int32))
    del tr, ro
    torch.cuda.empty_cache()
