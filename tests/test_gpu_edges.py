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


def _bits16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_tree_mode_exponent_range(dtype):
    """The tree mode's partials keep their exponent reference within |k| < 2^30, i.e. a
    row maximum below about 7.4e8 in magnitude: rows inside match the oracle (to the fp32
    rounding of the output), rows beyond fail closed with NaN outputs on either sign, and
    logits far below the row maximum add nothing wherever they sit in the row (a whole
    leading wave group of them included)."""
    B = B_()
    V = 1024
    x = torch.zeros((6, V), device="cuda", dtype=torch.float32)
    x[0, 100] = 5.0e8       # inside: logp of column 0 is about -5e8
    x[1, 100] = 1.0e9       # beyond: fails closed
    x[2, :] = -5.0e8        # inside, uniform: -ln V
    x[3, :] = -1.0e9        # beyond, every logit: fails closed
    x[4, :600] = -1.0e30    # far below, leading: like absent columns
    x[5, 600:] = -1.0e30    # far below, trailing
    x = x.to(dtype)
    ids_h = np.array([0, 0, 3, 3, 700, 0], np.int32)
    ids = torch.as_tensor(ids_h, device="cuda")
    t, r, d, a, ws = B.selected_logprob(x, x, ids, layout="right", batch=6, seq_len=1)
    st, bad = B.drift_get_status(ws)
    assert status_name(st) == "ENONFINITE" and bad == 1
    t_h, d_h = t.cpu().numpy(), d.cpu().numpy()
    host = x.float().cpu().numpy() if dtype == torch.float32 else _bits16(x)
    want, _, _ = oracle.score_rows(host, host, "f32" if dtype == torch.float32 else "bf16",
                                   ids_h)
    for row in (0, 2, 4, 5):
        w = np.float32(want[row])
        assert abs(float(t_h[row]) - float(want[row])) <= float(np.spacing(abs(w))) + 1e-5, row
        assert d_h[row] == 0.0
    assert abs(float(t_h[4]) + math.log(V - 600)) <= 1e-5
    assert abs(float(t_h[5]) + math.log(600)) <= 1e-5
    for row in (1, 3):
        assert math.isnan(t_h[row]) and math.isnan(d_h[row]), row


def test_lmhead_exponent_range():
    """The fused head's partials follow the same exponent range: a token whose largest
    logit is about 6.4e9 fails closed with a NaN logprob, one at about 6.4e8 matches the
    oracle, the others are unaffected."""
    B = B_()
    T, H, V = 8, 64, 512
    gen = torch.Generator(device="cuda").manual_seed(5)
    hid = torch.randn((T, H), generator=gen, device="cuda").to(torch.bfloat16)
    w = (torch.randn((H, V), generator=gen, device="cuda") * 0.1).to(torch.bfloat16)
    w[:, 5] = 1.0e4
    hid[0, :] = 1.0e4       # z[0, 5] = 64 x 1e8: beyond
    hid[1, :] = 1.0e3       # z[1, 5] = 64 x 1e7: inside
    hid[2, :] = 10.0        # z[2, 5] = 6.4e6, the selected logit: logp about 0, where a
                            # scale error in the log-sum-exp would show
    ids_h = np.array([5, 7, 5, 2, 3, 4, 6, 8], np.int32)
    ids = torch.as_tensor(ids_h, device="cuda")
    logp, ws = B.lmhead_logprob(hid, w.contiguous(), ids)
    st, bad = B.drift_get_status(ws)
    assert status_name(st) == "ENONFINITE" and bad == 0
    got = logp.cpu().numpy()
    assert math.isnan(got[0])
    want = oracle.lmhead_logprob(_bits16(hid), oracle.widen(_bits16(w), "bf16"), ids_h)
    # the head accumulates each logit in fp32 over H products: allow the classic bound
    # H 2^-24 sum_k |h_k w_kj| on the largest logit of the row, and the output's rounding
    habs = np.abs(oracle.widen(_bits16(hid), "bf16")) @ np.abs(oracle.widen(_bits16(w), "bf16"))
    for t in range(1, T):
        tol = (float(np.spacing(np.float32(abs(want[t])))) + 2e-5 +
               2.0 * H * 2.0 ** -24 * float(habs[t].max()))
        assert abs(float(got[t]) - float(want[t])) <= tol, (t, got[t], want[t])
    assert abs(float(got[2]) - float(want[2])) <= LOGP_TOL  # its products sum exactly


@pytest.mark.parametrize("reduction", ["tree", "exact"])
def test_large_logits_keep_the_tolerance(reduction):
    """A constant added to every logit of a row leaves its log-softmax unchanged. The
    kernels take their exponents with log2(e) rounded to fp32 and convert the log-sum-exp
    back with that same constant, so rows shifted by up to 1e5 stay within 2e-5 of the
    oracle, also where the selected logit is the row maximum (logp near 0, where a scale
    error of the log-sum-exp would show). Under a temperature chain (folded for the
    log-sum-exp terms, whose way back to natural log undoes the fp32 rounding of the fold's
    factors) the selected logit takes the chain in fp32, so its rounding, at most
    2^-23 |z_y| (the reciprocal and the product), adds to the bound."""
    B = B_()
    V, N = 4099, 8
    gen = torch.Generator(device="cuda").manual_seed(9)
    base = torch.randn((N, V), generator=gen, device="cuda") * 2.0
    shifts = torch.tensor([1e4, -1e4, 1e5, -1e5, 3e3, -3e3, 5e4, 0.0], device="cuda")
    x = (base + shifts[:, None]).contiguous()
    xh = x.cpu().numpy()
    ids_h = xh.argmax(axis=1).astype(np.int32)
    ids_h[1::2] = np.random.default_rng(9).integers(0, V, N // 2)
    ids = torch.as_tensor(ids_h, device="cuda")
    for chain in (None, [("temperature", 0.7)]):
        print(f"[case] large logits {reduction} chain={chain}", flush=True)
        t, r, d, a, ws = B.selected_logprob(x, x, ids, layout="right", batch=N, seq_len=1,
                                            reduction=reduction, transforms=(chain, chain),
                                            check=True)
        want, _, _ = oracle.score_rows(xh, xh, "f32", ids_h, None, (chain, chain))
        err = np.abs(t.cpu().numpy().astype(np.float64) - want)
        zy = np.abs(xh[np.arange(N), ids_h].astype(np.float64)) / (0.7 if chain else 1.0)
        tol = LOGP_TOL + (2.0 ** -23 * zy if chain else 0.0)
        assert np.all(err <= tol), (chain, err, tol)
        assert float(d.abs().max()) == 0.0
