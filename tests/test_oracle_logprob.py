"""Pins of the oracle's log-softmax gather, dlogp and input validation against closed
forms, 50-digit brute force and textbook library routines (CPU only)."""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from oracle.logprob import score_row

RNG = np.random.default_rng(1234)


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------- widening

def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x7F80, 0xFF80, 0x0001, 0x0000, 0x8000, 0x4300],
                    dtype=np.uint16)
    got = oracle.widen(bits, "bf16")
    want = [1.0, -1.0, 3.140625, math.inf, -math.inf, 2.0 ** -133, 0.0, -0.0, 128.0]
    for g, w in zip(got, want):
        assert g == w
    assert math.copysign(1.0, got[7]) == -1.0


def test_f32_widening_is_exact():
    x = RNG.standard_normal(1000).astype(np.float32)
    assert np.array_equal(oracle.widen(x, "f32"), x.astype(np.float64))


# --------------------------------------------------------------------------- LSE closed forms

@pytest.mark.parametrize("V", [1, 2, 7, 1024, 151936])
@pytest.mark.parametrize("c", [0.0, 3.5, -1.0e4, 1.0e4])
def test_uniform_row_gives_minus_log_V(V, c):
    x = np.full(V, c)
    lp = x[V // 2] - oracle.logsumexp_row(x)
    assert abs(lp - (-math.log(V))) <= 1e-12 * max(1.0, abs(c))
    if c == 0.0:
        assert lp == -math.log(V)


@pytest.mark.parametrize("V,k,a,b", [(10, 3, 1.5, -2.0), (151936, 1, 16.0, 0.0),
                                     (32000, 17, -3.0, 2.25), (5, 4, 100.0, 99.0)])
def test_two_valued_row(V, k, a, b):
    x = np.full(V, b)
    x[:k] = a
    want = math.log(k * math.exp(a - max(a, b)) + (V - k) * math.exp(b - max(a, b))) + max(a, b)
    got = oracle.logsumexp_row(x)
    assert abs(got - want) <= 1e-13 * max(1.0, abs(want))
    # the selected token being one of the ``a`` entries vs one of the ``b`` entries
    assert abs((x[0] - got) - (a - want)) <= 1e-13 * max(1.0, abs(want))
    assert abs((x[V - 1] - got) - (b - want)) <= 1e-13 * max(1.0, abs(want))


@pytest.mark.parametrize("xy,xo", [(0.0, 0.0), (3.0, -1.0), (-20.0, 15.0), (700.0, 650.0)])
def test_two_token_vocab(xy, xo):
    x = _f64([xo, xy])
    got = x[1] - oracle.logsumexp_row(x)
    assert abs(got - (-math.log1p(math.exp(xo - xy)))) <= 1e-13 * max(1.0, abs(got))


@pytest.mark.parametrize("c", [0.5, 64.0, -1024.0, 3.0e5])
def test_shift_invariance(c):
    x = RNG.standard_normal(4096) * 3.0
    y = 77
    a = x[y] - oracle.logsumexp_row(x)
    b = (x[y] + c) - oracle.logsumexp_row(x + c)
    assert abs(a - b) <= 1e-12 * max(1.0, abs(c))


def _decimal_logp(x, y, digits=50):
    getcontext().prec = digits
    xs = [Decimal(float(v)) for v in x]
    s = sum((v.exp() for v in xs), Decimal(0))
    return float(xs[y] - s.ln())


@pytest.mark.parametrize("V", [1, 2, 3, 17, 64])
def test_brute_force_50_digits(V):
    for trial in range(20):
        x = RNG.standard_normal(V) * float(RNG.choice([0.1, 2.0, 30.0]))
        y = int(RNG.integers(0, V))
        got = x[y] - oracle.logsumexp_row(x)
        want = _decimal_logp(x, y)
        assert abs(got - want) <= 1e-13 * max(1.0, abs(want)), (V, trial)


def test_against_scipy_and_torch_on_big_rows():
    from scipy.special import logsumexp
    import torch

    for V, sig in [(151936, 3.0), (32000, 2.0), (1024, 2.0)]:
        x = RNG.standard_normal(V) * sig
        x[5] += 8.0
        got = oracle.logsumexp_row(x)
        assert abs(got - float(logsumexp(x))) <= 1e-12 * abs(got)
        lsm = torch.log_softmax(torch.from_numpy(x), dim=0).numpy()
        assert abs((x[5] - got) - float(lsm[5])) <= 1e-12


def test_minus_inf_entries_have_probability_zero():
    x = RNG.standard_normal(100)
    xm = x.copy()
    xm[10:20] = -math.inf
    keep = np.concatenate([x[:10], x[20:]])
    assert abs(oracle.logsumexp_row(xm) - oracle.logsumexp_row(keep)) <= 1e-14 * 10
    assert oracle.logsumexp_row(np.full(4, -math.inf)) == -math.inf


# --------------------------------------------------------------------------- dlogp

def test_dlogp_selected_logit_raised():
    """Train row = rollout row with only the selected logit raised by delta.
    With k 'b' entries: p_y = e^a / (e^a + (V-1) e^b), and
    dlogp = delta - log1p(p_y * expm1(delta)) > 0 for delta > 0."""
    V, a, b, delta, y = 50, 1.0, -0.5, 0.01, 3
    ro = np.full(V, b)
    ro[y] = a
    tr = ro.copy()
    tr[y] += delta
    p_y = math.exp(a) / (math.exp(a) + (V - 1) * math.exp(b))
    want = delta - math.log1p(p_y * math.expm1(delta))
    _, _, d, bad = score_row(tr, ro, y)
    assert not bad
    assert d > 0
    assert abs(d - want) <= 1e-15


def test_identical_sides_give_exact_zero():
    N, V = 12, 300
    x = (RNG.standard_normal((N, V)) * 2).astype(np.float32)
    act = np.ones(N, np.uint8)
    ids = RNG.integers(0, V, N)
    out = oracle.selected_logprob(x, x.copy(), "f32", ids, None, act, V, "right", 1, N)
    assert out["status"] == "OK"
    assert np.all(out["dlogp"] == 0.0)
    assert np.array_equal(out["train_logp"], out["rollout_logp"])


def test_uniform_shift_of_one_side_gives_zero_drift():
    V = 257
    x = RNG.standard_normal(V)
    _, _, d, _ = score_row(x + 0.75, x, 9)
    assert abs(d) <= 1e-14


# --------------------------------------------------------------------------- active rule + validation

def _small(layout="right"):
    B, L, V = 2, 6, 11
    N = B * L
    att = np.array([1, 1, 1, 1, 0, 0, 1, 1, 1, 1, 1, 1], np.uint8)
    act = np.array([0, 0, 1, 1, 0, 0, 0, 1, 0, 1, 1, 1], np.uint8)
    if layout == "left":
        att = np.array([0, 0, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1], np.uint8)
        act = np.array([0, 0, 0, 1, 1, 1, 0, 0, 1, 1, 0, 1], np.uint8)
    ids = (np.arange(N) * 7) % V
    x = (RNG.standard_normal((N, V))).astype(np.float32)
    return B, L, V, N, att, act, ids, x


@pytest.mark.parametrize("layout", ["right", "left"])
def test_active_rows_are_exactly_attended_action_rows(layout):
    B, L, V, N, att, act, ids, x = _small(layout)
    out = oracle.selected_logprob(x, x + 0.001, "f32", ids, att, act, V, layout, B, L)
    assert out["status"] == "OK"
    want = np.array([a and b for a, b in zip(att, act)], np.uint8)
    assert np.array_equal(out["active"], want)
    assert np.all(out["train_logp"][want == 0] == 0.0)
    assert np.all(out["train_logp"][want == 1] < 0.0)


def test_validation_classes():
    B, L, V, N, att, act, ids, x = _small("right")
    st = lambda **kw: oracle.selected_logprob(
        kw.get("x", x), kw.get("x", x), "f32", kw.get("ids", ids), kw.get("att", att),
        kw.get("act", act), V, kw.get("layout", "right"), B, L)["status"]
    assert st() == "OK"
    hole = att.copy(); hole[1] = 0                       # 1,0,1,1,0,0: not contiguous
    assert st(att=hole) == "EMASK"
    assert st(layout="left") == "EMASK"                   # right-padded mask under "left"
    bad = act.copy(); bad[4] = 1                          # action on a padded row
    assert st(act=bad) == "EMASK"
    two = act.copy(); two[2] = 2                          # mask byte other than 0/1
    assert st(act=two) == "EMASK"
    oov = ids.copy(); oov[3] = V                          # active row, id == V
    assert st(ids=oov) == "ETOKEN"
    neg = ids.copy(); neg[3] = -100                       # ignore_index on an active row
    assert st(ids=neg) == "ETOKEN"
    ign = ids.copy(); ign[0] = -100; ign[4] = V + 5       # only on inactive rows: fine
    assert st(ids=ign) == "OK"
    both = oov.copy()
    assert st(ids=both, att=hole) == "EMASK"              # EMASK outranks ETOKEN
    xn = x.copy(); xn[3, 5] = np.nan
    assert st(x=xn) == "ENONFINITE"
    xi = x.copy(); xi[3, 5] = np.inf
    assert st(x=xi) == "ENONFINITE"
    xs = x.copy(); xs[3, ids[3]] = -np.inf                # selected logit -inf
    assert st(x=xs) == "ENONFINITE"
    xo = x.copy(); xo[3, (ids[3] + 1) % V] = -np.inf      # another logit -inf: fine
    assert st(x=xo) == "OK"
    xp = x.copy(); xp[0, :] = np.nan                      # NaN on an inactive row: fine
    assert st(x=xp) == "OK"


def test_packed_validation():
    V, N = 9, 10
    x = RNG.standard_normal((N, V)).astype(np.float32)
    ids = np.arange(N) % V
    act = np.array([0, 1, 1, 0, 1, 1, 1, 0, 0, 0], np.uint8)
    ok = np.array([0, 3, 7], np.int32)
    f = lambda cu, a=act, att=None: oracle.selected_logprob(
        x, x, "f32", ids, att, a, V, "packed", cu_seqlens=cu)
    out = f(ok)
    assert out["status"] == "OK"
    assert np.array_equal(out["active"], act)
    assert f(np.array([1, 3, 7], np.int32))["status"] == "EMASK"
    assert f(np.array([0, 5, 3], np.int32))["status"] == "EMASK"
    assert f(np.array([0, 3, 11], np.int32))["status"] == "EMASK"
    tail = act.copy(); tail[8] = 1                        # action in the packed tail
    assert f(ok, a=tail)["status"] == "EMASK"
    att = (np.arange(N) < 7).astype(np.uint8)
    assert f(ok, att=att)["status"] == "OK"
    att2 = att.copy(); att2[2] = 0
    assert f(ok, att=att2)["status"] == "EMASK"


def test_bf16_path_widens_before_scoring():
    import torch
    V = 64
    xf = torch.randn(3, V) * 3
    xb = xf.to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    ids = np.array([1, 2, 3])
    out = oracle.selected_logprob(bits, bits, "bf16", ids, None, np.ones(3, np.uint8), V,
                                  "right", 1, 3)
    ref = torch.log_softmax(xb.double(), dim=1).numpy()
    for r in range(3):
        assert abs(out["train_logp"][r] - ref[r, ids[r]]) <= 1e-13


# --------------------------------------------------------------------------- mask + transforms

def test_transform_identities_and_closed_forms():
    x = RNG.standard_normal(500) * 3
    assert np.array_equal(oracle.apply_transforms(x, None), x)
    assert np.array_equal(oracle.apply_transforms(x, [("temperature", 1.0)]), x)
    assert np.array_equal(oracle.apply_transforms(x, [("scale", 2.0), ("temperature", 2.0)]), x)
    # soft cap: value * tanh(x / value), odd, bounded by the cap, ~x for |x| << cap
    y = oracle.apply_transforms(x, [("softcap", 5.0)])
    assert np.all(np.abs(y) < 5.0) and np.allclose(-y, oracle.apply_transforms(-x, [("softcap", 5.0)]))
    small = np.array([1e-4, -2e-4])
    assert np.allclose(oracle.apply_transforms(small, [("softcap", 30.0)]), small, rtol=1e-8)
    assert oracle.apply_transforms(np.array([15.0]), [("softcap", 30.0)])[0] == 30.0 * math.tanh(0.5)


def test_transform_order_matters_two_token_closed_form():
    """V = 2: logp(y) = -log1p(exp(f(x_o) - f(x_y))) for the chain f; scale-then-cap and
    cap-then-scale give different closed forms."""
    xy, xo = 4.0, -2.0
    f1 = lambda v: 10.0 * math.tanh((v * 3.0) / 10.0)     # scale 3 then cap 10
    f2 = lambda v: 3.0 * (10.0 * math.tanh(v / 10.0))     # cap 10 then scale 3
    row = np.array([xo, xy])
    for chain, f in (([("scale", 3.0), ("softcap", 10.0)], f1),
                     ([("softcap", 10.0), ("scale", 3.0)], f2)):
        z = oracle.apply_transforms(row, chain)
        got = z[1] - oracle.logsumexp_row(z)
        want = -math.log1p(math.exp(f(xo) - f(xy)))
        assert abs(got - want) <= 1e-14
    assert abs(f1(xy) - f2(xy)) > 1.0


def test_vocab_mask_excludes_padded_columns():
    N, V, Vr = 4, 40, 33
    x = RNG.standard_normal((N, V)).astype(np.float32)
    x[:, Vr:] = 50.0                                       # padded columns, huge logits
    ids = np.array([0, 5, 32, 17])
    act = np.ones(N, np.uint8)
    out = oracle.selected_logprob(x, x, "f32", ids, None, act, V, "right", 1, N, vocab_real=Vr)
    assert out["status"] == "OK"
    for r in range(N):
        want = _decimal_logp(x[r, :Vr].astype(np.float64), int(ids[r]))
        assert abs(out["train_logp"][r] - want) <= 1e-13
    inc = oracle.selected_logprob(x, x, "f32", ids, None, act, V, "right", 1, N)
    assert np.all(inc["train_logp"] < out["train_logp"] - 10)   # "include" sees the pad mass
    bad = ids.copy(); bad[1] = Vr                          # an id in the padded region
    assert oracle.selected_logprob(x, x, "f32", bad, None, act, V, "right", 1, N,
                                   vocab_real=Vr)["status"] == "ETOKEN"


def test_per_side_transforms_make_drift():
    """Same logits, temperature 1 on train and 2 on rollout: the closed form of a
    two-valued row."""
    V, a, b, y = 20, 3.0, 1.0, 0
    row = np.full((1, V), b, np.float32)
    row[0, y] = a
    out = oracle.selected_logprob(row, row, "f32", np.array([y]), None, np.ones(1, np.uint8), V,
                                  "right", 1, 1, transforms=(None, [("temperature", 2.0)]))
    lp = lambda aa, bb: aa - math.log(math.exp(aa) + (V - 1) * math.exp(bb))
    want = lp(a, b) - lp(a / 2, b / 2)
    assert abs(out["dlogp"][0] - want) <= 1e-14


def test_active_row_list_worked_example_and_properties():
    """The ascending active-row list: a hand-worked example, the edge cases, and the
    properties that define it (sorted, each active row once, nothing else)."""
    assert oracle.active_row_list([0, 1, 1, 0, 1]).tolist() == [1, 2, 4]
    assert oracle.active_row_list([]).tolist() == []
    assert oracle.active_row_list([0, 0, 0]).tolist() == []
    assert oracle.active_row_list([1, 1, 1]).tolist() == [0, 1, 2]
    assert oracle.active_row_list(np.array([0, 2, 0, 255], np.uint8)).tolist() == [1, 3]
    rng = np.random.default_rng(5)
    a = (rng.random(5003) < 0.3).astype(np.uint8)
    got = oracle.active_row_list(a)
    assert np.all(np.diff(got) > 0)
    assert len(got) == int(a.sum())
    assert np.all(a[got] == 1)
    assert np.array_equal(got, np.flatnonzero(a))
