"""Pins of the entropy and dlogits oracle (CPU only): closed forms, 50-digit brute force,
scipy's entropy, torch autograd of log_softmax, invariants."""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(77)


@pytest.mark.parametrize("V", [1, 2, 5, 1024, 151936])
def test_uniform_entropy_is_log_V(V):
    assert abs(oracle.entropy_row(np.full(V, 1.25)) - math.log(V)) <= 1e-12 * max(1, math.log(V))


def test_two_valued_entropy_closed_form():
    V, k, a, b = 100, 7, 2.0, -1.0
    x = np.full(V, b)
    x[:k] = a
    Z = k * math.exp(a) + (V - k) * math.exp(b)
    pa, pb = math.exp(a) / Z, math.exp(b) / Z
    want = -(k * pa * math.log(pa) + (V - k) * pb * math.log(pb))
    assert abs(oracle.entropy_row(x) - want) <= 1e-13


def test_entropy_against_scipy_and_decimal():
    from scipy.stats import entropy as sp_entropy
    getcontext().prec = 50
    for V in (3, 17, 64, 4096):
        x = RNG.standard_normal(V) * 3
        p, _ = oracle.softmax_row(x)
        assert abs(oracle.entropy_row(x) - float(sp_entropy(p))) <= 1e-12
        if V <= 64:
            xs = [Decimal(float(v)) for v in x]
            Zd = sum((v.exp() for v in xs), Decimal(0))
            Hd = -sum(((v.exp() / Zd) * (v.exp() / Zd).ln() for v in xs), Decimal(0))
            assert abs(oracle.entropy_row(x) - float(Hd)) <= 1e-13


def test_entropy_minus_inf_terms_and_peaked_limit():
    x = RNG.standard_normal(50)
    xm = x.copy()
    xm[:10] = -np.inf
    assert abs(oracle.entropy_row(xm) - oracle.entropy_row(x[10:])) <= 1e-13
    peaked = np.zeros(1000)
    peaked[3] = 60.0
    assert 0.0 <= oracle.entropy_row(peaked) < 1e-20


def test_dlogits_against_torch_autograd_and_invariants():
    import torch
    for V in (2, 33, 5000):
        x = RNG.standard_normal(V) * 2
        y = int(RNG.integers(0, V))
        xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
        torch.log_softmax(xt, dim=0)[y].backward()
        g = oracle.dlogits_row(x, y)
        assert np.abs(g - xt.grad.numpy()).max() <= 1e-14
        assert abs(math.fsum(g.tolist())) <= 1e-13          # rows sum to zero
        assert g[y] > 0 and np.all(np.delete(g, y) <= 0)
    # V = 2 closed form: g_y = 1 - sigmoid(x_y - x_o) = sigmoid(x_o - x_y)
    x = np.array([0.3, -1.1])
    g = oracle.dlogits_row(x, 0)
    s = 1.0 / (1.0 + math.exp(-(x[1] - x[0])))
    assert abs(g[0] - s) <= 1e-15 and abs(g[1] + s) <= 1e-15


CHAINS = [None, [("temperature", 0.7)], [("scale", -1.3)], [("softcap", 3.0)],
          [("scale", 2.0), ("softcap", 5.0), ("temperature", 1.5)],
          [("softcap", 30.0), ("temperature", 0.9), ("scale", 0.5), ("softcap", 2.0)]]


@pytest.mark.parametrize("chain", CHAINS)
def test_chain_derivative_against_central_differences(chain):
    # independent of the analytic form: (f(x+h) - f(x-h)) / 2h with the forward chain
    x = RNG.standard_normal(200) * 4
    h = 1e-6
    fd = (oracle.apply_transforms(x + h, chain) - oracle.apply_transforms(x - h, chain)) / (2 * h)
    d = oracle.chain_derivative(x, chain)
    assert np.abs(d - fd).max() <= 1e-7 * max(1.0, np.abs(d).max())


@pytest.mark.parametrize("chain", CHAINS)
def test_dlogits_rows_against_torch_autograd(chain):
    import torch
    N, V, Vr = 5, 40, 33
    x = (RNG.standard_normal((N, V)) * 3).astype(np.float32)
    ids = RNG.integers(0, Vr, N)
    active = np.array([1, 0, 1, 1, 1], dtype=np.uint8)
    grad = RNG.standard_normal(N)
    xt = torch.tensor(x.astype(np.float64), requires_grad=True)
    z = xt[:, :Vr]
    for kind, v in (chain or ()):
        z = z * v if kind == "scale" else z / v if kind == "temperature" else v * torch.tanh(z / v)
    lp = torch.log_softmax(z, dim=1).gather(1, torch.tensor(ids).view(-1, 1)).view(-1)
    loss = (lp * torch.tensor(grad * active)).sum()
    loss.backward()
    got = oracle.dlogits_rows(x, "f32", ids, active, vocab_real=Vr, transform=chain,
                              grad=grad)
    assert np.abs(got - xt.grad.numpy()).max() <= 1e-13
    assert np.all(got[1] == 0) and np.all(got[:, Vr:] == 0)


def test_dlogits_rows_edge_cases():
    V = 16
    x = RNG.standard_normal((3, V)).astype(np.float32)
    ids = np.array([3, V, -1])                     # valid, past the end, negative
    g = oracle.dlogits_rows(x, "f32", ids, np.ones(3, np.uint8))
    assert np.all(np.isfinite(g[0])) and np.all(np.isnan(g[1])) and np.all(np.isnan(g[2]))
    # an id inside V but past vocab_real is rejected too
    g = oracle.dlogits_rows(x, "f32", np.array([12, 0, 0]), np.ones(3, np.uint8),
                            vocab_real=12)
    assert np.all(np.isnan(g[0, :12])) and np.all(g[0, 12:] == 0)
    # a zero upstream gradient gives an exact zero row; -inf logits get exactly 0
    x[1, :4] = -np.inf
    g = oracle.dlogits_rows(x, "f32", np.array([5, 5, 5]), np.ones(3, np.uint8),
                            grad=np.array([0.0, 1.0, 2.0]))
    assert np.all(g[0] == 0) and np.all(g[1, :4] == 0)
    assert np.allclose(g[2], 2.0 * oracle.dlogits_row(x[2].astype(np.float64), 5), rtol=0,
                       atol=1e-15)


def test_entropy_rows_with_temperature_and_mask():
    # a very high temperature flattens any row to the uniform law: H -> ln Vr
    x = RNG.standard_normal((2, 50)).astype(np.float32)
    H = oracle.entropy_rows(x, "f32", vocab_real=40, transform=[("temperature", 1e9)])
    assert np.abs(H - math.log(40)).max() <= 1e-9
    # two-valued row under a soft cap: closed form with the capped values
    V, k, a, b, c = 64, 5, 9.0, -2.0, 4.0
    row = np.full(V, b, np.float32)
    row[:k] = a
    za, zb = c * math.tanh(a / c), c * math.tanh(b / c)
    Z = k * math.exp(za) + (V - k) * math.exp(zb)
    pa, pb = math.exp(za) / Z, math.exp(zb) / Z
    want = -(k * pa * math.log(pa) + (V - k) * pb * math.log(pb))
    got = oracle.entropy_rows(row[None], "f32", transform=[("softcap", c)])[0]
    assert abs(got - want) <= 1e-13
