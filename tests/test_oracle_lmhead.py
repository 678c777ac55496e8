"""Pins of the LM-head oracle (CPU only): zero weights give -ln V, 50-digit brute force on
non-square shapes (a transposed operand cannot pass), and agreement with the logits oracle
when the logits are formed explicitly."""
import math
from decimal import Decimal, getcontext

import numpy as np
import torch

import oracle

RNG = np.random.default_rng(7)


def _bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_zero_weight_gives_minus_log_V():
    T, H, V = 5, 8, 13
    h = _bf16_bits(torch.randn(T, H))
    w = np.zeros((H, V))
    lp = oracle.lmhead_logprob(h, w, np.arange(T) % V)
    assert np.all(np.abs(lp + math.log(V)) <= 1e-15)


def test_brute_force_non_square():
    getcontext().prec = 50
    T, H, V = 3, 5, 7
    h = _bf16_bits(torch.randn(T, H))
    hw = oracle.widen(h, "bf16")
    w = RNG.standard_normal((H, V)) * 0.7
    ids = np.array([6, 0, 3])
    got = oracle.lmhead_logprob(h, w, ids)
    for t in range(T):
        z = [sum((Decimal(float(hw[t, k])) * Decimal(float(w[k, v])) for k in range(H)),
                 Decimal(0)) for v in range(V)]
        lse = sum((zz.exp() for zz in z), Decimal(0)).ln()
        assert abs(got[t] - float(z[ids[t]] - lse)) <= 1e-13


def test_row_subset_matches_full():
    T, H, V = 40, 16, 50
    h = _bf16_bits(torch.randn(T, H))
    w = RNG.standard_normal((H, V)) * 0.3
    ids = RNG.integers(0, V, T)
    full = oracle.lmhead_logprob(h, w, ids, chunk=7)
    sub = oracle.lmhead_logprob(h, w, ids, rows=[39, 0, 17])
    assert np.array_equal(sub, full[[39, 0, 17]])


def test_chain_two_columns_closed_form():
    """With V = 2 the selected logprob is -log1p(exp(z_other - z_y)) of the transformed
    logits; here a soft-cap of 3 after a scale of 2 on hand-made logits (hidden one-hot, so
    z is a column of W)."""
    H, V = 4, 2
    h = np.zeros((2, H), dtype=np.uint16)
    h[0, 1] = 0x3F80                       # bf16 1.0 at k = 1
    h[1, 3] = 0x3F80                       # bf16 1.0 at k = 3
    w = np.zeros((H, V))
    w[1] = [0.5, -1.25]
    w[3] = [4.0, 7.5]
    chain = [("scale", 2.0), ("softcap", 3.0)]
    got = oracle.lmhead_logprob(h, w, np.array([0, 1]), transforms=chain)
    cap = lambda v: 3.0 * math.tanh(2.0 * v / 3.0)
    want0 = -math.log1p(math.exp(cap(-1.25) - cap(0.5)))
    want1 = -math.log1p(math.exp(cap(4.0) - cap(7.5)))
    assert abs(got[0] - want0) <= 1e-15 and abs(got[1] - want1) <= 1e-15


def test_chain_matches_the_logits_oracle():
    """The head with a chain equals the logits oracle on the materialised logits with the
    same chain (a different code path through score_rows)."""
    T, H, V = 6, 8, 40
    # small multiples of 1/8 and 1/64, so every logit is exact in fp32 and the logits
    # oracle (which takes fp32 rows) sees the same values
    h = _bf16_bits(torch.from_numpy(RNG.integers(-16, 17, (T, H)) / 8.0).float())
    w = RNG.integers(-64, 65, (H, V)) / 64.0
    ids = RNG.integers(0, V, T)
    chain = [("temperature", 0.7), ("softcap", 5.0)]
    got = oracle.lmhead_logprob(h, w, ids, transforms=chain)
    z = oracle.widen(h, "bf16") @ w
    assert np.array_equal(z.astype(np.float32).astype(np.float64), z)
    z32 = z.astype(np.float32)
    want = oracle.score_rows(z32, z32, "f32", ids, transforms=(chain, chain))[0]
    assert np.max(np.abs(got - want)) <= 1e-13
