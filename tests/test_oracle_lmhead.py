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
