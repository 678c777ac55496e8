"""Oracle: training-side state of the selected-token logprob ("[WS2] Framework for ablation
experiment", LogProb knobs row 11: entropy reduction and dlogits).

Test infrastructure only (see the package docstring). float64, textbook forms:

* entropy of the softmax of a row: H = -sum_i p_i log p_i with p = softmax(x); terms with
  p_i = 0 (x_i = -inf) contribute 0;
* dlogits of the selected logprob: d(x_y - LSE(x)) / dx_v = [v == y] - p_v;
* through a transform chain z = chain(x) (LogProb knobs row 7) the chain rule multiplies
  by dz_v/dx_v, the product of each step's derivative at its own input: a scale step by
  its value, a temperature step by 1/value, a soft cap v*tanh(x/v) by 1 - tanh(x/v)^2.
* a padded vocabulary (row 2, "mask") excludes the columns past vocab_real from the
  softmax; their gradient is 0.
"""
from __future__ import annotations

import math

import numpy as np

from .logprob import apply_transforms, logsumexp_row, widen


def softmax_row(x):
    x = np.asarray(x, dtype=np.float64)
    lse = logsumexp_row(x)
    with np.errstate(invalid="ignore", over="ignore"):
        return np.exp(x - lse), lse


def entropy_row(x) -> float:
    p, lse = softmax_row(x)
    x = np.asarray(x, dtype=np.float64)
    nz = p > 0
    return -math.fsum((p[nz] * (x[nz] - lse)).tolist())


def dlogits_row(x, y):
    p, _ = softmax_row(x)
    g = -p
    g[int(y)] += 1.0
    return g


def chain_derivative(x, chain):
    """float64 dz/dx of the ordered transform chain at x (None or [] = identity)."""
    x = np.asarray(x, dtype=np.float64)
    d = np.ones_like(x)
    for kind, value in (chain or ()):
        v = float(value)
        if kind == "scale":
            d = d * v
            x = x * v
        elif kind == "temperature":
            d = d / v
            x = x / v
        elif kind == "softcap":
            t = np.tanh(x / v)
            d = d * (1.0 - t * t)
            x = v * t
        else:
            raise ValueError(kind)
    return d


def dlogits_rows(rows, dtype, ids, active, vocab_real=None, transform=None, grad=None):
    """Gradient of each row's selected logprob with respect to its stored logits.

    rows: stored logits [N, V] ("f32", or "bf16" bit patterns); ids [N]; active [N] (0/1);
    grad: upstream dL/dlogp per row (None = 1). Inactive rows are 0; an active row with an
    id outside [0, vocab_real) is NaN on [0, vocab_real) (the forward pass rejects it)."""
    rows = np.asarray(rows)
    N, V = rows.shape
    Vr = V if vocab_real is None else int(vocab_real)
    out = np.zeros((N, V))
    for r in range(N):
        if not active[r]:
            continue
        y = int(ids[r])
        if not 0 <= y < Vr:
            out[r, :Vr] = np.nan
            continue
        x = widen(rows[r, :Vr], dtype)
        z = apply_transforms(x, transform)
        g = dlogits_row(z, y) * chain_derivative(x, transform)
        out[r, :Vr] = g * (1.0 if grad is None else float(grad[r]))
    return out


def entropy_rows(rows, dtype, vocab_real=None, transform=None):
    """Entropy of each stored row (float32 or bf16 bit patterns)."""
    out = np.empty(len(rows))
    for i, r in enumerate(rows):
        V = len(r) if vocab_real is None else int(vocab_real)
        out[i] = entropy_row(apply_transforms(widen(r[:V], dtype), transform))
    return out
