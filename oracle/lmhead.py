"""Oracle: fused LM-head selected-token logprob.

Test infrastructure only (see the package docstring).

The logits of row t are z_t = hidden_t . W (W stored [H, V], vocabulary contiguous), the
head GEMM that runs before any softmax ("[WS2] Framework for ablation experiment", LogProb
knobs row 9, "LM-head GEMM and materialization boundary"). The selected logprob is then
z_t[y_t] - LSE(z_t), exactly as for given logits (rows 6, 8 and 10 of the same table).

The product is taken in float64 with numpy's matmul (a library primitive), in row chunks;
nothing else is blocked or reordered. An optional transform chain (temperature, logit scale,
soft-cap; row 7 of the same table) is applied to the head's logits before the softmax, as
for given logits.
"""
from __future__ import annotations

import numpy as np

from .logprob import apply_transforms, logsumexp_row, widen


def lmhead_logprob(hidden_bits, weight_f64, ids, rows=None, chunk=256, transforms=None):
    """hidden_bits: bf16 bit patterns [T, H] (uint16); weight_f64: W widened to float64
    [H, V]; ids: int [T]. ``rows``: optional subset of rows to score. ``transforms``: an
    optional chain applied to every row's logits (``apply_transforms``).
    Returns float64 logp for the chosen rows (all rows when ``rows`` is None)."""
    T = hidden_bits.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    out = np.empty(len(rows))
    for a in range(0, len(rows), chunk):
        sel = rows[a: a + chunk]
        h = widen(hidden_bits[sel], "bf16")
        z = apply_transforms(h @ weight_f64, transforms)
        for i, r in enumerate(sel):
            out[a + i] = z[i, int(ids[r])] - logsumexp_row(z[i])
    return out
