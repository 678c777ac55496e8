"""Oracle: vocab-parallel selected logprob, shard partials merged in global shard order.

Test infrastructure only (see the package docstring).

Follows "[WS2] Framework for ablation experiment", LogProb knobs rows 3-5 and 8: each rank
owns the vocabulary columns [vocab_start, vocab_end) of every row; it reports per row a
log-sum-exp partial over its columns and, if it owns the selected id, the selected logit
(single-owner gather); the partials of all ranks are gathered and merged in the order of
the global shard index (the allgather_partials_fixed_merge topology), and the logprob is
the owner's selected logit minus the merged LSE. float64 throughout:

* partial of columns x[a:b]:  (m, z) = (max x, sum exp(x - m)); (-inf, 0) if every
  column is -inf or the range is empty;
* merge of (m_s, z_s), s = 0..S-1:  M = max m_s, LSE = M + log(sum_s z_s exp(m_s - M)).

Mathematically LSE equals the unsharded logsumexp of the row for every partition.
"""
from __future__ import annotations

import math

import numpy as np

from .logprob import apply_transforms, widen


def shard_partial(x, start: int, end: int):
    """(m, z) of the float64 row x over columns [start, end)."""
    seg = np.asarray(x, dtype=np.float64)[start:end]
    if seg.size == 0 or np.all(seg == -math.inf):
        return -math.inf, 0.0
    m = float(np.max(seg))
    if math.isnan(m) or m == math.inf:
        return m, math.nan
    return m, math.fsum(np.exp(seg - m).tolist())


def merge_partials(parts):
    """Merged natural-log LSE of partials [(m_s, z_s)] taken in shard order."""
    ms = [m for m, _ in parts]
    if any(math.isnan(m) or m == math.inf for m in ms):
        return math.nan
    live = [(m, z) for m, z in parts if m > -math.inf]
    if not live:
        return -math.inf
    M = max(m for m, _ in live)
    return M + math.log(math.fsum(z * math.exp(m - M) for m, z in live))


def owner_of(y: int, boundaries) -> int:
    """Index of the shard [b_s, b_{s+1}) that owns column y, or -1."""
    for s in range(len(boundaries) - 1):
        if boundaries[s] <= y < boundaries[s + 1]:
            return s
    return -1


def sharded_score_rows(train_rows, rollout_rows, dtype, ids, boundaries, vocab_real=None,
                       transforms=(None, None)):
    """Per-row (train_logp, rollout_logp, dlogp) of valid active rows through shard
    partials over the column boundaries b_0 = 0 < ... <= b_S (columns at or past
    vocab_real never enter). The selected logit comes from its single owner."""
    k = len(ids)
    out = np.empty((3, k))
    for i in range(k):
        V = train_rows.shape[1] if vocab_real is None else int(vocab_real)
        y = int(ids[i])
        s = owner_of(y, boundaries)
        if s < 0 or y >= V:
            out[:, i] = math.nan
            continue
        lps = []
        for side, rows in enumerate((train_rows, rollout_rows)):
            x = apply_transforms(widen(rows[i][:V], dtype), transforms[side])
            parts = [shard_partial(x, min(boundaries[j], V), min(boundaries[j + 1], V))
                     for j in range(len(boundaries) - 1)]
            lse = merge_partials(parts)
            lps.append(float(x[y]) - lse)
        out[0, i], out[1, i] = lps
        out[2, i] = lps[0] - lps[1]
    return out[0], out[1], out[2]
