"""Oracle: active rows, logical-input validation, selected-token logprob and dlogp.

Test infrastructure only (see the package docstring). Plain float64 numpy, textbook
two-pass log-sum-exp; no blocking, fusion or reordering.

Readings where the pages leave a step open (each is listed with its reason in the design
notes of the repository):

* Rows are pre-shifted: the logits of row r score ``ids[r]``; nothing shifts ("[WS2]
  Framework for ablation experiment", LogProb knobs row 8, "pre-shifted input
  convention").
* Active rows are ``attention != 0 and action != 0``; the caller's action mask is 0 on
  prompt rows ("WS2 Cross-Config Logprob Drift Contract", Measurement Contract: only
  response/action tokens count; prompt, padding and masked response rows never do).
* The padding side never changes the arithmetic; it only fixes which attention-mask
  shapes are valid (Measurement Contract, "same padding layout semantics").
* All V columns enter the log-sum-exp (LogProb knobs row 2, policy "include"); inputs are
  final logits, no temperature or other transform (LogProb knobs row 7).
* A logical-input violation makes the comparison invalid, not noisy (Drift Source
  Taxonomy, "Logical Input and Metadata Drift"): it is reported as a status, with the
  priority EMASK > ETOKEN > ENONFINITE.
"""
from __future__ import annotations

import math

import numpy as np

# Symbolic statuses. The oracle reports names; tests map them to the library's codes.
STATUS = ("OK", "EMASK", "ETOKEN", "ENONFINITE")


def widen(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored logits to float64.

    bf16 values arrive as their uint16 bit patterns; a bf16 number is the upper half of
    the float32 with the same bits, so (u16 << 16) reinterpreted as float32 is exact.
    """
    if dtype == "bf16":
        u = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def logsumexp_row(x: np.ndarray) -> float:
    """Natural-log log-sum-exp of one row, textbook two-pass form:
    m = max_i x_i, lse = m + log(sum_i exp(x_i - m)).

    The log-softmax of the selected token is then x_y - lse ("[WS2] Framework for
    ablation experiment", LogProb knobs row 6 asks for an fp32-or-better reference; this
    one is float64, natural-log domain as in Attention knobs row 6).
    """
    x = np.asarray(x, dtype=np.float64)
    m = float(np.max(x))
    if m == -math.inf:
        return -math.inf
    with np.errstate(invalid="ignore", over="ignore"):
        return m + math.log(float(np.sum(np.exp(x - m))))


def active_rows(attention, action, N, layout, cu_seqlens=None) -> np.ndarray:
    """Active-row rule ("WS2 Cross-Config Logprob Drift Contract", Measurement Contract):
    a row counts only if it is a real (attended) row and an action/response row.
    Packed batches: rows at or beyond cu_seqlens[-1] are padding of the packed buffer."""
    att = np.ones(N, dtype=bool) if attention is None else (np.asarray(attention) != 0)
    act = np.ones(N, dtype=bool) if action is None else (np.asarray(action) != 0)
    if layout == "packed":
        end = int(np.clip(int(cu_seqlens[-1]), 0, N))
        att = att & (np.arange(N) < end)
    return att & act


def active_row_list(active) -> np.ndarray:
    """The active rows as a list in ascending order (the compaction of the Measurement
    Contract's active-token rule): every r with active[r] != 0, each once, smallest first."""
    a = np.asarray(active)
    return np.array([r for r in range(a.shape[0]) if a[r] != 0], dtype=np.int64)


def validate_inputs(attention, action, ids, V, N, layout, B=0, L=0, cu_seqlens=None):
    """Logical-input checks that make a comparison invalid rather than noisy.

    Returns the set of violated classes among {"EMASK", "ETOKEN"}.

    EMASK: a mask byte other than 0/1; an action row that is not attended; an attention
    mask that is not one contiguous block on the declared padding side (right: ones then
    zeros, left: zeros then ones, in every sequence); for packed batches, cu_seqlens not
    starting at 0, decreasing, or ending past the buffer, or an attention mask that is
    not exactly the rows before cu_seqlens[-1].
    ETOKEN: an active row whose selected id is outside [0, V) (LogProb knobs row 8,
    out-of-vocabulary targets, ignore_index on an active row).
    """
    errs = set()
    for m in (attention, action):
        if m is not None and np.any((np.asarray(m) != 0) & (np.asarray(m) != 1)):
            errs.add("EMASK")
    if layout == "packed":
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        if cu[0] != 0 or np.any(cu[1:] < cu[:-1]) or cu[-1] > N:
            errs.add("EMASK")
        end = int(np.clip(cu[-1], 0, N))
        real = np.arange(N) < end
        if attention is not None and np.any((np.asarray(attention) != 0) != real):
            errs.add("EMASK")
        att = real
    else:
        att = np.ones(N, dtype=bool) if attention is None else (np.asarray(attention) != 0)
        if attention is not None:
            a2 = att.reshape(B, L)
            for b in range(B):
                for t in range(L - 1):
                    if layout == "right" and (not a2[b, t]) and a2[b, t + 1]:
                        errs.add("EMASK")
                    if layout == "left" and a2[b, t] and (not a2[b, t + 1]):
                        errs.add("EMASK")
    if action is not None:
        act = np.asarray(action) != 0
        if np.any(act & ~att):
            errs.add("EMASK")
    act_rows = active_rows(attention, action, N, layout, cu_seqlens)
    ids = np.asarray(ids, dtype=np.int64)
    if np.any(act_rows & ((ids < 0) | (ids >= V))):
        errs.add("ETOKEN")
    return errs


# Logit transforms, applied element-wise in the order given, before the softmax ("[WS2]
# Framework for ablation experiment", LogProb knobs row 7: temperature, logit_scale,
# soft_cap as an ordered chain). Each step is (kind, value):
#   "scale"        x -> x * value
#   "temperature"  x -> x / value
#   "softcap"      x -> value * tanh(x / value)
TRANSFORMS = ("scale", "temperature", "softcap")


def apply_transforms(x, chain):
    """float64 logits after the ordered transform chain (None or [] = identity)."""
    x = np.asarray(x, dtype=np.float64)
    for kind, value in (chain or ()):
        v = float(value)
        if kind == "scale":
            x = x * v
        elif kind == "temperature":
            x = x / v
        elif kind == "softcap":
            x = v * np.tanh(x / v)
        else:
            raise ValueError(kind)
    return x


def score_row(train_row, rollout_row, y):
    """Per-row teacher-forced scoring of one active row with a valid id.

    logp = x_y - LSE(x) on each side; dlogp = train_recomputed_logp - rollout_old_logp
    ("WS2 Cross-Config Logprob Drift Contract", Measurement Contract), in float64.
    Returns (train_logp, rollout_logp, dlogp, nonfinite) where ``nonfinite`` marks a NaN
    or +inf logit on either side, or a selected logit of -inf (probability zero, so the
    logprob is not a finite number).
    """
    lt = logsumexp_row(train_row)
    lr = logsumexp_row(rollout_row)
    xt = float(train_row[y])
    xr = float(rollout_row[y])
    bad = (np.any(np.isnan(train_row)) or np.any(np.isnan(rollout_row))
           or np.any(train_row == math.inf) or np.any(rollout_row == math.inf)
           or xt == -math.inf or xr == -math.inf)
    lpt = xt - lt
    lpr = xr - lr
    return lpt, lpr, lpt - lpr, bool(bad)


def selected_logprob(train, rollout, dtype, ids, attention, action, V, layout,
                     B=0, L=0, cu_seqlens=None, vocab_real=None, transforms=(None, None)):
    """Whole-batch oracle.

    train, rollout: stored logits [N, >=V] (float32 or bf16 bit patterns as uint16).
    vocab_real: number of leading columns that enter the log-sum-exp (the "mask" vocab
    padding policy of LogProb knobs row 2); None = all V ("include"). Selected ids must
    lie below it. transforms: (train chain, rollout chain), see `apply_transforms`.
    Returns dict(train_logp, rollout_logp, dlogp: float64 [N], active: uint8 [N],
    status: str). Inactive rows carry 0.0; active rows with an out-of-range id carry NaN.
    """
    if vocab_real is not None:
        V = int(vocab_real)
    train = np.asarray(train)
    rollout = np.asarray(rollout)
    N = train.shape[0]
    errs = validate_inputs(attention, action, ids, V, N, layout, B, L, cu_seqlens)
    act = active_rows(attention, action, N, layout, cu_seqlens)
    out_t = np.zeros(N)
    out_r = np.zeros(N)
    out_d = np.zeros(N)
    ids64 = np.asarray(ids, dtype=np.int64)
    for r in np.nonzero(act)[0]:
        y = int(ids64[r])
        if not (0 <= y < V):
            out_t[r] = out_r[r] = out_d[r] = math.nan
            continue
        xt = apply_transforms(widen(train[r, :V], dtype), transforms[0])
        xr = apply_transforms(widen(rollout[r, :V], dtype), transforms[1])
        lpt, lpr, d, bad = score_row(xt, xr, y)
        out_t[r], out_r[r], out_d[r] = lpt, lpr, d
        if bad:
            errs.add("ENONFINITE")
    status = "OK"
    for s in ("EMASK", "ETOKEN", "ENONFINITE"):
        if s in errs:
            status = s
            break
    return {"train_logp": out_t, "rollout_logp": out_r, "dlogp": out_d,
            "active": act.astype(np.uint8), "status": status}


def score_rows(train_rows, rollout_rows, dtype, ids_rows, vocab_real=None,
               transforms=(None, None)):
    """Oracle on a sample of active rows (rows already known valid): returns float64
    arrays (train_logp, rollout_logp, dlogp). Used at full sizes, where only sampled rows
    are copied to the host."""
    k = len(ids_rows)
    t = np.empty(k)
    r = np.empty(k)
    d = np.empty(k)
    for i in range(k):
        V = train_rows.shape[1] if vocab_real is None else int(vocab_real)
        xt = apply_transforms(widen(train_rows[i][:V], dtype), transforms[0])
        xr = apply_transforms(widen(rollout_rows[i][:V], dtype), transforms[1])
        t[i], r[i], d[i], _ = score_row(xt, xr, int(ids_rows[i]))
    return t, r, d
