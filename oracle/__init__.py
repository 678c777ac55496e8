"""fp64 CPU oracle of the selected-token logprob drift contract.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute this
package: only the tests, the smoke check of the entry module and the CPU-baseline leg of
the benchmark use it. It shares no code, tables or helpers with the HIP library.

It is a plain, slow, textbook implementation in float64 numpy / Python:

* ``logprob``     - active-row rule and the ascending active-row list, logical-input
                    validation, two-pass log-sum-exp,
                    selected-logit gather and dlogp (page "WS2 Cross-Config Logprob Drift
                    Contract", section "Measurement Contract"; page "[WS2] Framework for
                    ablation experiment", LogProb knobs rows 2, 6, 8), the vocab-padding
                    mask (row 2) and the ordered logit transform chain (row 7).
* ``diagnostics`` - ratio0, clipfrac0, approx_kl0, mismatch_kl and mean/p95/p99/max
                    |dlogp| (page "WS2 Cross-Config Logprob Drift Contract", section
                    "Diagnostics" table; "Attention Debug Matrix", Metrics), whole batch and
                    per segment.
* ``lmhead``      - hidden x W_vocab followed by the same log-softmax gather (page "[WS2]
                    Framework for ablation experiment", LogProb knobs rows 9 and 10).
* ``training``    - entropy of the softmax and dlogits of the selected logprob (LogProb
                    knobs row 11).
* ``sharding``    - vocab-shard partials and their merge in global shard order (LogProb
                    knobs rows 3-5, single-owner gather of row 8).

Each function is pinned by tests against closed forms, brute force at 50 decimal digits
and textbook library routines; none is "parity unpinned".
"""
from .logprob import (STATUS, widen, logsumexp_row, selected_logprob, validate_inputs,
                      active_rows, active_row_list, score_row, score_rows, apply_transforms,
                      TRANSFORMS)
from .diagnostics import diagnostics, nearest_rank, segment_diagnostics
from .lmhead import lmhead_logprob
from .sharding import merge_partials, owner_of, shard_partial, sharded_score_rows
from .training import (chain_derivative, dlogits_row, dlogits_rows, entropy_row, entropy_rows,
                       softmax_row)

__all__ = ["STATUS", "widen", "logsumexp_row", "selected_logprob", "validate_inputs",
           "active_rows", "active_row_list", "score_row", "score_rows", "apply_transforms", "TRANSFORMS", "diagnostics", "nearest_rank", "segment_diagnostics", "lmhead_logprob",
           "shard_partial", "merge_partials", "owner_of", "sharded_score_rows",
           "entropy_row", "entropy_rows", "dlogits_row", "dlogits_rows", "chain_derivative",
           "softmax_row"]
