"""Pins of the vocab-shard oracle (CPU only): the merged LSE of any partition equals the
textbook logsumexp of the whole row (scipy), closed forms, owner uniqueness, -inf and NaN
shards."""
import math

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(99)


def _partitions(V):
    yield [0, V]
    yield [0, V // 2, V]
    if V > 24:
        yield [0, 8, 16, V - 8, V]
    cuts = np.sort(RNG.choice(np.arange(1, V), min(6, V - 1), replace=False))
    yield [0, *cuts.tolist(), V]
    yield [0, 0, V // 3, V // 3, V]                 # empty shards


@pytest.mark.parametrize("V", [2, 37, 1000, 151936])
def test_merged_lse_equals_whole_row_logsumexp(V):
    from scipy.special import logsumexp
    x = RNG.standard_normal(V) * 4
    want = float(logsumexp(x))
    for b in _partitions(V):
        parts = [oracle.shard_partial(x, b[i], b[i + 1]) for i in range(len(b) - 1)]
        got = oracle.merge_partials(parts)
        assert abs(got - want) <= 1e-13 * max(1.0, abs(want)), (b, got, want)


def test_uniform_rows_and_single_owner():
    V = 4096
    x = np.full(V, 0.75)
    for b in _partitions(V):
        parts = [oracle.shard_partial(x, b[i], b[i + 1]) for i in range(len(b) - 1)]
        assert abs(oracle.merge_partials(parts) - (0.75 + math.log(V))) <= 1e-12
        for y in (0, 1, V // 2, V - 1):
            s = oracle.owner_of(y, b)
            assert b[s] <= y < b[s + 1]
            assert sum(1 for i in range(len(b) - 1) if b[i] <= y < b[i + 1]) == 1
    assert oracle.owner_of(V, [0, V]) == -1 and oracle.owner_of(-1, [0, V]) == -1


def test_minus_inf_and_nan_shards():
    x = RNG.standard_normal(64)
    x[:32] = -np.inf
    assert oracle.shard_partial(x, 0, 32) == (-math.inf, 0.0)
    parts = [oracle.shard_partial(x, 0, 32), oracle.shard_partial(x, 32, 64)]
    from scipy.special import logsumexp
    assert abs(oracle.merge_partials(parts) - float(logsumexp(x[32:]))) <= 1e-13
    assert oracle.merge_partials([(-math.inf, 0.0)]) == -math.inf
    x[40] = np.nan
    assert math.isnan(oracle.merge_partials([oracle.shard_partial(x, 32, 64)]))


def test_sharded_rows_equal_unsharded_rows():
    V, k = 3001, 6
    tr = (RNG.standard_normal((k, V)) * 2).astype(np.float32)
    ro = (tr + RNG.standard_normal((k, V)).astype(np.float32) * 1e-3).astype(np.float32)
    ids = RNG.integers(0, V - 1, k)
    chain = ([("softcap", 20.0)], [("temperature", 0.9)])
    want = oracle.score_rows(tr, ro, "f32", ids, vocab_real=V - 1, transforms=chain)
    for b in ([0, V], [0, 1000, 2000, V], [0, 8, V - 1, V]):
        got = oracle.sharded_score_rows(tr, ro, "f32", ids, b, vocab_real=V - 1,
                                        transforms=chain)
        for g, w in zip(got, want):
            assert np.abs(g - w).max() <= 1e-12
    # an id that no shard owns gives NaN
    t, _, _ = oracle.sharded_score_rows(tr[:1], ro[:1], "f32", [V - 1], [0, V], vocab_real=V - 1)
    assert math.isnan(t[0])
