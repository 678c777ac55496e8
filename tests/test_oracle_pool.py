"""The oracle's worker pool adds no arithmetic: rows scored through the shared buffer by
several workers equal, bit for bit, the same rows scored by one call in this process."""
import numpy as np

import oracle
from oracle.pool import OraclePool, default_workers


def _rows(rng, n, V, dtype):
    x = rng.normal(0.0, 3.0, size=(n, V)).astype(np.float32)
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    return x


def test_pool_matches_one_process():
    rng = np.random.default_rng(5)
    with OraclePool(workers=3) as pool:
        for dtype, n, V in (("bf16", 37, 1001), ("f32", 50, 257)):
            tr = _rows(rng, n, V, dtype)
            ro = _rows(rng, n, V, dtype)
            ids = rng.integers(0, V, size=n)
            bt, br = pool.buffers(n + 5, V, dtype)  # a buffer larger than the chunk
            bt[:n] = tr
            br[:n] = ro
            t, r, d, secs = pool.score(n, V, dtype, ids)
            wt, wr, wd = oracle.score_rows(tr, ro, dtype, ids)
            assert secs > 0
            for g, w in ((t, wt), (r, wr), (d, wd)):
                assert np.array_equal(g, w)


def test_default_workers_bounded():
    assert 1 <= default_workers() <= 16
