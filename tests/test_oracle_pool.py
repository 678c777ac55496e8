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


def test_pool_entropy_and_lse_match_one_process():
    rng = np.random.default_rng(6)
    chain = [("softcap", 5.0)]
    with OraclePool(workers=3) as pool:
        for dtype, n, V, tr in (("bf16", 29, 1001, (None, None)), ("f32", 40, 257, (chain, None))):
            a = _rows(rng, n, V, dtype)
            b = _rows(rng, n, V, dtype)
            bt, br = pool.buffers(n + 3, V, dtype)
            bt[:n] = a
            br[:n] = b
            et, er, lt, lr = pool.entropy(n, V, dtype, transforms=tr)
            assert np.array_equal(et, oracle.entropy_rows(a, dtype, None, tr[0]))
            assert np.array_equal(er, oracle.entropy_rows(b, dtype, None, tr[1]))
            for got, rows, c in ((lt, a, tr[0]), (lr, b, tr[1])):
                want = [oracle.logsumexp_row(oracle.apply_transforms(oracle.widen(r, dtype), c))
                        for r in rows]
                assert np.array_equal(got, np.array(want))


def test_pool_dlogits_excess():
    """Side 1 holding the oracle's own gradient rounded to bf16 stays within half a bf16 ulp
    of it (excess <= 0 with c = 2^-8); one planted wrong element shows in its row only."""
    rng = np.random.default_rng(7)
    n, V = 23, 515
    x = _rows(rng, n, V, "bf16")
    ids = rng.integers(0, V, size=n)
    want = oracle.dlogits_rows(x, "bf16", ids, np.ones(n, np.uint8))
    w32 = want.astype(np.float32)
    bits = ((w32.view(np.uint32) + 0x7FFF + ((w32.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    with OraclePool(workers=3) as pool:
        bt, br = pool.buffers(n, V, "bf16")
        bt[:] = x
        br[:] = bits
        ex, ey = pool.dlogits_excess(n, V, "bf16", "bf16", ids, 2.0 ** -8)
        assert ex.shape == ey.shape == (n,) and np.all(ex <= 0.0) and np.all(ey <= 0.0)
        col = (int(ids[4]) + 9) % V
        br[4, col] ^= np.uint16(0x4000)     # a large error in one other element of row 4
        br[7, int(ids[7])] ^= np.uint16(0x4000)  # and one at row 7's selected column
        ex, ey = pool.dlogits_excess(n, V, "bf16", "bf16", ids, 2.0 ** -8)
        assert ex[4] > 0.1 and np.all(np.delete(ex, 4) <= 0.0)
        assert ey[7] > 0.1 and np.all(np.delete(ey, 7) <= 0.0)
