"""Runs the oracle's per-row functions over many rows in a pool of CPU worker processes.

Test infrastructure only (see the package docstring): the full-size parity tests and the
CPU-baseline leg of the benchmark use it. It adds no arithmetic of its own: every row is
scored by `score_rows` of this package (textbook two-pass log-sum-exp in float64), its
entropy by `entropy_rows` and its log-sum-exp by `logsumexp_row`, its gradient by
`dlogits_rows`, one call per contiguous range of rows, and the results are put back in row
order. For the gradient the workers also compare it with a given array (so that no
[rows, V] float64 array travels back): per row, the largest |got - want| - c |want| over
the other columns, and the same quantity at the selected column.

Rows reach the workers through a shared host buffer: the caller writes a chunk of rows of
both sides into a memory-mapped file (in /dev/shm when it has room, else the temporary
directory) and the workers map the same file read-only, so no row is pickled or sent
through a pipe. The pool uses the "spawn" start method: its workers are fresh
interpreters that import only numpy and this package, whatever the parent process has
initialised (create the pool before the parent touches a GPU all the same).
"""
from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile
import time

import numpy as np

# Worker processes at most: the host share that goes with one GPU on the machines this
# runs on, whatever the affinity mask lists.
MAX_WORKERS = 16

_NP = {"bf16": np.uint16, "f32": np.float32}


def default_workers() -> int:
    """Workers for this host: the CPUs this process may run on, at most MAX_WORKERS."""
    return max(1, min(len(os.sched_getaffinity(0)), MAX_WORKERS))


def _score_range(task):
    """Worker body: score rows [lo, hi) of the shared buffer with the oracle."""
    from .logprob import score_rows

    path, rows, cols, dtype, lo, hi, ids, vocab_real, transforms = task
    t0 = time.perf_counter()
    mm = np.memmap(path, dtype=_NP[dtype], mode="r", shape=(2, rows, cols))
    t, r, d = score_rows(mm[0, lo:hi], mm[1, lo:hi], dtype, ids, vocab_real, transforms)
    del mm
    return lo, t, r, d, time.perf_counter() - t0


def _entropy_range(task):
    """Worker body: entropy and natural-log log-sum-exp of rows [lo, hi) of both sides."""
    from .logprob import apply_transforms, logsumexp_row, widen
    from .training import entropy_rows

    path, rows, cols, dtype, lo, hi, vocab_real, transforms = task
    mm = np.memmap(path, dtype=_NP[dtype], mode="r", shape=(2, rows, cols))
    V = cols if vocab_real is None else int(vocab_real)
    ent, lse = [], []
    for s in (0, 1):
        part = mm[s, lo:hi]
        ent.append(entropy_rows(part, dtype, vocab_real, transforms[s]))
        lse.append(np.array([logsumexp_row(apply_transforms(widen(r[:V], dtype), transforms[s]))
                             for r in part]))
    del mm
    return lo, ent + lse  # entropy train, rollout; lse train, rollout


def _dlogits_range(task):
    """Worker body: the oracle's gradient of rows [lo, hi) (side 0 of the buffer holds the
    logits, side 1 the gradient to compare, both in the stored type), and per row the
    largest |got - want| - c |want| over the columns other than the selected one, and that
    quantity at the selected column."""
    from .logprob import widen
    from .training import dlogits_rows

    path, rows, cols, dtype, out_dtype, lo, hi, ids, c, vocab_real, transform = task
    mm = np.memmap(path, dtype=_NP[dtype], mode="r", shape=(2, rows, cols))
    want = dlogits_rows(mm[0, lo:hi], dtype, ids, np.ones(hi - lo, np.uint8), vocab_real,
                        transform)
    got = widen(mm[1, lo:hi], out_dtype).reshape(want.shape)
    del mm
    ex = np.abs(got - want) - c * np.abs(want)
    k = np.arange(hi - lo)
    y = np.asarray(ids, dtype=np.int64)
    at_y = ex[k, y].copy()
    ex[k, y] = -np.inf
    return lo, ex.max(axis=1), at_y


class OraclePool:
    """A pool of oracle workers and one shared row buffer (both sides, sized by the last
    `buffers` call).

        with OraclePool() as pool:
            tr, ro = pool.buffers(n, V, "bf16")   # numpy views to fill with raw rows
            ...                                   # copy n rows of each side into them
            t, r, d, secs = pool.score(n, V, "bf16", ids)
    """

    def __init__(self, workers: int | None = None):
        self.workers = workers or default_workers()
        self._pool = mp.get_context("spawn").Pool(self.workers)
        self._dir = None
        self._path = None
        self._shape = None
        self._mm = None

    # -- shared buffer ------------------------------------------------------------------
    def _place(self, nbytes):
        for d in ("/dev/shm", tempfile.gettempdir()):
            try:
                st = os.statvfs(d)
            except OSError:
                continue
            if st.f_bavail * st.f_frsize >= 2 * nbytes:
                return d
        return tempfile.gettempdir()

    def buffers(self, rows: int, cols: int, dtype: str):
        """Writable [rows, cols] views (train, rollout) of the shared buffer, in the stored
        element type (float32, or uint16 bit patterns for bf16)."""
        shape = (2, rows, cols)
        if self._shape != (shape, dtype):
            self._release()
            nbytes = 2 * rows * cols * np.dtype(_NP[dtype]).itemsize
            self._dir = tempfile.mkdtemp(prefix="oracle_rows_", dir=self._place(nbytes))
            self._path = os.path.join(self._dir, "rows.bin")
            self._mm = np.memmap(self._path, dtype=_NP[dtype], mode="w+", shape=shape)
            self._shape = (shape, dtype)
        return self._mm[0], self._mm[1]

    def score(self, rows: int, cols: int, dtype: str, ids, vocab_real=None,
              transforms=(None, None)):
        """Scores rows [0, rows) of the buffer (ids: their selected ids). Returns float64
        (train_logp, rollout_logp, dlogp) and the wall time of the parallel part."""
        assert self._shape is not None and self._shape[0][1] >= rows
        self._mm.flush()
        total = self._shape[0][1]
        ids = np.asarray(ids, dtype=np.int64)
        tasks = [(self._path, total, cols, dtype, lo, hi, ids[lo:hi], vocab_real, transforms)
                 for lo, hi in self._ranges(rows)]
        t0 = time.perf_counter()
        res = self._pool.map(_score_range, tasks, chunksize=1)
        wall = time.perf_counter() - t0
        t = np.empty(rows)
        r = np.empty(rows)
        d = np.empty(rows)
        for lo, a, b, c, _ in res:
            t[lo:lo + len(a)] = a
            r[lo:lo + len(a)] = b
            d[lo:lo + len(a)] = c
        return t, r, d, wall

    def _ranges(self, rows):
        # about four ranges per worker, so that uneven row costs even out
        step = max(1, -(-rows // (4 * self.workers)))
        return [(lo, min(rows, lo + step)) for lo in range(0, rows, step)]

    def entropy(self, rows: int, cols: int, dtype: str, vocab_real=None,
                transforms=(None, None)):
        """Entropy (nats) and natural-log log-sum-exp of rows [0, rows) of both sides of the
        buffer, float64: (entropy_train, entropy_rollout, lse_train, lse_rollout)."""
        assert self._shape is not None and self._shape[0][1] >= rows
        self._mm.flush()
        total = self._shape[0][1]
        tasks = [(self._path, total, cols, dtype, lo, hi, vocab_real, transforms)
                 for lo, hi in self._ranges(rows)]
        out = np.empty((4, rows))
        for lo, parts in self._pool.map(_entropy_range, tasks, chunksize=1):
            for k in range(4):
                out[k, lo:lo + len(parts[k])] = parts[k]
        return tuple(out)

    def dlogits_excess(self, rows: int, cols: int, dtype: str, out_dtype: str, ids, c: float,
                       vocab_real=None, transform=None):
        """Rows [0, rows) of side 0 are logits, of side 1 a gradient of them to check (both
        stored as `dtype`, which `out_dtype` must share, e.g. bf16 logits and a bf16
        gradient). Returns, per row, the largest |got - want| - c |want| over the other
        columns and its value at the selected column, against the oracle's gradient of the
        selected logprob (upstream gradient 1)."""
        assert self._shape is not None and self._shape[0][1] >= rows
        assert _NP[dtype] == _NP[out_dtype]
        self._mm.flush()
        total = self._shape[0][1]
        ids = np.asarray(ids, dtype=np.int64)
        tasks = [(self._path, total, cols, dtype, out_dtype, lo, hi, ids[lo:hi], c, vocab_real,
                  transform) for lo, hi in self._ranges(rows)]
        other, at_y = np.empty(rows), np.empty(rows)
        for lo, ex, ey in self._pool.map(_dlogits_range, tasks, chunksize=1):
            other[lo:lo + len(ex)] = ex
            at_y[lo:lo + len(ey)] = ey
        return other, at_y

    def _release(self):
        self._mm = None
        if self._dir:
            shutil.rmtree(self._dir, ignore_errors=True)
        self._dir = self._path = self._shape = None

    def close(self):
        self._release()
        if self._pool is not None:
            self._pool.terminate()
            self._pool.join()
            self._pool = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
