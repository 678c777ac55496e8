"""Runs the oracle's per-row scoring over many rows in a pool of CPU worker processes.

Test infrastructure only (see the package docstring): the full-size parity tests and the
CPU-baseline leg of the benchmark use it. It adds no arithmetic of its own: every row is
scored by `score_rows` of this package (textbook two-pass log-sum-exp in float64), one
call per contiguous range of rows, and the results are put back in row order.

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
        # about four ranges per worker, so that uneven row costs even out
        step = max(1, -(-rows // (4 * self.workers)))
        tasks = [(self._path, total, cols, dtype, lo, min(rows, lo + step), ids[lo:lo + step],
                  vocab_real, transforms) for lo in range(0, rows, step)]
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
