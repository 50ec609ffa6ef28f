"""Runs the fp64 oracle for many sequences in worker processes (test infrastructure).

The workers are started with the "spawn" method: fresh interpreters that import
only numpy and the oracle (never torch or the GPU runtime).  The pages a batch
of sequences reads sit in POSIX shared memory, so each worker attaches to them
instead of receiving a copy.  Each task is one sequence: its query rows, its
block-table row (indices into the shared pages) and its context length.
"""
from __future__ import annotations

import multiprocessing as mp
from concurrent.futures import ProcessPoolExecutor
from multiprocessing import shared_memory

import numpy as np

_ATTACHED = {}  # worker side: shared-memory name -> (handle, array), the current batch's only


def _attach(name, shape, dtype, keep):
    """Map a batch's segment; segments of earlier batches (names not in `keep`) are released."""
    for old in [n for n in _ATTACHED if n not in keep]:
        h, _ = _ATTACHED.pop(old)
        h.close()
    if name not in _ATTACHED:
        h = shared_memory.SharedMemory(name=name)
        _ATTACHED[name] = (h, np.ndarray(shape, dtype=dtype, buffer=h.buf))
    return _ATTACHED[name][1]


def _worker_init():
    # one BLAS thread per worker: the workers already use every core
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def _one(task):
    from oracle import attention as oattn
    (kname, kshape, vname, vshape, pdtype, q_rows, table, L, scale, dtype) = task
    keep = (kname, vname)
    kp = _attach(kname, kshape, pdtype, keep)
    vp = _attach(vname, vshape, pdtype, keep)
    return oattn.paged_attention(q_rows, kp, vp, table[None, :], np.array([L], np.int32),
                                 np.array([0, q_rows.shape[0]], np.int32), scale, dtype)


class OraclePool:
    """A pool of oracle worker processes; use as a context manager."""

    def __init__(self, workers: int):
        self.workers = workers
        self.ex = ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn"), initializer=_worker_init)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.ex.shutdown(wait=True, cancel_futures=True)

    def run(self, kp: np.ndarray, vp: np.ndarray, tasks):
        """tasks: list of (q_rows, table_row, L, scale, dtype) over the pages kp/vp; returns the
        oracle outputs in task order."""
        segs = []
        try:
            names = []
            for a in (kp, vp):
                h = shared_memory.SharedMemory(create=True, size=max(a.nbytes, 1))
                np.ndarray(a.shape, dtype=a.dtype, buffer=h.buf)[...] = a
                segs.append(h)
                names.append(h.name)
            packed = [(names[0], kp.shape, names[1], vp.shape, kp.dtype) + tuple(t) for t in tasks]
            return list(self.ex.map(_one, packed, chunksize=max(1, len(packed) // (4 * self.workers))))
        finally:
            for h in segs:
                h.close()
                h.unlink()
