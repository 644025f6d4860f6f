"""Fan the unchanged oracle out over worker processes, for parity checks of every row of
the full-size workloads.

The workers are spawned (fresh interpreters that never touch the GPU, so none inherits
the test process's GPU context) and read the batch through memory-mapped .npy files,
so the pools are not copied into each of them.  Each task is one call of the oracle's
own functions on a subset of sequences or rows; nothing here does any arithmetic of
the method.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np

# the box gives one GPU's job 16 host cores, whatever the affinity mask shows
CPU_SHARE = 16

_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
_ARR = {}
_META = {}


def _init(directory, meta):
    for f in os.listdir(directory):
        if f.endswith(".npy"):
            _ARR[f[:-4]] = np.load(os.path.join(directory, f), mmap_mode="r")
    _META.update(meta)


def _decode_task(seqs):
    from oracle import paged as O
    out = O.decode(_ARR["q"], _ARR["k"], _ARR["v"], _ARR["tables"], _ARR["ctx"], _META["scale"],
                   _META["dtype"], _META["num_kv_heads"], seqs=seqs)
    return seqs, out[seqs]


def _prefill_task(rows):
    from oracle import paged as O
    out = O.prefill_chunk(_ARR["q"], _ARR["cu"], _ARR["k"], _ARR["v"], _ARR["tables"], _ARR["ctx"],
                          _META["scale"], _META["dtype"], _META["num_kv_heads"], rows=rows)
    idx = np.array(rows, dtype=np.int64)
    return rows, out[idx[:, 0], idx[:, 1]]


class _Pool:
    def __init__(self, arrays, meta):
        base = "/dev/shm" if os.path.isdir("/dev/shm") else None
        self.dir = tempfile.mkdtemp(prefix="pkv_oracle_", dir=base)
        for name, a in arrays.items():
            np.save(os.path.join(self.dir, name + ".npy"), np.ascontiguousarray(a))
        n = max(1, min(CPU_SHARE, len(os.sched_getaffinity(0))))
        # one BLAS thread per worker: the workers already use every core of the share
        saved = {v: os.environ.get(v) for v in _THREAD_VARS}
        os.environ.update({v: "1" for v in _THREAD_VARS})
        try:
            self.pool = mp.get_context("spawn").Pool(n, initializer=_init, initargs=(self.dir, meta))
        except BaseException:
            shutil.rmtree(self.dir, ignore_errors=True)
            raise
        finally:
            for v, x in saved.items():
                if x is None:
                    os.environ.pop(v, None)
                else:
                    os.environ[v] = x

    def close(self):
        self.pool.close()
        self.pool.join()
        shutil.rmtree(self.dir, ignore_errors=True)


def decode_all(q, k_pool, v_pool, block_tables, context_lens, scale, dtype, num_kv_heads,
               seqs_per_task=4) -> np.ndarray:
    """oracle.decode over every sequence, computed in parallel; float64 [S][Hq][D]."""
    S = q.shape[0]
    p = _Pool(dict(q=q, k=k_pool, v=v_pool, tables=block_tables, ctx=context_lens),
              dict(scale=float(scale), dtype=dtype, num_kv_heads=int(num_kv_heads)))
    try:
        out = np.full(q.shape, np.nan)
        tasks = [list(range(s, min(S, s + seqs_per_task))) for s in range(0, S, seqs_per_task)]
        for seqs, rows in p.pool.imap_unordered(_decode_task, tasks):
            out[seqs] = rows
        return out
    finally:
        p.close()


def prefill_all(q, cu_q_lens, k_pool, v_pool, block_tables, context_lens, scale, dtype,
                num_kv_heads, rows_per_task=256) -> np.ndarray:
    """oracle.prefill_chunk over every (query row, q head), computed in parallel;
    float64 [sum n_q][Hq][D].  A task holds rows of one chunk and one q head."""
    Tq, Hq, _ = q.shape
    p = _Pool(dict(q=q, cu=cu_q_lens, k=k_pool, v=v_pool, tables=block_tables, ctx=context_lens),
              dict(scale=float(scale), dtype=dtype, num_kv_heads=int(num_kv_heads)))
    try:
        tasks = []
        for c in range(len(context_lens)):
            q0, q1 = int(cu_q_lens[c]), int(cu_q_lens[c + 1])
            for hq in range(Hq):
                for r0 in range(q0, q1, rows_per_task):
                    tasks.append([(i, hq) for i in range(r0, min(q1, r0 + rows_per_task))])
        out = np.full(q.shape, np.nan)
        for rows, vals in p.pool.imap_unordered(_prefill_task, tasks):
            idx = np.array(rows, dtype=np.int64)
            out[idx[:, 0], idx[:, 1]] = vals
        return out
    finally:
        p.close()
