"""Runs the fp64 oracle on many (head, tile) pairs of one large problem in parallel.

Worker processes are spawned (they import numpy and the oracle only, never the GPU
runtime) and read one KV group's fp64 Q, K and V from shared memory. The oracle runs
on the group's sub-problem: its G query heads over one KV head, the same arithmetic
as on the whole problem, since a query head only reads its own KV head.
"""
import multiprocessing as mp
import os
from multiprocessing import shared_memory

import numpy as np

from oracle import poem_oracle as O

_W = {}


def _attach(spec):
    out = {}
    for key, (name, shape) in spec.items():
        shm = shared_memory.SharedMemory(name=name)
        _W.setdefault("_shm", []).append(shm)
        out[key] = np.ndarray(shape, dtype=np.float64, buffer=shm.buf)
    return out


def _init(spec, problem):
    try:
        from threadpoolctl import threadpool_limits
        _W["_limit"] = threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass
    _W.update(_attach(spec))
    _W["problem"] = problem
    _W["tiles"] = O.tiles(problem)


def _select_job(job):
    """job = (h, gtile, tau, n_sink, n_local, S, kept): the oracle's selection (per-row
    I and m dropped) and, on the GPU's kept list, each sampled row's error
    ||O_dense - O_sparse|| recomputed in fp64."""
    h, gt, tau, n_sink, n_local, S, kept = job
    p, q, k, v = _W["problem"], _W["q"], _W["k"], _W["v"]
    t = _W["tiles"][gt]
    sel = O.select_tile(p, q, k, v, h, t, tau, n_sink, n_local, S)
    g = h // p.group
    K = k[t.k_row0:t.k_row0 + t.n_k, g]
    V = v[t.k_row0:t.k_row0 + t.n_k, g]
    qr = np.stack([q[t.q_row0 + r, h] for r in sel.rows])
    pos = [t.pos0 + r for r in sel.rows]
    od, _ = O.attention_rows(qr, K, V, p.scale, pos)
    allowed = np.zeros(t.n_k, dtype=bool)
    for b in kept:
        allowed[b * p.block_size:(b + 1) * p.block_size] = True
    osp, _ = O.attention_rows(qr, K, V, p.scale, pos, allowed)
    err = np.linalg.norm(od - osp, axis=1)
    m_rows = sel.m
    sel.I = None
    sel.m = None
    dropped = [b for b in range(t.diag + 1) if b not in set(kept)]
    delta = m_rows[:, dropped].sum(axis=1) if dropped else np.zeros(len(sel.rows))
    return sel, err, delta


def _attn_job(job):
    """job = (h, gtile, kept): (O, LSE) of the whole tile, dense and over the kept blocks."""
    h, gt, kept = job
    p, q, k, v = _W["problem"], _W["q"], _W["k"], _W["v"]
    t = _W["tiles"][gt]
    return O.tile_attention(p, q, k, v, h, t), O.tile_attention(p, q, k, v, h, t, kept)


class GroupPool:
    """A pool over one KV group's sub-problem. q: [N_q, G, d], k, v: [N_k, 1, d] (fp64)."""

    def __init__(self, problem, q, k, v, workers=None):
        self.problem = problem
        self._shm = []
        spec = {}
        for key, arr in (("q", q), ("k", k), ("v", v)):
            arr = np.ascontiguousarray(arr, dtype=np.float64)
            shm = shared_memory.SharedMemory(create=True, size=max(arr.nbytes, 1))
            np.ndarray(arr.shape, dtype=np.float64, buffer=shm.buf)[...] = arr
            self._shm.append(shm)
            spec[key] = (shm.name, arr.shape)
        n = workers or min(16, len(os.sched_getaffinity(0)))
        old = {k_: os.environ.get(k_) for k_ in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}
        os.environ.update(OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
        try:
            self.pool = mp.get_context("spawn").Pool(n, initializer=_init, initargs=(spec, problem))
        finally:
            for k_, val in old.items():
                if val is None:
                    os.environ.pop(k_, None)
                else:
                    os.environ[k_] = val

    def select(self, jobs):
        return self.pool.map(_select_job, jobs, chunksize=4)

    def attention(self, jobs):
        return self.pool.map(_attn_job, jobs, chunksize=1)

    def close(self):
        self.pool.close()
        self.pool.join()
        for shm in self._shm:
            shm.close()
            shm.unlink()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
