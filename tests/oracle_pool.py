"""Run the fp64 attention oracle over heads in parallel worker processes.

Test infrastructure: the oracle itself (oracle.attention) is unchanged; this
only splits its work by head.  numpy's exp runs on one thread, so checking all
35050 rows of the 480p-latent joint attention takes ~90 s in one process and
a fraction of that spread over the host's cores.  Workers are spawned (not
forked), import only numpy and the oracle, never touch the GPU, and use one
BLAS thread each.
"""
import multiprocessing as mp
import os

import numpy as np


def workers():
    """Worker count: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _head_task(args):
    from oracle import attention as A
    qh, kh, vh, scale = args
    # 128-row slices keep the logit block in cache (larger ones make the
    # workers contend for memory bandwidth)
    return A.attention(qh[:, None], kh[:, None], vh[:, None], scale=scale, chunk=128)[:, 0]


def _call(args):
    import importlib
    modname, fname, a, kw = args
    return getattr(importlib.import_module(modname), fname)(*a, **kw)


_POOL = None


def pool():
    global _POOL
    if _POOL is None:
        _POOL = mp.get_context("spawn").Pool(workers(), initializer=_init)
    return _POOL


def attention_rows(q, k, v, rows=None, scale=None, chunk_rows=None):
    """oracle.attention(q, k, v, scale, rows) computed head by head (and in
    slices of chunk_rows query rows; by default about four slices per worker
    in all) by the worker pool.  q [Nq, h, d], k, v [Nk, h, d] as float
    arrays (bf16 values are exact in float32, which halves what is sent to the
    workers); returns fp64 [len(rows), h, d]."""
    q = np.asarray(q)
    if rows is not None:
        q = q[np.asarray(rows)]
    k, v = np.asarray(k), np.asarray(v)
    nq, h, d = q.shape
    if chunk_rows is None:
        per_head = max(1, -(-4 * workers() // h))
        chunk_rows = max(1, -(-nq // per_head))
    tasks, where = [], []
    for hd in range(h):
        kh = np.ascontiguousarray(k[:, hd])
        vh = np.ascontiguousarray(v[:, hd])
        for r0 in range(0, nq, chunk_rows):
            tasks.append((np.ascontiguousarray(q[r0:r0 + chunk_rows, hd]), kh, vh, scale))
            where.append((hd, r0))
    out = np.empty((nq, h, v.shape[2]), dtype=np.float64)
    for (hd, r0), res in zip(where, pool().imap(_head_task, tasks)):
        out[r0:r0 + res.shape[0], hd] = res
    return out


def starmap(modname, fname, calls):
    """[modname.fname(*a, **kw) for (a, kw) in calls], run by the pool."""
    return pool().map(_call, [(modname, fname, a, kw) for a, kw in calls], chunksize=1)


def as_f32(t):
    """A torch tensor (bf16 or fp32) on the host as a float32 numpy array."""
    import torch
    return t.detach().to("cpu", torch.float32).numpy()
