"""The recurrent oracle run over many CPU cores.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Sequences are independent, and so are the Q/K heads with the value heads
that read them (value head hv reads Q/K head hv // (HV // H)), so the
float64 recurrence of a large workload splits into (sequence, Q/K head)
tasks that run in separate processes.  Each task calls ``recurrent`` on its
own slice; this module only slices, dispatches and reassembles -- it adds
no arithmetic of its own.
"""

import multiprocessing as mp
import os

import numpy as np

from .recurrent import recurrent


def _task(args):
    q, k, v, g, beta, s0 = args
    return recurrent(q, k, v, g, beta, s0)


def default_workers():
    """Worker processes to use: the host's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def recurrent_parallel(q, k, v, g, beta, initial_state=None, cu_seqlens=None, workers=None):
    """Same contract and result as ``recurrent`` (float64 o and final
    state), computed by a process pool over (sequence, Q/K head) tasks.
    Inputs are NumPy arrays (bf16 values as float32)."""
    q = np.asarray(q, dtype=np.float32)
    k = np.asarray(k, dtype=np.float32)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    grp = HV // H
    if cu_seqlens is None:
        segs = [(b, 0, T) for b in range(B)]
    else:
        cu = [int(c) for c in np.asarray(cu_seqlens).tolist()]
        segs = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    tasks, where = [], []
    for n, (b, t0, t1) in enumerate(segs):
        for h in range(H):
            hv = slice(h * grp, (h + 1) * grp)
            s0 = None if initial_state is None else np.asarray(initial_state[n:n + 1, hv])
            tasks.append((q[b:b + 1, t0:t1, h:h + 1], k[b:b + 1, t0:t1, h:h + 1], v[b:b + 1, t0:t1, hv],
                          g[b:b + 1, t0:t1, hv], beta[b:b + 1, t0:t1, hv], s0))
            where.append((n, b, t0, t1, hv))
    # longest tasks first, so the pool's tail is short
    order = sorted(range(len(tasks)), key=lambda i: -(where[i][3] - where[i][2]))
    o = np.zeros((B, T, HV, V), dtype=np.float64)
    final = np.zeros((len(segs), HV, K, V), dtype=np.float64)
    n_workers = workers or default_workers()
    if n_workers == 1 or len(tasks) == 1:
        results = [_task(tasks[i]) for i in order]
    else:
        with mp.get_context("spawn").Pool(min(n_workers, len(tasks))) as pool:
            results = pool.map(_task, [tasks[i] for i in order], chunksize=1)
    for i, (o_t, s_t) in zip(order, results):
        n, b, t0, t1, hv = where[i]
        o[b, t0:t1, hv] = o_t[0]
        final[n, hv] = s_t[0]
    return o, final
