"""The fp64 oracle over every sequence of a full-size batch, in a pool of host processes.

The parent hands the post-step pools (already written and copied by the oracle) to
worker processes through files in /dev/shm (memory-mapped, read-only); each worker
gathers one sequence's context through its table and runs the oracle's attention
for its query rows.  Workers are started with `spawn` (never fork a process that
has used the GPU) and import only NumPy, the oracle and the sensitivity helper.
"""

from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np

# One GPU's share of a host is 16 cores, whatever the machine reports: never more workers.
MAX_WORKERS = 16


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(MAX_WORKERS, n))


def _worker(args):
    d, s, margins = args
    import oracle
    z = np.load(os.path.join(d, "meta.npz"))
    kp = np.load(os.path.join(d, "k.npy"), mmap_mode="r")
    vp = np.load(os.path.join(d, "v.npy"), mmap_mode="r")
    bt, cl, qsl, B = z["bt"], z["cl"], z["qsl"], int(z["B"])
    a, b = int(qsl[s]), int(qsl[s + 1])
    L = int(cl[s])
    window = int(z["window"])
    alibi = z["alibi"] if z["alibi"].size else None
    q = np.load(os.path.join(d, "q.npy"), mmap_mode="r")[a:b]
    out = oracle.paged_attention_seq(np.asarray(q), kp, vp, bt[s], L, B, window=window,
                                     alibi_slopes=alibi)
    m = None
    if margins and b - a == 1 and L > B:
        from sensitivity import drop_block_margins
        keys = oracle.gather_context(kp, bt[s], L, B)
        vals = oracle.gather_context(vp, bt[s], L, B)
        m = float(drop_block_margins(np.asarray(q[0], np.float64), keys, vals, B,
                                     float(z["atol"]), float(z["rtol"])).min())
    return s, out, m


def attention_all(k_pool, v_pool, block_tables, context_lens, q_start_loc, q, block_size,
                  seqs=None, window=0, alibi=None, margins_tol=None):
    """Oracle attention of the query rows of `seqs` (all when None) over the given host pools.

    Returns ({s: [n_s][H][d] fp64}, {s: smallest drop-one-block margin} when margins_tol =
    (atol, rtol) is given; decode sequences longer than one block only)."""
    S = len(context_lens)
    seqs = list(range(S)) if seqs is None else list(seqs)
    qsl = np.arange(S + 1, dtype=np.int64) if q_start_loc is None else np.asarray(q_start_loc)
    d = tempfile.mkdtemp(prefix="pa_oracle_",
                         dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        np.save(os.path.join(d, "k.npy"), k_pool)
        np.save(os.path.join(d, "v.npy"), v_pool)
        np.save(os.path.join(d, "q.npy"), q)
        atol, rtol = margins_tol if margins_tol is not None else (0.0, 0.0)
        np.savez(os.path.join(d, "meta.npz"), bt=block_tables, cl=context_lens, qsl=qsl,
                 B=block_size, window=window,
                 alibi=np.zeros(0) if alibi is None else np.asarray(alibi, np.float64),
                 atol=atol, rtol=rtol)
        ctx = mp.get_context("spawn")
        outs, margins = {}, {}
        with ctx.Pool(workers()) as pool:
            # longest contexts first, so the pool does not end on one long sequence
            order = sorted(seqs, key=lambda s: -int(context_lens[s]) * int(qsl[s + 1] - qsl[s]))
            for s, o, m in pool.imap_unordered(
                    _worker, [(d, s, margins_tol is not None) for s in order], chunksize=1):
                outs[s] = o
                if m is not None:
                    margins[s] = m
        return outs, margins
    finally:
        shutil.rmtree(d, ignore_errors=True)
