"""Oracle: slot write and copy-on-write block copy — TEST INFRASTRUCTURE ONLY.

write_kv [P2 "アルゴリズムの擬似コード", append_token; P1 sec. 5, Fig. 7]: a new
token's K and V rows (all heads) go into the next free slot of the sequence's
last logical block.  With the context length L counting the n tokens appended
in this step, the i-th of them (0-based) is token L-n+i and lands in table
entry (L-n+i) // B at slot (L-n+i) % B.

copy_blocks [P2 pseudocode, copy_on_write; P1 sec. 6, Fig. 9]: the new block
receives a copy of the whole shared block (every slot, filled or not), for
K and for V.  All pairs read the pool as it was before any of them is applied.

swap_blocks [P1 sec. 5, preemption: a sequence's KV blocks move to CPU memory
and back; P3 "오프로딩": blocks are copied into a pre-allocated pinned CPU
buffer in one batched transfer and copied back when the request resumes, with
nothing recomputed]: block dst of the destination pool receives the whole
block src of the source pool, K and V, unchanged.  Which pool lives on the
host only decides the direction; the result is the same copy.
"""

from __future__ import annotations

import numpy as np


def write_kv(k_pool, v_pool, k_new, v_new, block_tables, context_lens, block_size,
             write_start_loc=None):
    """Return new (k_pool, v_pool) with the appended rows stored.

    k_new, v_new: [T][H][d]; sequence s appends rows write_start_loc[s]..[s+1]-1
    (one row per sequence when write_start_loc is None).
    """
    S = len(context_lens)
    if write_start_loc is None:
        write_start_loc = np.arange(S + 1)
    k_out, v_out = k_pool.copy(), v_pool.copy()
    for s in range(S):
        a, b = int(write_start_loc[s]), int(write_start_loc[s + 1])
        L = int(context_lens[s])
        n = b - a
        for i in range(n):
            pos = L - n + i
            physical = int(block_tables[s][pos // block_size])
            slot = pos % block_size
            k_out[physical, slot] = k_new[a + i]
            v_out[physical, slot] = v_new[a + i]
    return k_out, v_out


def copy_blocks(k_pool, v_pool, pairs):
    """Return new (k_pool, v_pool) where block dst holds what block src held, per (src, dst)."""
    k_out, v_out = k_pool.copy(), v_pool.copy()
    for src, dst in np.asarray(pairs).reshape(-1, 2):
        k_out[int(dst)] = k_pool[int(src)]
        v_out[int(dst)] = v_pool[int(src)]
    return k_out, v_out


def swap_blocks(dst_k, dst_v, src_k, src_v, pairs):
    """Return new (dst_k, dst_v): destination block dst holds source block src, per (src, dst).

    dst_* and src_* are two different pools of the same block layout (the device pool and a
    host swap pool, either way round)."""
    k_out, v_out = dst_k.copy(), dst_v.copy()
    for src, dst in np.asarray(pairs).reshape(-1, 2):
        k_out[int(dst)] = src_k[int(src)]
        v_out[int(dst)] = src_v[int(src)]
    return k_out, v_out
