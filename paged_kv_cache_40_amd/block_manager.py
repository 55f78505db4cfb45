"""Host-side block manager: physical block allocation, reference counts and
copy-on-write decisions for a paged KV cache.

Semantics follow the block-manager pseudocode of P2 ("SOSP 2023論文解説: vLLM —
PagedAttentionによるKVキャッシュメモリ管理の革新", section
"アルゴリズムの擬似コード") and the sharing rules of P1 ("Efficient Memory
Management for Large Language Model Serving with PagedAttention", sec. 5-6,
Fig. 7-10):
  * the free list is a stack: allocation takes the most recently pushed id,
    and an empty pool raises MemoryError;
  * freeing drops one reference; the block returns to the pool at zero;
  * forking a sequence (parallel samples, beams) adds a reference to each of
    its blocks instead of copying them;
  * appending a token takes the next slot of the last block, a new block when
    the last one is full, and a private copy of the last block when it is
    shared (copy-on-write: the copy carries over the fill count and drops one
    reference from the source; the last sharer left finds a count of one and
    writes in place).

Swapping [P1 sec. 5: under memory pressure a preempted sequence's blocks move
to CPU memory and come back later; P3 "오프로딩": one batched copy into a
pre-allocated pinned CPU pool, copied back on resume]: a second, host pool
has its own stack free list and counts.  swap_out moves a group of sequences
(e.g. the samples of one request, which share blocks) to host blocks, one
host block per distinct device block so sharing survives, and drops the
group's device references; swap_in does the reverse.  Both are all or
nothing: without room they raise MemoryError and change nothing.  Which
request to swap, and when, is the scheduler's policy and not modelled here.

The manager holds no K/V data.  It returns where each token goes and records
the (src, dst) block pairs whose contents the device must copy; the device
pools, the slot writes and the block copies are the library's
pa_write_kv / pa_copy_blocks / pa_swap_blocks.
"""

from __future__ import annotations

from typing import Iterable, List, Sequence, Tuple

import numpy as np


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, num_host_blocks: int = 0):
        if num_blocks <= 0 or block_size <= 0 or num_host_blocks < 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.free_blocks: List[int] = list(range(self.num_blocks))
        self.ref_count = np.zeros(self.num_blocks, dtype=np.int64)
        self.num_filled = np.zeros(self.num_blocks, dtype=np.int64)
        self._copies: List[Tuple[int, int]] = []
        self.num_host_blocks = int(num_host_blocks)
        self.host_free: List[int] = list(range(self.num_host_blocks))
        self.host_ref = np.zeros(self.num_host_blocks, dtype=np.int64)
        self.host_filled = np.zeros(self.num_host_blocks, dtype=np.int64)

    # -- allocation ------------------------------------------------------
    def allocate_block(self) -> int:
        if not self.free_blocks:
            raise MemoryError("no free KV cache blocks")
        bid = self.free_blocks.pop()
        self.ref_count[bid] = 1
        self.num_filled[bid] = 0
        return bid

    def free_block(self, bid: int) -> None:
        if self.ref_count[bid] <= 0:
            raise ValueError(f"block {bid} is not allocated")
        self.ref_count[bid] -= 1
        if self.ref_count[bid] == 0:
            self.free_blocks.append(int(bid))

    def copy_on_write(self, bid: int) -> int:
        """Private copy of a shared block (or the block itself when unshared).

        The device copy is deferred: the (src, dst) pair is queued for
        take_copies(), to be run by one batched pa_copy_blocks call.
        """
        if self.ref_count[bid] == 1:
            return bid
        new = self.allocate_block()
        self._copies.append((int(bid), int(new)))
        self.num_filled[new] = self.num_filled[bid]
        self.ref_count[bid] -= 1
        return new

    # -- sequences -------------------------------------------------------
    def append_slot(self, table: List[int]) -> Tuple[int, int]:
        """Reserve the slot for one new token of the sequence whose block table is `table`.

        `table` is updated in place.  Returns (physical block, slot).
        """
        if not table:
            table.append(self.allocate_block())
        last = table[-1]
        if self.num_filled[last] >= self.block_size:
            last = self.allocate_block()
            table.append(last)
        if self.ref_count[last] > 1:
            last = self.copy_on_write(last)
            table[-1] = last
        slot = int(self.num_filled[last])
        self.num_filled[last] += 1
        return int(last), slot

    def append_slots(self, table: List[int], n: int) -> List[Tuple[int, int]]:
        return [self.append_slot(table) for _ in range(n)]

    def fork(self, table: Sequence[int]) -> List[int]:
        """A new sequence sharing every block of `table` (reference counts +1)."""
        for bid in table:
            if self.ref_count[bid] <= 0:
                raise ValueError(f"block {bid} is not allocated")
            self.ref_count[bid] += 1
        return list(table)

    def free_table(self, table: List[int]) -> None:
        for bid in table:
            self.free_block(bid)
        table.clear()

    def take_copies(self) -> np.ndarray:
        """Queued copy-on-write pairs as int32 [n][2] (src, dst); clears the queue."""
        pairs = np.asarray(self._copies, dtype=np.int32).reshape(-1, 2)
        self._copies = []
        return pairs

    # -- swapping --------------------------------------------------------
    def swap_out(self, tables: Sequence[List[int]]) -> np.ndarray:
        """Move the blocks of a group of sequences to the host pool.

        Each table is rewritten in place with host block ids.  Returns the int32 [n][2]
        (device src, host dst) pairs to copy, one per distinct device block, before any of
        those device blocks is reused.
        """
        distinct = list(dict.fromkeys(int(b) for t in tables for b in t))
        for b in distinct:
            if self.ref_count[b] <= 0:
                raise ValueError(f"block {b} is not allocated")
        if len(distinct) > len(self.host_free):
            raise MemoryError("no room in the host swap pool")
        mapping = {}
        for b in distinct:
            h = self.host_free.pop()
            mapping[b] = h
            self.host_filled[h] = self.num_filled[b]
        for t in tables:
            for i, b in enumerate(t):
                h = mapping[int(b)]
                self.host_ref[h] += 1
                self.free_block(int(b))
                t[i] = h
        return np.asarray([(b, mapping[b]) for b in distinct], np.int32).reshape(-1, 2)

    def swap_in(self, tables: Sequence[List[int]]) -> np.ndarray:
        """Bring a swapped-out group back into newly allocated device blocks.

        Each table is rewritten in place with device block ids.  Returns the int32 [n][2]
        (host src, device dst) pairs to copy before the group runs again.
        """
        distinct = list(dict.fromkeys(int(h) for t in tables for h in t))
        for h in distinct:
            if self.host_ref[h] <= 0:
                raise ValueError(f"host block {h} is not in use")
        if len(distinct) > len(self.free_blocks):
            raise MemoryError("no free KV cache blocks for swap-in")
        mapping = {}
        for h in distinct:
            b = self.allocate_block()
            self.ref_count[b] = 0
            self.num_filled[b] = self.host_filled[h]
            mapping[h] = b
        for t in tables:
            for i, h in enumerate(t):
                b = mapping[int(h)]
                self.ref_count[b] += 1
                self.host_ref[int(h)] -= 1
                if self.host_ref[int(h)] == 0:
                    self.host_free.append(int(h))
                t[i] = b
        return np.asarray([(h, mapping[h]) for h in distinct], np.int32).reshape(-1, 2)

    # -- reporting -------------------------------------------------------
    def num_tokens(self, table: Sequence[int]) -> int:
        if not table:
            return 0
        return (len(table) - 1) * self.block_size + int(self.num_filled[table[-1]])

    def num_free(self) -> int:
        return len(self.free_blocks)

    def waste(self, tables: Iterable[Sequence[int]]) -> float:
        """Unfilled fraction of the slots in allocated blocks: (allocated - filled) / allocated."""
        used = set()
        for t in tables:
            used.update(int(b) for b in t)
        if not used:
            return 0.0
        alloc = len(used) * self.block_size
        filled = int(sum(self.num_filled[b] for b in used))
        return (alloc - filled) / alloc


def tables_to_array(tables: Sequence[Sequence[int]], width: int = 0) -> np.ndarray:
    """Pad per-sequence tables with -1 into an int32 [S][width] array."""
    width = max([width] + [len(t) for t in tables])
    out = np.full((len(tables), max(width, 1)), -1, dtype=np.int32)
    for s, t in enumerate(tables):
        out[s, :len(t)] = t
    return out
