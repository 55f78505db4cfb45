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

The manager holds no K/V data.  It returns where each token goes and records
the (src, dst) block pairs whose contents the device must copy; the device
pools, the slot writes and the block copies are the library's
pa_write_kv / pa_copy_blocks.
"""

from __future__ import annotations

from typing import Iterable, List, Sequence, Tuple

import numpy as np


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.free_blocks: List[int] = list(range(self.num_blocks))
        self.ref_count = np.zeros(self.num_blocks, dtype=np.int64)
        self.num_filled = np.zeros(self.num_blocks, dtype=np.int64)
        self._copies: List[Tuple[int, int]] = []

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
