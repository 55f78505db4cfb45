"""Prefix caching by block content hash, with lazy eviction of freed blocks.

P3 ("연속 배치 처리 아키텍처", sections "Prefix 캐싱" and "제거"): every
completed block is keyed by a hash of its content; a later request whose
prompt starts with the same blocks reuses them (reference counted) and skips
their prefill; a block goes back to the free pool only when no request uses
it.  A freed block keeps its content and hash ("initialized") so that later
requests can still match it; only when no uninitialized block is left does the
allocator demote an initialized one (dropping its hash) and hand it out.  The
cache is best effort: the allocator may discard it whenever it needs blocks.
P1 sec. 6 (shared prefix, Fig. 11) is the sharing this automates.

Readings where the pages leave a step open:
  * "content hash": a block's K/V depend on every token before it, so the key
    of block i chains the key of block i-1 with the token ids of block i
    (BLAKE2b, 16 bytes); equal keys mean equal prefixes up to the block's end;
  * only full blocks are keyed and shared; the last, partial block of a
    request stays private, and the block holding a prompt's last token is
    never matched (that token's query has to run to continue the request);
  * "the most recent initialized block" is demoted first: freed initialized
    blocks form a stack and allocation pops its top;
  * if a block completes with a key already in the cache (two requests filled
    the same prefix in one step), the cached block keeps the key and the new
    one stays private.
The allocator holds no K/V data: it returns block tables and how many prompt
tokens are already cached; the library's pa_write_kv stores the rest and
pa_decode's multi-query path attends over the whole context.
"""

from __future__ import annotations

import hashlib
from collections import OrderedDict
from typing import Dict, List, Sequence, Tuple

import numpy as np

ROOT_KEY = b"\x00" * 16


def block_key(parent: bytes, tokens: Sequence[int]) -> bytes:
    """Key of a full block: its parent's key chained with its token ids."""
    h = hashlib.blake2b(parent, digest_size=16)
    h.update(np.asarray(tokens, dtype=np.int64).tobytes())
    return h.digest()


class PrefixCachingAllocator:
    def __init__(self, num_blocks: int, block_size: int, allow_block_sharing: bool = True):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.allow_block_sharing = bool(allow_block_sharing)
        self.free_uninit: List[int] = list(range(self.num_blocks))   # stack
        # freed blocks that keep their key, oldest first (the newest is demoted first)
        self.free_init: "OrderedDict[int, None]" = OrderedDict()
        self.ref_count = np.zeros(self.num_blocks, dtype=np.int64)
        self.key_of: Dict[int, bytes] = {}
        self.block_of: Dict[bytes, int] = {}
        self.lookups = 0
        self.hits = 0
        self.evictions = 0

    # -- allocation ------------------------------------------------------
    def _take_free(self) -> int:
        if self.free_uninit:
            b = self.free_uninit.pop()
        elif self.free_init:
            b, _ = self.free_init.popitem(last=True)                  # demote the newest
            del self.block_of[self.key_of.pop(b)]
            self.evictions += 1
        else:
            raise MemoryError("no free KV cache blocks")
        self.ref_count[b] = 1
        return b

    def num_free(self) -> int:
        return len(self.free_uninit) + len(self.free_init)

    def match(self, tokens: Sequence[int]) -> List[int]:
        """Cached blocks holding the longest run of whole leading blocks of `tokens`."""
        if not self.allow_block_sharing:
            return []
        B = self.block_size
        key = ROOT_KEY
        out = []
        for i in range(len(tokens) // B):
            key = block_key(key, tokens[i * B:(i + 1) * B])
            b = self.block_of.get(key)
            if b is None:
                break
            out.append(b)
        return out

    def allocate(self, tokens: Sequence[int]) -> Tuple[List[int], int]:
        """Block table for a new request whose prompt is `tokens`.

        Returns (table, cached): the first `cached` tokens (whole blocks) are already in
        the pool; the caller writes tokens cached .. len-1 and then calls commit().
        All or nothing: without room, MemoryError and nothing changes."""
        B = self.block_size
        if len(tokens) == 0:
            raise ValueError("empty prompt")
        # the block holding the last prompt token is never matched: its query must run
        matched = self.match(tokens[:len(tokens) - 1])
        need = -(-len(tokens) // B) - len(matched)
        reviving = sum(1 for b in matched if self.ref_count[b] == 0)
        if need > self.num_free() - reviving:
            raise MemoryError("no free KV cache blocks for the request")
        if self.allow_block_sharing:
            self.lookups += min(len(matched) + 1, (len(tokens) - 1) // B)
            self.hits += len(matched)
        for b in matched:
            if self.ref_count[b] == 0:
                del self.free_init[b]                                   # cached and free: revive
            self.ref_count[b] += 1
        table = matched + [self._take_free() for _ in range(need)]
        return table, len(matched) * B

    def commit(self, table: Sequence[int], tokens: Sequence[int]) -> None:
        """Key every full block of `table` whose K/V are now written (prompt or decode)."""
        if not self.allow_block_sharing:
            return
        B = self.block_size
        key = ROOT_KEY
        for i in range(len(tokens) // B):
            key = block_key(key, tokens[i * B:(i + 1) * B])
            b = table[i]
            if b in self.key_of:
                continue
            if key not in self.block_of:
                self.block_of[key] = b
                self.key_of[b] = key

    def append_slot(self, table: List[int], num_tokens: int) -> Tuple[int, int]:
        """Reserve the slot of token number `num_tokens` (0-based) of a running request."""
        B = self.block_size
        if num_tokens == len(table) * B:
            table.append(self._take_free())
        return table[num_tokens // B], num_tokens % B

    def free(self, table: List[int]) -> None:
        for b in table:
            if self.ref_count[b] <= 0:
                raise ValueError(f"block {b} is not allocated")
            self.ref_count[b] -= 1
            if self.ref_count[b] == 0:
                if b in self.key_of:
                    self.free_init[b] = None
                else:
                    self.free_uninit.append(b)
        table.clear()

    # -- reporting -------------------------------------------------------
    def hit_rate(self) -> float:
        return self.hits / self.lookups if self.lookups else 0.0
