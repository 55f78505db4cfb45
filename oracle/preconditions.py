"""Oracle: the device-side preconditions of the calls — TEST INFRASTRUCTURE ONLY.

The calls read block tables, context lengths, start locations and block pairs
from device memory and take them on trust.  What they must satisfy follows
from the addressing the calls implement and from copy-on-write:
  * token j of sequence s sits in block block_tables[s][j // B], slot j % B
    [P1 sec. 4, the addressing sentence after the attention equation; P1
    sec. 5, Fig. 7], so every block a call touches must be a real block, and
    a sequence cannot be longer than its table;
  * the n new tokens of a step are the last n of the context [P2
    "アルゴリズムの擬似コード", append_token: the new token goes into the next
    slot], so 0 <= n <= L (at least one query for attention), and two new
    tokens never share a slot;
  * copy_on_write gives a writer its own new block holding a copy of the
    shared one [P2 pseudocode, copy_on_write; P1 sec. 6, Fig. 9], so each
    copy lands in a distinct block that is not itself being copied from.

Each function returns None when every precondition holds, else (kind, index):
the smallest kind violated and, for that kind, the smallest sequence (or
pair) index that violates it.  Kinds:
  1 START_LOC      start locations not 0-based, decreasing, or last > num_tokens
  2 QUERY_COUNT    attention: fewer than one query, or more than max_query_len
  3 CONTEXT_LEN    L < n, L longer than the table, or (attention) > max_context_len
  4 BLOCK_ID       a table entry the call uses is not a block of the pool
  5 SLOT_REUSED    write: a token of this sequence shares its slot with another
  6 PAIR_ID        pairs: src or dst is not a block of its pool
  7 DEST_REUSED    pairs: this pair's destination is another pair's destination
  8 DEST_IS_SOURCE pairs inside one pool: this pair's source is a destination
Plain loops over the definitions; no code shared with the library.
"""

from __future__ import annotations

from collections import defaultdict

START_LOC, QUERY_COUNT, CONTEXT_LEN, BLOCK_ID = 1, 2, 3, 4
SLOT_REUSED, PAIR_ID, DEST_REUSED, DEST_IS_SOURCE = 5, 6, 7, 8

KIND_NAMES = {START_LOC: "START_LOC", QUERY_COUNT: "QUERY_COUNT", CONTEXT_LEN: "CONTEXT_LEN",
              BLOCK_ID: "BLOCK_ID", SLOT_REUSED: "SLOT_REUSED", PAIR_ID: "PAIR_ID",
              DEST_REUSED: "DEST_REUSED", DEST_IS_SOURCE: "DEST_IS_SOURCE"}


def _first(hits):
    return min(hits) if hits else None


def _counts(start_loc, num_seqs, num_tokens, hits):
    """Token count of every sequence from the start locations (one each when None)."""
    if start_loc is None:
        return [1] * num_seqs
    n = []
    for s in range(num_seqs):
        a, b = int(start_loc[s]), int(start_loc[s + 1])
        if (s == 0 and a != 0) or b < a or (s == num_seqs - 1 and b > num_tokens):
            hits.append((START_LOC, s))
        n.append(b - a)
    return n


def check_attention(block_tables, context_lens, q_start_loc, num_blocks, block_size,
                    num_tokens, max_context_len, max_query_len, window=0):
    """Preconditions of attention over the batch (decode and chunked prefill)."""
    S = len(context_lens)
    width = block_tables.shape[1]
    hits = []
    counts = _counts(q_start_loc, S, num_tokens, hits)
    for s in range(S):
        n, L = counts[s], int(context_lens[s])
        if n < 1 or n > max_query_len:
            hits.append((QUERY_COUNT, s))
        if L < n or L > width * block_size or L > max_context_len:
            hits.append((CONTEXT_LEN, s))
            continue
        if n < 1:
            continue
        # blocks holding a key some query attends to: query i at position p = L-n+i sees
        # keys max(0, p-W+1) .. p with a window W > 0, else 0 .. p
        used = set()
        for i in range(n):
            p = L - n + i
            lo = max(0, p - window + 1) if window > 0 else 0
            used.update(range(lo // block_size, p // block_size + 1))
        if any(not 0 <= int(block_tables[s][j]) < num_blocks for j in used):
            hits.append((BLOCK_ID, s))
    return _first(hits)


def check_write(block_tables, context_lens, write_start_loc, num_blocks, block_size,
                num_tokens):
    """Preconditions of the slot write."""
    S = len(context_lens)
    width = block_tables.shape[1]
    hits = []
    counts = _counts(write_start_loc, S, num_tokens, hits)
    writers = defaultdict(list)  # slot -> sequences writing it
    for s in range(S):
        n, L = counts[s], int(context_lens[s])
        if L < n or L > width * block_size:
            hits.append((CONTEXT_LEN, s))
            continue
        for i in range(max(n, 0)):
            p = L - n + i
            blk = int(block_tables[s][p // block_size])
            if not 0 <= blk < num_blocks:
                hits.append((BLOCK_ID, s))
                continue
            writers[(blk, p % block_size)].append(s)
    for seqs in writers.values():
        if len(seqs) > 1:
            hits.extend((SLOT_REUSED, s) for s in seqs)
    return _first(hits)


def check_pairs(pairs, num_src_blocks, num_dst_blocks, same_pool):
    """Preconditions of a batch of block copies (same_pool) or swaps."""
    hits = []
    dst_count = defaultdict(int)
    for i, (src, dst) in enumerate(pairs):
        src, dst = int(src), int(dst)
        if not (0 <= src < num_src_blocks and 0 <= dst < num_dst_blocks):
            hits.append((PAIR_ID, i))
        if 0 <= dst < num_dst_blocks:
            dst_count[dst] += 1
    for i, (src, dst) in enumerate(pairs):
        src, dst = int(src), int(dst)
        if dst_count.get(dst, 0) > 1:
            hits.append((DEST_REUSED, i))
        if same_pool and dst_count.get(src, 0) > 0:
            hits.append((DEST_IS_SOURCE, i))
    return _first(hits)
