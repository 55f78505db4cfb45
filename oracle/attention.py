"""Oracle: paged softmax attention in fp64 — TEST INFRASTRUCTURE ONLY.

Definition followed [P1 sec. 4 "PagedAttention 알고리즘", attention equation;
P2 "PagedAttentionの仕組み", blockwise attention equation]: for the query of
token i and the keys/values of tokens j <= i of the same sequence,
    A_ij = exp(q_i . k_j / sqrt(d)) / sum_{j' <= i} exp(q_i . k_j' / sqrt(d))
    o_i  = sum_{j <= i} A_ij v_j
per attention head, with d the head dimension.

Addressing [P1 sec. 4, the sentence after the equation; P1 sec. 5, Fig. 7]:
token j (counted from 1 on the page) lives in logical block floor((j-1)/B) at
slot (j-1) mod B, and the block table maps a logical block to a physical one.
Here tokens are counted from 0, so token j is at table entry j // B, slot
j % B: the same mapping.

Variants [P1 sec. 10, limitations: sliding-window and ALiBi attention need the
block indexing adapted; P3 "메모리 관리": sliding layers keep only a fixed
window of the most recent tokens].  The pages name them without formulas; the
plainest readings are used:
  * sliding window W > 0: the query at position p sees keys p-W+1 .. p (the W
    most recent tokens, itself included); W = 0 means no window;
  * ALiBi: a per-head slope m_h adds m_h * (j - p) to the score of key j (a
    penalty growing linearly with distance; 0 for the query's own token).

Readings where the pages leave a step open:
  * the query of the token at 0-based position p attends to keys 0..p, itself
    included (the sums run up to j = i);
  * a sequence with n new query tokens and context length L holds them at
    positions L-n .. L-1 (context length counts the new tokens);
  * the maximum score is subtracted before exponentiating; the common factor
    cancels between numerator and denominator, so this is the same quantity.
"""

from __future__ import annotations

import numpy as np


def gather_context(pool: np.ndarray, table_row: np.ndarray, length: int,
                   block_size: int) -> np.ndarray:
    """Rows of tokens 0..length-1 of one sequence, fetched through its block table.

    pool: [num_blocks][block_size][H][d]; table_row: that sequence's block table.
    Returns fp64 [length][H][d].
    """
    out = np.empty((length,) + pool.shape[2:], dtype=np.float64)
    for j in range(length):
        physical = int(table_row[j // block_size])
        out[j] = pool[physical, j % block_size]
    return out


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
           positions: np.ndarray, window: int = 0, alibi_slopes=None) -> np.ndarray:
    """Causal softmax attention in fp64.

    q: [n][H][d] queries; keys, values: [L][H][d] (token order);
    positions: [n] 0-based token position of each query (query attends keys 0..p,
    or p-window+1..p with a window); alibi_slopes: optional [H] slopes, adding
    slope * (j - p) to the score of key j.
    Returns [n][H][d].
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    d = q.shape[-1]
    out = np.empty(q.shape, dtype=np.float64)
    for r, p in enumerate(positions):
        p = int(p)
        lo = max(0, p - window + 1) if window > 0 else 0
        k = keys[lo:p + 1]                                   # [n_keys][H][d]
        v = values[lo:p + 1]
        x = np.einsum("hd,jhd->hj", q[r], k) / np.sqrt(d)    # [H][n_keys]
        if alibi_slopes is not None:
            dist = np.arange(lo, p + 1, dtype=np.float64) - p          # j - p
            x = x + np.asarray(alibi_slopes, np.float64)[:, None] * dist[None, :]
        x = x - x.max(axis=1, keepdims=True)
        w = np.exp(x)
        a = w / w.sum(axis=1, keepdims=True)                 # A_rj
        out[r] = np.einsum("hj,jhd->hd", a, v)
    return out


def paged_attention_seq(q_rows: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                        table_row: np.ndarray, context_len: int, block_size: int,
                        heads=None, window: int = 0, alibi_slopes=None) -> np.ndarray:
    """Attention for the n query rows of one sequence (the last n of its context_len tokens).

    heads: optional list of head indices to compute (others are skipped); the result
    keeps only those heads, in that order.
    """
    n = q_rows.shape[0]
    keys = gather_context(k_pool, table_row, context_len, block_size)
    values = gather_context(v_pool, table_row, context_len, block_size)
    if heads is not None:
        heads = list(heads)
        keys, values, q_rows = keys[:, heads], values[:, heads], q_rows[:, heads]
        if alibi_slopes is not None:
            alibi_slopes = np.asarray(alibi_slopes)[heads]
    positions = np.arange(context_len - n, context_len)
    return attend(q_rows, keys, values, positions, window, alibi_slopes)


def paged_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                    block_tables: np.ndarray, context_lens: np.ndarray, block_size: int,
                    q_start_loc=None, window: int = 0, alibi_slopes=None) -> np.ndarray:
    """Attention for a whole batch.

    q: [T][H][d]; sequence s owns query rows q_start_loc[s] .. q_start_loc[s+1]-1
    (one row per sequence when q_start_loc is None).  Returns fp64 [T][H][d].
    """
    S = len(context_lens)
    if q_start_loc is None:
        q_start_loc = np.arange(S + 1)
    out = np.empty(q.shape, dtype=np.float64)
    for s in range(S):
        a, b = int(q_start_loc[s]), int(q_start_loc[s + 1])
        L = int(context_lens[s])
        if not (1 <= b - a <= L):
            raise ValueError(f"sequence {s}: {b - a} queries for context length {L}")
        out[a:b] = paged_attention_seq(q[a:b], k_pool, v_pool, block_tables[s], L, block_size,
                                       window=window, alibi_slopes=alibi_slopes)
    return out
