"""How sharp a parity check is: how far the exact result moves when one group of
context tokens (one block, one partition, one token) is left out.

Used by tests to show that their inputs would expose a dropped, repeated or
misplaced block: if leaving out any one block moves some output element by more
than the tolerance atol + rtol*|ref|, a kernel that skipped that block would fail
the elementwise comparison.

For one decode query (position L-1, attending to every token) with fp64 scores
x_j = q.k_j / sqrt(d) and weights w_j = exp(x_j - max x):
    o = S / W,   S = sum_j w_j v_j,  W = sum_j w_j;
leaving out the tokens of group g gives o_g = (S - S_g) / (W - W_g), S_g and W_g
the same sums over the group.  Pinned against the oracle's attention over the
history with the group removed (tests/test_sensitivity.py).
"""

from __future__ import annotations

import numpy as np


def outputs_without(q, keys, values, groups):
    """(o_g for every group id 0..G-1 of `groups` (int [L], non-decreasing), o): the exact
    output without each group's tokens, and with all of them.

    q: [H][d]; keys, values: [L][H][d] (token order)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(keys, np.float64)
    v = np.asarray(values, np.float64)
    groups = np.asarray(groups, np.int64)
    assert np.all(np.diff(groups) >= 0), "groups must be contiguous runs of tokens"
    d = q.shape[-1]
    x = np.einsum("hd,jhd->hj", q, k) / np.sqrt(d)
    w = np.exp(x - x.max(axis=1, keepdims=True))             # [H][L]
    W = w.sum(axis=1)                                          # [H]
    wv = w.T[:, :, None] * v                                   # [L][H][d]
    S = wv.sum(axis=0)                                         # [H][d]
    starts = np.flatnonzero(np.r_[True, np.diff(groups) != 0])
    Wg = np.add.reduceat(w, starts, axis=1).T                  # [G][H]
    Sg = np.add.reduceat(wv, starts, axis=0)                   # [G][H][d]
    o = S / W[:, None]
    og = (S[None] - Sg) / (W[None] - Wg)[:, :, None]
    return og, o


def drop_one_margins(q, keys, values, groups, atol: float, rtol: float) -> np.ndarray:
    """For every group of `groups` (see outputs_without), the largest ratio
    |o_g - o| / (atol + rtol*|o|) over heads and dims."""
    og, o = outputs_without(q, keys, values, groups)
    tol = atol + rtol * np.abs(o)
    return (np.abs(og - o[None]) / tol[None]).reshape(og.shape[0], -1).max(axis=1)


def drop_block_margins(q, keys, values, block_size: int, atol: float, rtol: float):
    """drop_one_margins over the blocks of the context (tokens b*B .. b*B+B-1)."""
    L = np.asarray(keys).shape[0]
    return drop_one_margins(q, keys, values, np.arange(L) // block_size, atol, rtol)


def drop_last_token_margin(q, keys, values, atol: float, rtol: float) -> float:
    """Margin for leaving out only the last token (the query's own row)."""
    L = np.asarray(keys).shape[0]
    return float(drop_one_margins(q, keys, values, (np.arange(L) == L - 1).astype(np.int64),
                                  atol, rtol)[1])
