"""Synthetic beam-search trees: which beam each new candidate extends (structure only).

A request starts as one sequence holding its prompt.  At every step the
search keeps `width` candidates; candidate b of step t extends candidate
parents[t][b] of step t-1 by one token (at step 0 every candidate extends the
prompt).  Parents are drawn from a seeded categorical over the previous
candidates whose logits are redrawn every step, so some candidates leave
several children (branch points) and some none (pruned): the shape of the
trees in the beam-search example of P1 sec. 6 (Fig. 10).  Children of one
parent are adjacent, as a search that ranks candidates by parent produces.

Token ids: the prompt holds tokens 0 .. prompt_len-1; the token candidate b
appends at step t is prompt_len + t*width + b.  K/V rows and queries are
counter-generated values indexed by token id (streams below), so a
candidate's whole history can be regenerated from its ancestry alone.
Nothing here computes attention or manages blocks.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np

from .gen import normal_array, normal_values_torch

STREAM_BEAM_K, STREAM_BEAM_V, STREAM_BEAM_Q = 11, 12, 13


@dataclass
class BeamTree:
    seed: int
    width: int
    steps: int
    prompt_len: int
    parents: np.ndarray          # int32 [steps][width]

    def token_id(self, step: int, beam: int) -> int:
        return self.prompt_len + step * self.width + beam

    @property
    def num_token_ids(self) -> int:
        return self.prompt_len + self.steps * self.width

    def histories(self, upto: int) -> List[List[int]]:
        """Token ids held by each candidate after step `upto` (inclusive), in position order."""
        hist = [list(range(self.prompt_len))]
        for t in range(upto + 1):
            hist = [hist[int(p)] + [self.token_id(t, b)] for b, p in enumerate(self.parents[t])]
        return hist


def make_beam_tree(seed: int, width: int, steps: int, prompt_len: int,
                   spread: float = 1.5) -> BeamTree:
    rng = np.random.default_rng(seed)
    parents = np.zeros((steps, width), np.int32)
    for t in range(1, steps):
        logits = rng.standard_normal(width) * spread
        p = np.exp(logits - logits.max())
        parents[t] = np.sort(rng.choice(width, size=width, p=p / p.sum()))
    return BeamTree(seed, width, steps, prompt_len, parents)


def beam_rows(tree: BeamTree, num_heads: int, head_dim: int, dtype=np.float16):
    """Host K and V rows for every token id: two [num_token_ids][H][d] arrays."""
    shape = (tree.num_token_ids, num_heads, head_dim)
    return (normal_array(tree.seed, STREAM_BEAM_K, shape, dtype),
            normal_array(tree.seed, STREAM_BEAM_V, shape, dtype))


def beam_queries(tree: BeamTree, num_heads: int, head_dim: int, dtype=np.float16):
    """Host queries [steps][width][H][d]: the query of each candidate's newest token."""
    return normal_array(tree.seed, STREAM_BEAM_Q, (tree.steps, tree.width, num_heads, head_dim),
                        dtype)


def beam_rows_torch(tree: BeamTree, num_heads: int, head_dim: int, dtype, device):
    """The same K, V rows and queries generated in place on `device`."""
    import torch

    out = []
    for stream, shape in ((STREAM_BEAM_K, (tree.num_token_ids, num_heads, head_dim)),
                          (STREAM_BEAM_V, (tree.num_token_ids, num_heads, head_dim)),
                          (STREAM_BEAM_Q, (tree.steps, tree.width, num_heads, head_dim))):
        t = torch.empty(shape, dtype=dtype, device=device)
        normal_values_torch(tree.seed, stream, t)
        out.append(t)
    return out
