"""Block bookkeeping of beam search on the host block manager.

P1 sec. 6 (beam search, Fig. 10): the candidates of a beam search share the
blocks of their common ancestry; a new candidate only adds a reference to its
parent's blocks, a pruned candidate drops its references (blocks whose count
reaches zero return to the pool at once), and a block is copied only when a
candidate appends into a last block that others still hold (copy-on-write, as
in the block-manager pseudocode of P2).

One step, for every request: reorder the candidates by the parent each new
candidate extends (the first child of a parent takes the parent's table, any
further child forks it), free the tables of parents left without children,
then reserve one slot per candidate.  The copy-on-write pairs queue in the
BlockManager (take_copies) for one pa_copy_blocks call, the slots go to
pa_write_kv, the tables to pa_decode.  Which candidates survive is the search's
business (scores from a model); here the parents are given.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

from .block_manager import BlockManager


class BeamSearchKV:
    """The block tables of one beam-search request."""

    def __init__(self, bm: BlockManager, prompt_len: int):
        if prompt_len <= 0:
            raise ValueError("prompt_len must be positive")
        self.bm = bm
        root: List[int] = []
        bm.append_slots(root, prompt_len)
        self.beams: List[List[int]] = [root]      # one sequence until the first step

    def step(self, parents: Sequence[int]) -> List[Tuple[int, int]]:
        """Fork / prune to the new candidates, then reserve one slot per candidate.

        parents[b] indexes the current candidates.  Returns the (block, slot) of each
        candidate's new token; copy-on-write pairs are queued in the manager.
        """
        taken = set()
        new: List[List[int]] = []
        for p in parents:
            p = int(p)
            if not 0 <= p < len(self.beams):
                raise IndexError(f"parent {p} out of range")
            if p in taken:
                new.append(self.bm.fork(self.beams[p]))
            else:
                taken.add(p)
                new.append(self.beams[p])
        for j, t in enumerate(self.beams):
            if j not in taken:
                self.bm.free_table(t)
        self.beams = new
        return [self.bm.append_slot(t) for t in self.beams]

    def num_tokens(self) -> List[int]:
        return [self.bm.num_tokens(t) for t in self.beams]

    def release(self) -> None:
        for t in self.beams:
            self.bm.free_table(t)
        self.beams = []


def memory_saving(requests: Sequence[BeamSearchKV]) -> Tuple[int, int, float]:
    """(blocks held, blocks without sharing, saving = 1 - held / unshared).

    Without sharing every candidate would hold a private copy of its whole history:
    ceil(tokens / block_size) blocks each."""
    held = set()
    unshared = 0
    for r in requests:
        B = r.bm.block_size
        for t in r.beams:
            held.update(t)
            unshared += -(-r.bm.num_tokens(t) // B)
    n = len(held)
    return n, unshared, (1.0 - n / unshared) if unshared else 0.0
