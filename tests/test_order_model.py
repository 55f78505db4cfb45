"""CPU model of the longest-first order of the decode's partition pass (decode_order_kernel in
pa_decode.hip): the keys, the quarters the four waves count over, the zero padding and the
rank sum, restated with the kernel's own index arithmetic.  Checks that the ranks are a
permutation of the sequences, that every index the kernel touches stays inside its LDS
arrays, and that the order is by clamped length, longest first, ties by index, on lengths
with many ties and malformed values (negative, beyond the cap).  The numerical parity of the
launches that use the order is tests/test_gpu_parity.py."""

import numpy as np
import pytest

MAX_SEQS, WAVES, WAVE = 1024, 4, 64


def order_model(lens, cap):
    S = len(lens)
    quarter = ((S + WAVES - 1) // WAVES + 7) & ~7
    assert quarter * WAVES <= MAX_SEQS
    key = np.zeros(quarter * WAVES, dtype=np.uint64)
    for j in range(S):
        ln = min(max(int(lens[j]), 0), cap)
        key[j] = np.uint64((ln << 32) | (~j & 0xFFFFFFFF))
    order = np.full(S, -1, dtype=np.int64)
    for b in range((S + WAVE - 1) // WAVE):
        for lane in range(WAVE):
            t = b * WAVE + lane
            if t >= S:
                continue
            rank = 0
            for w in range(WAVES):
                rank += int((key[w * quarter:(w + 1) * quarter] > key[t]).sum())
            assert 0 <= rank < S
            assert order[rank] == -1, "two sequences took one rank"
            order[rank] = t
    return order


@pytest.mark.parametrize("seed", range(6))
def test_order_is_longest_first_permutation(seed):
    rng = np.random.default_rng(seed)
    for S in [2, 3, 63, 64, 65, 255, 256, 257, 600, 1023, 1024][seed % 3::3] + [int(rng.integers(2, 1025))]:
        cap = int(rng.integers(1, 5000))
        lens = rng.choice([-5, 0, 1, 16, 17, cap - 1, cap, cap + 1, 2**31 - 1], size=S)
        lens = np.where(rng.random(S) < 0.5, rng.integers(0, cap + 2, size=S), lens)
        order = order_model(lens, cap)
        assert sorted(order.tolist()) == list(range(S))
        clamped = np.clip(lens, 0, cap)
        expect = sorted(range(S), key=lambda j: (-int(clamped[j]), j))
        assert order.tolist() == expect
