"""CPU model of the grouped decode's work split (decode_group_kernel in pa_decode.hip).

One workgroup per (run of G neighbouring sequences, head, P-token partition).  From the
members' context lengths and table entries alone it derives:
  * the active members: those whose context reaches into the partition;
  * t = the longest prefix of the partition, in whole trips, that every active member's
    context covers and that lies in the same physical blocks for all of them (at least two
    active members, else t = 0);
  * the work items: the t/trip joint trips (each token row read once, through the first
    active member's entries, and used for every active member), then each active member's own
    trips from t to the end of its context in the partition (through its own entries);
and deals the items to its waves round-robin.  The kernel's correctness rests on every
(sequence, token) being used exactly once, read through a block equal to its own table entry
(invalid entries read block 0 on both sides), with every table index in range.  This model
restates the rule and checks that, and that the waves' shares partition the items, on random
run layouts including malformed entries and lengths.  No attention arithmetic: the numerical
parity of the kernel itself is tests/test_gpu_group.py.
"""

import numpy as np
import pytest


def sim(ctx, tables, G, P, BS, trip, nblocks, maxb, max_ctx, waves=4):
    S = len(ctx)
    cap = min(maxb * BS, max_ctx)
    cover = {}
    nparts = -(-max_ctx // P)
    nruns = -(-S // G)
    for r in range(nruns):
        lead = r * G
        nmem = min(G, S - lead)
        for part in range(nparts):
            start = part * P
            ck = [min(ctx[lead + k], cap) for k in range(nmem)]
            active = [k for k in range(nmem) if ck[k] > start]
            blk = {}
            for k in active:
                nb = -(-min(ck[k] - start, P) // BS)
                row = []
                for i in range(nb):
                    j = start // BS + i
                    assert j < maxb and i < P // BS <= 128
                    b = tables[lead + k][j]
                    row.append(b if 0 <= b < nblocks else 0)
                blk[k] = row
            t = 0
            if len(active) >= 2:
                reach = min(min(ck[k] - start for k in active), P)
                nchk = -(-reach // BS)
                fd = nchk
                for i in range(nchk):
                    if any(blk[k][i] != blk[active[0]][i] for k in active[1:]):
                        fd = i
                        break
                t = min(fd * BS, reach) // trip * trip
            items = [(-1, j * trip) for j in range(t // trip)]
            for k in active:
                end = min(ck[k] - start, P)
                items += [(k, rel) for rel in range(t, end, trip)]
            dealt = sorted(i for w in range(waves) for i in range(w, len(items), waves))
            assert dealt == list(range(len(items)))
            for k_item, rel in items:
                mem = active if k_item < 0 else [k_item]
                src = active[0] if k_item < 0 else k_item
                for k in mem:
                    end = min(ck[k] - start, P)
                    for pos in range(rel, min(rel + trip, end)):
                        bi = pos // BS
                        assert bi < len(blk[src])
                        key = (lead + k, start + pos)
                        assert key not in cover, key
                        cover[key] = blk[src][bi]
    for s in range(S):
        for pos in range(max(0, min(ctx[s], cap))):
            assert (s, pos) in cover, (s, pos)
            exp = tables[s][pos // BS]
            exp = exp if 0 <= exp < nblocks else 0
            assert cover[(s, pos)] == exp


@pytest.mark.parametrize("seed", range(4))
def test_group_split_covers_every_token_once(seed):
    rng = np.random.default_rng(seed)
    for _ in range(80):
        G = int(rng.integers(2, 7))
        BS = int(rng.choice([8, 16, 32]))
        P = int(rng.choice([256, 512, 1024]))
        trip = int(rng.choice([16, 32]))  # trips of head_dim 128 and 64
        S = int(rng.integers(1, 20))
        nblocks, maxb = 4000, 80
        base = int(rng.integers(0, 900))
        ctx, tables = [], []
        for s in range(S):
            if s % G == 0:
                shared = rng.permutation(nblocks)[:maxb]
            ctx.append(int(np.clip(base + rng.integers(-50, 300), -3, maxb * BS)))
            t = shared.copy()
            d = int(rng.integers(0, maxb))
            t[d:] = rng.integers(-2, nblocks + 2, size=maxb - d)
            tables.append(t)
        max_ctx = min(max(1, max(ctx)), maxb * BS)
        sim(ctx, tables, G, P, BS, trip, nblocks, maxb, max_ctx)
