"""CPU model of the grouped decode's work split (decode_group_kernel in pa_decode.hip).

The kernel's correctness rests on every wave of a run taking the same joint-or-alone decision
from the tables, so that each (sequence, token) is read exactly once, through its own table
entry (a shared block is the same physical block for every member).  This model restates the
decision rule (fixed P-token partitions; t = longest whole-trip prefix covered by every
member's context in identical blocks; joint when t > 0 and no member has more than P/8 further
tokens) and checks that property, and that every table index and block-entry slot it reads is
in range, on random run layouts including malformed entries and lengths.  No attention
arithmetic: the numerical parity of the kernel itself is tests/test_gpu_group.py.
"""

import numpy as np
import pytest


def sim(ctx, tables, G, P, BS, trip, nblocks, maxb, max_ctx):
    S = len(ctx); cap = min(maxb*BS, max_ctx); kRest = P//8
    cover = {}
    nparts = -(-max_ctx//P)
    for s in range(S):
        for part in range(nparts):
            start = part*P
            if min(ctx[s], cap) <= start: continue
            lead = s - s % G; nmem = min(G, S-lead)
            ck = [min(ctx[lead+k], cap) for k in range(nmem)]
            blk = []
            for k in range(nmem):
                row = []
                if ck[k] > start:
                    nb = -(-min(ck[k]-start, P)//BS)
                    for i in range(nb):
                        j = start//BS + i; assert j < maxb
                        b = tables[lead+k][j]; row.append(b if 0 <= b < nblocks else 0)
                blk.append(row)
            all_in = nmem > 1 and all(c > start for c in ck)
            t = 0
            if all_in:
                reach = min(min(ck)-start, P); nchk = -(-reach//BS)
                fd = nchk
                for i in range(nchk):
                    if any(blk[k][i] != blk[0][i] for k in range(1, nmem)): fd = i; break
                t = min(fd*BS, reach)//trip*trip
                if min(max(ck)-start, P) - t > kRest: t = 0
            joint = t > 0
            if joint and s != lead: continue
            mem = range(nmem) if joint else [s-lead]
            for k in mem:
                end = min(ck[k]-start, P)
                for pos in range(0, end):
                    bi = pos//BS; assert bi < len(blk[k]) and bi < P // BS <= 128
                    key = (lead+k, start+pos)
                    assert key not in cover, key
                    cover[key] = blk[0][bi] if (joint and pos < t) else blk[k][bi]
    for s in range(S):
        for pos in range(max(0, min(ctx[s], cap))):
            assert (s, pos) in cover, (s, pos)
            exp = tables[s][pos//BS]; exp = exp if 0 <= exp < nblocks else 0
            assert cover[(s, pos)] == exp


@pytest.mark.parametrize("seed", range(4))
def test_group_split_covers_every_token_once(seed):
    rng = np.random.default_rng(seed)
    for _ in range(80):
        G = int(rng.integers(2, 7))
        BS = int(rng.choice([8, 16, 32]))
        P = int(rng.choice([256, 512, 1024]))
        trip = int(rng.choice([16, 32]))
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
