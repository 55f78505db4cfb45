"""Prefix caching end to end on the GPU: the content-hash allocator decides which prompt
blocks are already in the pool, pa_write_kv stores only the rest, and pa_decode's
multi-query path computes the uncached tokens' attention over the whole context.  Every
output row is compared with the oracle's attention over the request's dense history.

K/V rows are synthetic values keyed by the token prefix they end (equal prefixes give equal
rows, as a model's K/V would be), so a cached block holds exactly what the new request would
have written.  [P3 "Prefix 캐싱", "제거"; P1 sec. 6, Fig. 11 and Fig. 22: shared prefixes
of 80 and 341 tokens.]
"""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_40_amd import api, tables_to_array
from paged_kv_cache_40_amd.prefix_cache import PrefixCachingAllocator
from workloads.gen import normal_array
from paged_harness import assert_close, log

pytestmark = pytest.mark.gpu

H, D, B = 8, 128, 16


class Rows:
    """K/V/q rows per distinct token prefix (row i = the prefix's last token)."""

    def __init__(self, seed, capacity=8192):
        self.index = {}
        self.k = normal_array(seed, 21, (capacity, H, D), np.float16)
        self.v = normal_array(seed, 22, (capacity, H, D), np.float16)
        self.q = normal_array(seed, 23, (capacity, H, D), np.float16)

    def ids(self, tokens):
        out = []
        for j in range(len(tokens)):
            key = tuple(tokens[:j + 1])
            if key not in self.index:
                self.index[key] = len(self.index)
            out.append(self.index[key])
        return np.asarray(out)


def family(f, n):
    return [f * 100000 + i for i in range(n)]


def run_wave(alloc, rows, kp, vp, prompts, expect_cached=None):
    """Admit `prompts` as one batch: allocate, write the uncached tokens, attend for them."""
    tables, cached = [], []
    for p in prompts:
        t, c = alloc.allocate(p)
        tables.append(t)
        cached.append(c)
    if expect_cached is not None:
        assert cached == expect_cached, cached
    lens = np.asarray([len(p) for p in prompts], np.int32)
    nq = lens - np.asarray(cached, np.int32)
    loc = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    ids = [rows.ids(p) for p in prompts]
    new_ids = np.concatenate([i[c:] for i, c in zip(ids, cached)])
    bt = torch.from_numpy(tables_to_array(tables)).cuda()
    cl = torch.from_numpy(lens).cuda()
    ql = torch.from_numpy(loc).cuda()
    api.pa_write_kv(kp, vp, torch.from_numpy(rows.k[new_ids]).cuda(),
                    torch.from_numpy(rows.v[new_ids]).cuda(), bt, cl, ql)
    q = torch.from_numpy(rows.q[new_ids]).cuda()
    out = torch.empty_like(q)
    api.pa_decode(out, q, kp, vp, bt, cl, ql, max_context_len=int(lens.max()),
                  max_query_len=int(nq.max()))
    got = out.cpu().numpy()
    for s, (p, i, c) in enumerate(zip(prompts, ids, cached)):
        ref = oracle.attend(rows.q[i[c:]], rows.k[i], rows.v[i], np.arange(c, len(p)))
        assert_close(got[loc[s]:loc[s + 1]], ref, "f16", f"request {s} (cached {c})")
    for t, p in zip(tables, prompts):
        alloc.commit(t, p)
    return tables, cached


def test_prefix_cache_waves_match_dense_attention():
    rows = Rows(7)
    alloc = PrefixCachingAllocator(400, B)
    kp = torch.full((400, B, H, D), float("nan"), dtype=torch.float16, device="cuda")
    vp = torch.full_like(kp, float("nan"))
    A, Bp = family(1, 80), family(2, 341)
    C = A[:40] + family(3, 30)                              # shares 2 full blocks with A
    log("[case] prefix wave 1 (cold)")
    w1, c1 = run_wave(alloc, rows, kp, vp, [A + [7, 8, 9], Bp + list(range(50))],
                      expect_cached=[0, 0])
    log("[case] prefix wave 2 (warm)")
    prompts = [A + list(range(1000, 1000 + n)) for n in (1, 17, 130)] + \
              [Bp + [5], C + [1, 2], A + [7, 8, 9]]
    w2, c2 = run_wave(alloc, rows, kp, vp, prompts,
                      expect_cached=[80, 80, 80, 336, 32, 80])
    for t in w2[:3]:
        assert t[:5] == w1[0][:5]
    assert w2[3][:21] == w1[1][:21]
    assert alloc.hits == 5 * 3 + 21 + 2 + 5
    log("[ok]")


def test_prefix_cache_after_eviction_rewrites_blocks():
    """A pool too small to keep every freed prefix: demoted blocks are handed to new prompts
    and rewritten; later matches only ever return blocks holding the right rows."""
    rows = Rows(8)
    NB = 48
    alloc = PrefixCachingAllocator(NB, B)
    kp = torch.full((NB, B, H, D), float("nan"), dtype=torch.float16, device="cuda")
    vp = torch.full_like(kp, float("nan"))
    rng = np.random.default_rng(3)
    fams = [family(10 + f, int(n)) for f, n in enumerate((80, 200, 341))]
    live = []
    for wave in range(12):
        log(f"[case] eviction wave {wave}")
        prompts = []
        for _ in range(2):
            f = fams[int(rng.integers(3))]
            cut = int(rng.integers(1, len(f) + 1))
            prompts.append(f[:cut] + [10**6 + wave * 100 + j for j in range(int(rng.integers(1, 40)))])
        need = sum(-(-len(p) // B) for p in prompts)
        while live and alloc.num_free() < need:
            alloc.free(live.pop(0))
        tables, _ = run_wave(alloc, rows, kp, vp, prompts)
        live.extend(tables)
    assert alloc.evictions > 0 and alloc.hits > 0
    log(f"[ok] hits {alloc.hits} / lookups {alloc.lookups}, evictions {alloc.evictions}")
