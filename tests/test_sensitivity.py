"""How sharp the parity checks are (no GPU).

* The drop-one helper (tests/sensitivity.py) equals the oracle's attention over the
  history with the group really removed.
* On exactly the inputs of the long-context GPU tests (tests/cases.py), leaving out any
  one block - or only the appended token - moves the exact output past the fp16
  tolerance, so a kernel that skipped a block, dropped the one-token last partition or
  merged partitions wrongly would fail them.
* On the fp32 batches the GPU tests use, the exact output of the inputs rounded to
  fp16 differs from the exact output by more than the fp32 tolerance, so an fp32 path
  that went through fp16 anywhere in q, K or V would fail them.
"""

import numpy as np
import pytest

import oracle
from cases import long_chunk_marked, long_decode_marked
from sensitivity import drop_block_margins, drop_last_token_margin, drop_one_margins, outputs_without
from workloads import make_config, make_custom_decode

F16 = (2e-3, 1e-2)


def test_drop_one_matches_oracle_with_the_group_removed():
    rng = np.random.default_rng(0)
    L, H, D, B = 203, 3, 64, 16
    q = rng.standard_normal((H, D))
    k = rng.standard_normal((L, H, D))
    v = rng.standard_normal((L, H, D))
    groups = np.arange(L) // B
    og, o = outputs_without(q, k, v, groups)
    ref = oracle.attend(q[None], k, v, [L - 1])[0]
    assert np.abs(o - ref).max() <= 1e-12 * np.abs(ref).max()
    for g in range(groups.max() + 1):
        keep = groups != g
        want = oracle.attend(q[None], k[keep], v[keep], [int(keep.sum()) - 1])[0]
        assert np.abs(og[g] - want).max() <= 1e-12 * np.abs(want).max(), g
    m = drop_one_margins(q, k, v, groups, *F16)
    want = np.array([np.max(np.abs(og[g] - o) / (F16[0] + F16[1] * np.abs(o)))
                     for g in range(len(og))])
    assert np.allclose(m, want, rtol=1e-12)


def _history(w, s, heads):
    """The sequence's keys and values after the step (heads given), through the oracle's own
    write and gather on a compact pool of its blocks; and its query row."""
    B = w.block_size
    L = int(w.context_lens[s])
    nb = -(-L // B)
    blocks = w.block_tables[s, :nb]
    rows = w.host_block_rows(blocks, heads)
    new = w.host_new_rows(heads)
    wsl = w.write_start_loc()
    a, b = (s, s + 1) if wsl is None else (int(wsl[s]), int(wsl[s + 1]))
    table = np.arange(nb, dtype=np.int32)[None]
    kp, vp = oracle.write_kv(rows["k_pool"], rows["v_pool"], new["k_new"][a:b], new["v_new"][a:b],
                             table, np.asarray([L], np.int32), B,
                             np.asarray([0, b - a], np.int32))
    keys = oracle.gather_context(kp, table[0], L, B)
    vals = oracle.gather_context(vp, table[0], L, B)
    return keys, vals


def _query_rows(w, heads):
    from workloads.gen import normal_array
    q = normal_array(w.seed, 3, (w.num_queries, w.num_heads, w.head_dim), w.np_dtype)
    return (q * w.np_dtype(w.q_scale))[:, heads].astype(np.float64)


@pytest.mark.parametrize("s", [0, 1])
def test_long_decode_inputs_expose_any_dropped_block(s):
    w = long_decode_marked()
    assert int(w.context_lens[s]) in (100000, 65537)
    heads = [0]
    keys, vals = _history(w, s, heads)
    q = _query_rows(w, heads)[s]
    blocks = drop_block_margins(q, keys, vals, w.block_size, *F16)
    last = drop_last_token_margin(q, keys, vals, *F16)
    # whole 2,048-token partitions are bigger still; a block is the smallest unit a kernel reads
    assert blocks.min() >= 3.0, (s, blocks.min(), int(blocks.argmin()))
    assert last >= 3.0, (s, last)


def test_long_chunk_inputs_expose_any_dropped_block():
    w = long_chunk_marked()
    s = int(np.argmax(w.context_lens))
    assert int(w.context_lens[s]) == 30300 and int(w.query_lens[s]) == 300
    heads = [0]
    keys, vals = _history(w, s, heads)
    q = _query_rows(w, heads)
    qsl = w.q_start_loc()
    L, n = int(w.context_lens[s]), int(w.query_lens[s])
    # the chunk's first query (position L-n: the prior plus itself) and its last one: every
    # whole block it sees (the block holding the query itself may be cut short)
    for i in (0, n - 1):
        p = L - n + i
        m = drop_block_margins(q[qsl[s] + i], keys[:p + 1], vals[:p + 1], w.block_size, *F16)
        m = m[:(p + 1) // w.block_size]
        assert m.min() >= 3.0, (i, m.min(), int(m.argmin()))


def _f32_cases():
    yield make_config(1, values="full")
    yield make_custom_decode(11, "f32", 3, 64, 16, [1, 2, 9, 17, 255, 257, 513, 1000],
                             values="full", name="edges_f32")


@pytest.mark.parametrize("case", list(range(2)))
def test_fp32_inputs_expose_an_fp16_rounding_path(case):
    w = list(_f32_cases())[case]
    h = w.host_tensors()
    ref = oracle.paged_attention(h["q"], h["k_pool"], h["v_pool"], h["block_tables"],
                                 h["context_lens"], w.block_size)
    for name in ("q", "k_pool", "v_pool"):
        planted = {k: h[k] for k in ("q", "k_pool", "v_pool")}
        planted[name] = h[name].astype(np.float16).astype(np.float32)
        bad = oracle.paged_attention(planted["q"], planted["k_pool"], planted["v_pool"],
                                     h["block_tables"], h["context_lens"], w.block_size)
        # the fp32 tolerance is 1e-5 absolute: the planted path must exceed it somewhere
        assert np.abs(bad - ref).max() > 3e-5, (w.name, name, np.abs(bad - ref).max())
