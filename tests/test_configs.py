"""Synthetic inputs: determinism, host/device generator agreement, structure (no GPU)."""

import numpy as np
import pytest
import torch

from workloads import make_config, make_small, normal_values, normal_values_torch
from workloads.gen import normal_array


def test_generator_host_and_torch_agree_bit_for_bit():
    for dt_np, dt_t in ((np.float16, torch.float16), (np.float32, torch.float32)):
        host = normal_array(7, 3, (3, 5, 64), dt_np, offset=(1 << 32) - 100)
        dev = torch.empty((3, 5, 64), dtype=dt_t)
        normal_values_torch(7, 3, dev, offset=(1 << 32) - 100, chunk=129)
        assert host.tobytes() == dev.numpy().tobytes()


def test_generator_is_exact_and_roughly_standard_normal():
    x = normal_values(1, 1, np.arange(1 << 20), np.float64)
    assert np.array_equal(x.astype(np.float16).astype(np.float64), x)   # exact in fp16
    assert np.all(np.round(x * 256) == x * 256)
    assert abs(x.mean()) < 5e-3 and abs(x.var() - 1) < 1e-2
    assert np.abs(x).max() < 6
    y = normal_values(1, 2, np.arange(1 << 20), np.float64)
    assert abs(np.corrcoef(x, y)[0, 1]) < 5e-3
    z = normal_values(2, 1, np.arange(1 << 20), np.float64)
    assert abs(np.corrcoef(x, z)[0, 1]) < 5e-3


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_configs_are_deterministic_and_consistent(idx):
    a, b = make_config(idx), make_config(idx)
    for f in ("context_lens", "query_lens", "write_lens", "block_tables", "filled_before"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    B = a.block_size
    S = a.num_seqs
    nb = -(-a.context_lens.astype(np.int64) // B)
    assert (a.query_lens >= 1).all() and (a.query_lens <= a.context_lens).all()
    assert (a.write_lens <= a.context_lens).all()
    for s in range(S):
        row = a.block_tables[s]
        assert (row[:nb[s]] >= 0).all() and (row[:nb[s]] < a.num_blocks).all()
        assert (row[nb[s]:] == -1).all()
    # every block read holds valid data once the step's copies and writes are done
    filled = a.filled_before.copy()
    if a.copy_pairs is not None:
        for src, dst in a.copy_pairs:
            filled[dst] = filled[src]
    for s in range(S):
        L = int(a.context_lens[s])
        for b in range(nb[s] - 1):
            blk = a.block_tables[s, b]
            pos0 = b * B
            before = L - int(a.write_lens[s])
            expect = min(B, max(0, before - pos0))
            assert filled[blk] >= expect
    # sequences own disjoint blocks except declared sharing (config 3)
    owners = {}
    for s in range(S):
        for blk in a.block_tables[s, :nb[s]]:
            owners.setdefault(int(blk), []).append(s)
    shared = [o for o in owners.values() if len(o) > 1]
    if idx != 3:
        assert not shared


def test_config_sizes():
    c1 = make_config(1)
    assert (c1.num_seqs, c1.num_heads, c1.head_dim, c1.block_size, c1.dtype, c1.num_blocks) == \
        (4, 2, 64, 16, "f32", 64)
    assert c1.context_lens.min() >= 1 and c1.context_lens.max() <= 100
    c2 = make_config(2)
    assert c2.num_seqs == 64 and c2.num_heads == 40 and c2.head_dim == 128
    assert 1 <= c2.context_lens.min() and c2.context_lens.max() <= 2048
    need = int((-(-c2.context_lens // 16)).sum())
    assert c2.num_blocks == -(-5 * need // 4)
    c3 = make_config(3)
    assert c3.num_seqs == 96 and len(c3.copy_pairs) == 80
    assert c3.context_lens.min() >= 1001 and c3.context_lens.max() <= 1300
    src, dst = c3.copy_pairs[:, 0], c3.copy_pairs[:, 1]
    assert len(set(dst)) == 80 and not set(dst) & set(src)
    assert (c3.filled_before[src] == 8).all() and (c3.filled_before[dst] == 0).all()
    c4 = make_config(4)
    assert c4.num_queries == 8 * 512 + 56 and c4.num_heads == 32
    assert sorted(c4.query_lens.tolist()).count(512) == 8
    chunks = c4.query_lens == 512
    assert (c4.context_lens[chunks] >= 512).all() and (c4.context_lens[chunks] <= 2560).all()
    assert (c4.context_lens[~chunks] <= 2048).all()
    c5 = make_config(5)
    assert c5.num_blocks == 47104 and c5.num_seqs == 256 and c5.num_heads == 40
    assert c5.context_lens.min() >= 1025 and c5.context_lens.max() <= 4097
    assert (c5.write_lens == 1).all()
    assert 12e9 < c5.kv_bytes_read() < 15e9


def test_small_variants_host_tensors():
    for idx in (1, 2, 3, 4, 5):
        w = make_small(idx)
        if w.num_blocks * w.block_size * w.num_heads * w.head_dim > 20_000_000:
            continue
        t = w.host_tensors()
        assert t["k_pool"].shape == w.pool_shape()
        valid = np.arange(w.block_size)[None, :] < w.filled_before[:, None]
        assert np.isfinite(t["k_pool"][valid]).all() and np.isnan(t["k_pool"][~valid]).all()
        assert t["q"].shape == (w.num_queries, w.num_heads, w.head_dim)
