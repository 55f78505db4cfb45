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


# ------------------------------------------------------------ value recipes --

def test_full_mantissa_host_and_torch_agree_and_are_not_fp16():
    from workloads.gen import full_values
    host = normal_array(9, 4, (7, 3, 64), np.float32, offset=(1 << 32) - 50, full=True)
    dev = torch.empty((7, 3, 64), dtype=torch.float32)
    normal_values_torch(9, 4, dev, offset=(1 << 32) - 50, chunk=97, full=True)
    assert host.tobytes() == dev.numpy().tobytes()
    x = full_values(1, 1, np.arange(1 << 18), np.float64)
    # close to the grid value it perturbs, a full fp32 mantissa, almost never exact in fp16
    base = normal_values(1, 1, np.arange(1 << 18), np.float64)
    assert np.abs(x - base).max() <= 2.0 ** -9
    x32 = x.astype(np.float32)
    assert np.mean(x32.astype(np.float16).astype(np.float32) != x32) > 0.999
    assert abs(x.mean()) < 1e-2 and abs(x.var() - 1) < 2e-2


def test_full_values_only_for_fp32():
    with pytest.raises(ValueError):
        make_small(2, values="full")
    w = make_config(1, values="full")
    h = w.host_tensors()
    for name in ("k_pool", "v_pool", "q"):
        a = h[name][np.isfinite(h[name])]
        assert np.mean(a.astype(np.float16).astype(np.float32) != a) > 0.99, name


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_marked_values_host_and_torch_agree(dtype):
    from workloads import make_custom_decode
    w = make_custom_decode(3, dtype, 3, 64, 16, [1, 17, 40, 100], write_one=True, k_scale=0.125,
                           v_mark=512.0)
    h = w.host_tensors()
    d = w.device_tensors("cpu")
    for name in ("k_pool", "v_pool", "q", "k_new", "v_new"):
        a, b = h[name], d[name].numpy()
        assert a.dtype == b.dtype and a.tobytes() == b.tobytes(), name


def test_marked_values_alternate_by_logical_block():
    from workloads import make_custom_decode
    w = make_custom_decode(4, "f16", 2, 64, 16, [70, 33], write_one=True, k_scale=0.125,
                           v_mark=1024.0)
    h = w.host_tensors()
    r = w.head_dim_signs()
    assert set(np.unique(r)) == {-1.0, 1.0}
    B = w.block_size
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        for j in range(L - 1):                      # tokens already in the pool
            blk = w.block_tables[s, j // B]
            v = h["v_pool"][blk, j % B].astype(np.float64)
            want = (1 if (j // B) % 2 == 0 else -1) * 1024.0 * r
            assert np.abs(v - want).max() <= 8, (s, j)
        # the appended token carries its own block's sign
        v = h["v_new"][s].astype(np.float64)
        want = (1 if ((L - 1) // B) % 2 == 0 else -1) * 1024.0 * B * r
        assert np.abs(v - want).max() <= 16
    k = h["k_pool"][np.isfinite(h["k_pool"])]
    assert np.abs(k).max() <= 6 / 8


@pytest.mark.parametrize("recipe", [dict(), dict(k_scale=0.125, v_mark=256.0)])
def test_host_block_rows_match_whole_pool(recipe):
    from workloads import make_custom_decode
    w = make_custom_decode(5, "f16", 3, 64, 16, [5, 40, 100], write_one=True, **recipe)
    h = w.host_tensors()
    blocks = [int(w.block_tables[1, 1]), int(w.block_tables[2, 0]), int(w.block_tables[0, 0])]
    for heads in (None, [2], [0, 2]):
        r = w.host_block_rows(blocks, heads)
        sel = slice(None) if heads is None else heads
        for name in ("k_pool", "v_pool"):
            want = h[name][blocks][:, :, sel]
            assert r[name].tobytes() == want.tobytes(), (name, heads)
    nr = w.host_new_rows([1, 2])
    assert nr["k_new"].tobytes() == h["k_new"][:, [1, 2]].tobytes()
    assert nr["v_new"].tobytes() == h["v_new"][:, [1, 2]].tobytes()
    wf = make_config(1, values="full")
    hf = wf.host_tensors()
    r = wf.host_block_rows([3, 7])
    assert r["v_pool"].tobytes() == hf["v_pool"][[3, 7]].tobytes()
