"""Pins for the oracle's slot write, block copy and size formulas (no GPU).

write_kv is checked against an independent route: pools built by whole-block
slices from each sequence's contiguous history.  Writing the last n tokens of
the history into a pool that holds only the first L-n must give exactly the
pool that holds all L [P2 "SOSP 2023論文解説: vLLM — PagedAttentionによる
KVキャッシュメモリ管理の革新", pseudocode: append_token].
copy_blocks is checked block by block [P2 pseudocode: copy_on_write copies the
whole block].  swap_blocks is checked by a preemption round trip: blocks moved
to a host pool, their device blocks overwritten, moved back into other blocks
and the tables rewritten must give bit-identical attention [P1 sec. 5:
swapped blocks are restored; P3 "오프로딩": resumed without recomputation].  Sizes are pinned to the figures the pages print
(tests/golden/kv_sizes.json) and to the byte size of real arrays.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import kv_ops

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def scatter(histories, counts, B, NB, tables):
    """Pool holding the first counts[s] tokens of each history, NaN elsewhere (block slices)."""
    H, d = histories[0].shape[1:]
    pool = np.full((NB, B, H, d), np.nan, dtype=np.float32)
    for s, h in enumerate(histories):
        n = counts[s]
        for b in range(-(-n // B)):
            lo, hi = b * B, min(n, (b + 1) * B)
            pool[tables[s][b], :hi - lo] = h[lo:hi]
    return pool


def make_case(rng, B=4, H=2, d=4, lens=(1, 4, 5, 9, 16, 17), wlens=(1, 1, 3, 9, 2, 17)):
    need = [-(-L // B) for L in lens]
    NB = sum(need) + 3
    perm = rng.permutation(NB)
    tables, pos = [], 0
    for n in need:
        tables.append(perm[pos:pos + n].tolist() + [-1])
        pos += n
    width = max(len(t) for t in tables)
    bt = np.asarray([t + [-1] * (width - len(t)) for t in tables], np.int32)
    kh = [rng.standard_normal((L, H, d)).astype(np.float32) for L in lens]
    vh = [rng.standard_normal((L, H, d)).astype(np.float32) for L in lens]
    return lens, wlens, NB, bt, kh, vh


@pytest.mark.parametrize("B", [1, 4, 16])
def test_write_equals_full_scatter(B):
    rng = np.random.default_rng(B)
    lens, wlens, NB, bt, kh, vh = make_case(rng, B=B)
    before = [L - n for L, n in zip(lens, wlens)]
    kp0 = scatter(kh, before, B, NB, bt)
    vp0 = scatter(vh, before, B, NB, bt)
    wsl = np.concatenate([[0], np.cumsum(wlens)])
    k_new = np.concatenate([h[L - n:] for h, L, n in zip(kh, lens, wlens)])
    v_new = np.concatenate([h[L - n:] for h, L, n in zip(vh, lens, wlens)])
    kp, vp = oracle.write_kv(kp0, vp0, k_new, v_new, bt, np.asarray(lens), B, write_start_loc=wsl)
    assert np.array_equal(kp, scatter(kh, lens, B, NB, bt), equal_nan=True)
    assert np.array_equal(vp, scatter(vh, lens, B, NB, bt), equal_nan=True)
    # inputs untouched
    assert np.array_equal(kp0, scatter(kh, before, B, NB, bt), equal_nan=True)


def test_write_one_token_per_sequence_default_layout():
    rng = np.random.default_rng(7)
    B = 4
    lens, _, NB, bt, kh, vh = make_case(rng, B=B)
    wl = [1] * len(lens)
    kp0 = scatter(kh, [L - 1 for L in lens], B, NB, bt)
    vp0 = scatter(vh, [L - 1 for L in lens], B, NB, bt)
    k_new = np.stack([h[-1] for h in kh])
    v_new = np.stack([h[-1] for h in vh])
    kp, vp = oracle.write_kv(kp0, vp0, k_new, v_new, bt, np.asarray(lens), B)
    assert np.array_equal(kp, scatter(kh, lens, B, NB, bt), equal_nan=True)
    assert np.array_equal(vp, scatter(vh, lens, B, NB, bt), equal_nan=True)
    del wl


def _mut_write_slot(k_pool, v_pool, k_new, v_new, block_tables, context_lens, block_size,
                    write_start_loc=None):
    S = len(context_lens)
    wsl = np.arange(S + 1) if write_start_loc is None else write_start_loc
    k_out, v_out = k_pool.copy(), v_pool.copy()
    for s in range(S):
        a, b = int(wsl[s]), int(wsl[s + 1])
        n, L = b - a, int(context_lens[s])
        for i in range(n):
            pos = L - n + i + 1                                    # planted: one slot late
            phys = int(block_tables[s][min(pos // block_size, len(block_tables[s]) - 1)])
            k_out[phys, pos % block_size] = k_new[a + i]
            v_out[phys, pos % block_size] = v_new[a + i]
    return k_out, v_out


def test_write_pin_catches_planted_slot_error(monkeypatch):
    monkeypatch.setattr(kv_ops, "write_kv", _mut_write_slot)
    monkeypatch.setattr(oracle, "write_kv", _mut_write_slot)
    with pytest.raises(AssertionError):
        test_write_equals_full_scatter(4)


def test_copy_blocks_whole_block_and_snapshot():
    rng = np.random.default_rng(3)
    kp = rng.standard_normal((10, 4, 2, 3)).astype(np.float16)
    vp = rng.standard_normal((10, 4, 2, 3)).astype(np.float16)
    kp[5, 2:] = np.nan                      # an unfilled tail is copied as it is
    pairs = np.asarray([[5, 1], [2, 7], [5, 9]], np.int32)
    k2, v2 = oracle.copy_blocks(kp, vp, pairs)
    for src, dst in pairs:
        assert k2[dst].tobytes() == kp[src].tobytes()
        assert v2[dst].tobytes() == vp[src].tobytes()
    untouched = [b for b in range(10) if b not in (1, 7, 9)]
    assert k2[untouched].tobytes() == kp[untouched].tobytes()
    # pairs read the pool as it was before the call
    k3, _ = oracle.copy_blocks(kp, vp, np.asarray([[0, 1], [1, 2]], np.int32))
    assert k3[2].tobytes() == kp[1].tobytes()
    # no pairs: unchanged copy
    k4, v4 = oracle.copy_blocks(kp, vp, np.zeros((0, 2), np.int32))
    assert k4.tobytes() == kp.tobytes() and k4 is not kp


# ------------------------------------------------------------------- swap --

def test_swap_blocks_bytes_and_payloads():
    rng = np.random.default_rng(4)
    dev_k = rng.standard_normal((12, 4, 2, 3)).astype(np.float16)
    dev_v = rng.standard_normal((12, 4, 2, 3)).astype(np.float16)
    # a NaN with a payload: swapping moves bits, so the payload must survive
    dev_k.view(np.uint16)[3, 1, 0, 0] = 0x7E5A
    host_k = np.full((12, 4, 2, 3), np.nan, np.float16)
    host_v = np.full((12, 4, 2, 3), np.nan, np.float16)
    pairs = np.asarray([[3, 0], [7, 4], [11, 5]], np.int32)
    hk, hv = oracle.swap_blocks(host_k, host_v, dev_k, dev_v, pairs)
    for src, dst in pairs:
        assert hk[dst].tobytes() == dev_k[src].tobytes()
        assert hv[dst].tobytes() == dev_v[src].tobytes()
    assert hk.view(np.uint16)[0, 1, 0, 0] == 0x7E5A
    for b in (1, 2, 3):
        assert hk[b].tobytes() == host_k[b].tobytes()
    # the source pool is only read; no pairs: an unchanged copy
    assert hk is not host_k
    e_k, e_v = oracle.swap_blocks(dev_k, dev_v, hk, hv, np.zeros((0, 2), np.int32))
    assert e_k.tobytes() == dev_k.tobytes() and e_v.tobytes() == dev_v.tobytes()


def test_swap_round_trip_restores_attention():
    rng = np.random.default_rng(5)
    B = 4
    lens, _, NB, bt, kh, vh = make_case(rng, B=B, lens=(3, 9, 16, 17), wlens=(1, 1, 1, 1))
    NB += 10                                                   # room to swap back elsewhere
    kp = scatter(kh, lens, B, NB, bt)
    vp = scatter(vh, lens, B, NB, bt)
    q = rng.standard_normal((4, 2, 4))
    before = oracle.paged_attention(q, kp, vp, bt, np.asarray(lens), B)
    # swap sequences 1 and 3 out to a host pool
    out_seqs = [1, 3]
    blocks = [int(b) for s in out_seqs for b in bt[s] if b >= 0]
    host_ids = rng.permutation(len(blocks) + 2)[:len(blocks)]
    hk = np.full((len(blocks) + 2,) + kp.shape[1:], np.nan, np.float32)
    hv = hk.copy()
    hk, hv = oracle.swap_blocks(hk, hv, kp, vp, np.stack([blocks, host_ids], 1))
    # their device blocks are reused by others meanwhile
    kp[blocks] = rng.standard_normal(kp[blocks].shape)
    vp[blocks] = rng.standard_normal(vp[blocks].shape)
    # swap back into blocks nobody holds, and rewrite the two tables
    used = {int(b) for b in bt.reshape(-1) if b >= 0}
    free = [b for b in rng.permutation(NB) if int(b) not in used][:len(blocks)]
    kp, vp = oracle.swap_blocks(kp, vp, hk, hv, np.stack([host_ids, free], 1))
    bt2 = bt.copy()
    it = iter(free)
    for s in out_seqs:
        for i, b in enumerate(bt2[s]):
            if b >= 0:
                bt2[s, i] = next(it)
    after = oracle.paged_attention(q, kp, vp, bt2, np.asarray(lens), B)
    assert np.array_equal(before, after)


def _mut_swap_kv_crossed(dst_k, dst_v, src_k, src_v, pairs):
    k_out, v_out = dst_k.copy(), dst_v.copy()
    for src, dst in np.asarray(pairs).reshape(-1, 2):
        k_out[int(dst)] = src_v[int(src)]                       # planted: K and V crossed
        v_out[int(dst)] = src_k[int(src)]
    return k_out, v_out


_swap = kv_ops.swap_blocks


def _mut_swap_pair_reversed(dst_k, dst_v, src_k, src_v, pairs):
    return _swap(dst_k, dst_v, src_k, src_v, np.asarray(pairs).reshape(-1, 2)[:, ::-1])


@pytest.mark.parametrize("mutant", [_mut_swap_kv_crossed, _mut_swap_pair_reversed])
def test_swap_pins_catch_planted_mistake(monkeypatch, mutant):
    monkeypatch.setattr(oracle, "swap_blocks", mutant)
    caught = 0
    for pin in (test_swap_blocks_bytes_and_payloads, test_swap_round_trip_restores_attention):
        try:
            pin()
        except AssertionError:
            caught += 1
        except IndexError:          # a reversed pair may also leave the pool; not counted
            pass
    assert caught >= 1


# ------------------------------------------------------------------ sizes --

def test_sizes_match_printed_figures():
    cases = json.load(open(os.path.join(GOLDEN, "kv_sizes.json")))["cases"]
    exact = cases[0]
    assert oracle.kv_bytes_per_token(exact["num_layers"], exact["num_heads"], exact["head_dim"],
                                     exact["elt_bytes"]) == exact["bytes_per_token"]
    approx = cases[1]
    got = oracle.kv_bytes_per_token(40, 40, 128, 2) / approx["approx_unit_bytes"]
    assert abs(got - approx["approx_value"]) <= approx["rel_tol"] * approx["approx_value"]
    req = cases[2]
    got = req["tokens"] * oracle.kv_bytes_per_token(40, 40, 128, 2) / req["approx_unit_bytes"]
    assert abs(got - req["approx_value"]) <= req["rel_tol"] * req["approx_value"]
    assert cases[3]["block_size"] == 16


def test_sizes_match_real_arrays():
    # one token: a K and a V row per layer, [layers][heads][head_dim] fp16 each
    L, H, d = 3, 5, 64
    kv = np.zeros((2, L, H, d), dtype=np.float16)
    assert oracle.kv_bytes_per_token(L, H, d, 2) == kv.nbytes
    blk = np.zeros((2, L, 16, H, d), dtype=np.float32)
    assert oracle.block_bytes(L, H, d, 16, 4) == blk.nbytes
    # a single-layer block of the [B][H][d] layout the pools use, K plus V
    pool_block = np.zeros((16, 40, 128), np.float16)
    assert 2 * pool_block.nbytes == oracle.block_bytes(1, 40, 128, 16, 2) == 327680
