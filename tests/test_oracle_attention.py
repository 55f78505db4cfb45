"""Pins for the fp64 attention oracle (no GPU).

The oracle is checked against routes that share none of its code:
  * brute force: pure-Python loops over the attention equation with math.exp
    and no max subtraction, run on each sequence's contiguous K/V history;
  * a library routine: torch's scaled_dot_product_attention in float64 on the
    CPU, on the same contiguous history;
  * closed forms: constant keys -> mean of values; one token -> its value;
    equal values -> that value; scaled values -> scaled output; one dominant
    key -> its value;
  * invariants the pages fix: same result for any placement of blocks in the
    pool, any block size, shared or duplicated prefix blocks
    [P1 "Efficient Memory Management for Large Language Model Serving with
    PagedAttention", sec. 4, Fig. 6: same result as standard attention;
    sec. 6: shared prefix blocks]; decode is invariant under a joint
    permutation of the context tokens;
  * causality: a query never sees a key after its own position.
The tests build pools from contiguous histories with their own block-slice
scatter (not the oracle's per-token gather), so a wrong index in the gather
shows up as a mismatch against brute force.
A final test plants plausible mistakes in copies of the oracle and checks
that these pins catch every one of them.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt


# ---------------------------------------------------------------- helpers --

def history(rng, L, H, d, dtype=np.float64):
    return (rng.standard_normal((L, H, d)).astype(dtype),
            rng.standard_normal((L, H, d)).astype(dtype))


def build_pool(histories, B, NB, rng, tables=None, poison=True):
    """Scatter contiguous per-sequence histories into a pool by whole-block slices.

    Returns (k_pool, v_pool, tables[S][maxb] with -1 padding).
    """
    H, d = histories[0][0].shape[1:]
    k_pool = np.full((NB, B, H, d), np.nan if poison else 0.0)
    v_pool = np.full((NB, B, H, d), np.nan if poison else 0.0)
    need = [-(-k.shape[0] // B) for k, _ in histories]
    if tables is None:
        perm = rng.permutation(NB)
        tables = np.full((len(histories), max(need) + 1), -1, dtype=np.int32)
        pos = 0
        for s, n in enumerate(need):
            tables[s, :n] = perm[pos:pos + n]
            pos += n
    for s, (k, v) in enumerate(histories):
        L = k.shape[0]
        for b in range(need[s]):
            chunk = slice(b * B, min(L, (b + 1) * B))
            n = chunk.stop - chunk.start
            k_pool[tables[s, b], :n] = k[chunk]
            v_pool[tables[s, b], :n] = v[chunk]
    return k_pool, v_pool, tables


def brute_force(q, K, V, p):
    """Attention of one query (position p) by the equation, pure Python, no max subtraction."""
    H, d = len(q), len(q[0])
    out = [[0.0] * d for _ in range(H)]
    for h in range(H):
        w = []
        for j in range(p + 1):
            dot = 0.0
            for e in range(d):
                dot += q[h][e] * K[j][h][e]
            w.append(math.exp(dot / math.sqrt(d)))
        den = sum(w)
        for e in range(d):
            acc = 0.0
            for j in range(p + 1):
                acc += w[j] * V[j][h][e]
            out[h][e] = acc / den
    return out


def sdpa(q, K, V, positions):
    """torch SDPA (float64, CPU) with an explicit causal mask aligned to absolute positions."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]     # [1][H][n][d]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    mask = torch.from_numpy(np.arange(K.shape[0])[None, :] <= np.asarray(positions)[:, None])
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return o[0].numpy().transpose(1, 0, 2)


def rel_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b) / (np.abs(b) + 1e-300))) if a.size else 0.0


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def mixed_batch(rng, B, H=2, d=8, lens=(1, 5, 16, 17, 33), qlens=(1, 3, 1, 17, 4), NB=None):
    hist = [history(rng, L, H, d) for L in lens]
    NB = NB or sum(-(-L // B) for L in lens) + 4
    k_pool, v_pool, bt = build_pool(hist, B, NB, rng)
    qlens = np.asarray(qlens)
    qsl = np.concatenate([[0], np.cumsum(qlens)])
    q = rng.standard_normal((int(qsl[-1]), H, d))
    return hist, k_pool, v_pool, bt, np.asarray(lens), qsl, q


# ------------------------------------------------------ brute force / SDPA --

@pytest.mark.parametrize("B", [1, 4, 16])
def test_matches_brute_force_mixed_batch(B):
    rng = np.random.default_rng(11 + B)
    hist, kp, vp, bt, lens, qsl, q = mixed_batch(rng, B)
    out = oracle.paged_attention(q, kp, vp, bt, lens, B, q_start_loc=qsl)
    for s, (K, V) in enumerate(hist):
        L = lens[s]
        for r in range(qsl[s], qsl[s + 1]):
            p = L - (qsl[s + 1] - qsl[s]) + (r - qsl[s])
            ref = brute_force(q[r].tolist(), K.tolist(), V.tolist(), int(p))
            assert rel_err(out[r], ref) < 1e-12


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_torch_sdpa(seed):
    rng = np.random.default_rng(100 + seed)
    B, H, d = 16, 4, 64
    lens = [1, 15, 16, 17, 100, 257]
    qlens = [1, 1, 16, 5, 37, 1]
    hist = [history(rng, L, H, d) for L in lens]
    kp, vp, bt = build_pool(hist, B, 64, rng)
    qsl = np.concatenate([[0], np.cumsum(qlens)])
    q = rng.standard_normal((int(qsl[-1]), H, d)) * 2.0
    out = oracle.paged_attention(q, kp, vp, bt, np.asarray(lens), B, q_start_loc=qsl)
    for s, (K, V) in enumerate(hist):
        n, L = qlens[s], lens[s]
        ref = sdpa(q[qsl[s]:qsl[s + 1]], K, V, np.arange(L - n, L))
        assert max_abs(out[qsl[s]:qsl[s + 1]], ref) < 1e-12 * max(1.0, np.abs(ref).max())


# ----------------------------------------------------------- closed forms --

def _decode_one(K, V, q, B=16, rng=None):
    rng = rng or np.random.default_rng(0)
    kp, vp, bt = build_pool([(K, V)], B, -(-K.shape[0] // B) + 3, rng)
    return oracle.paged_attention(q[None], kp, vp, bt, np.asarray([K.shape[0]]), B)[0]


def test_constant_keys_give_mean_of_values():
    rng = np.random.default_rng(3)
    L, H, d = 37, 3, 16
    K = np.broadcast_to(rng.standard_normal((1, H, d)), (L, H, d)).copy()
    V = rng.standard_normal((L, H, d))
    o = _decode_one(K, V, rng.standard_normal((H, d)))
    assert max_abs(o, V.mean(axis=0)) < 1e-14


def test_single_token_gives_its_value_exactly():
    rng = np.random.default_rng(4)
    K, V = history(rng, 1, 2, 8)
    o = _decode_one(K, V, rng.standard_normal((2, 8)))
    assert np.array_equal(o, V[0])


def test_equal_values_give_that_value():
    rng = np.random.default_rng(5)
    L, H, d = 50, 2, 8
    K = rng.standard_normal((L, H, d))
    c = rng.standard_normal((1, H, d))
    o = _decode_one(K, np.broadcast_to(c, (L, H, d)).copy(), rng.standard_normal((H, d)))
    assert max_abs(o, c[0]) < 1e-14


def test_values_scale_linearly():
    rng = np.random.default_rng(6)
    K, V = history(rng, 29, 2, 8)
    q = rng.standard_normal((2, 8))
    assert np.array_equal(_decode_one(K, 4.0 * V, q), 4.0 * _decode_one(K, V, q))


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(7)
    L, H, d = 40, 2, 16
    K, V = history(rng, L, H, d)
    q = rng.standard_normal((H, d))
    j = 23
    K[j] = 100.0 * q / np.linalg.norm(q, axis=-1, keepdims=True)
    assert max_abs(_decode_one(K, V, q), V[j]) < 1e-12


# ------------------------------------------------------------- invariants --

def test_block_permutation_is_bit_identical():
    rng = np.random.default_rng(8)
    hist, kp, vp, bt, lens, qsl, q = mixed_batch(rng, 4, NB=40)
    ref = oracle.paged_attention(q, kp, vp, bt, lens, 4, q_start_loc=qsl)
    for trial in range(3):
        kp2, vp2, bt2 = build_pool(hist, 4, 40, np.random.default_rng(50 + trial))
        assert not np.array_equal(bt, bt2)
        out = oracle.paged_attention(q, kp2, vp2, bt2, lens, 4, q_start_loc=qsl)
        assert np.array_equal(out, ref)


def test_block_size_is_bit_identical():
    rng = np.random.default_rng(9)
    lens = [1, 7, 64, 65, 130]
    hist = [history(rng, L, 2, 16) for L in lens]
    q = rng.standard_normal((len(lens), 2, 16))
    outs = []
    for B in (1, 2, 4, 8, 16, 32, 64):
        nb = sum(-(-L // B) for L in lens) + 2
        kp, vp, bt = build_pool(hist, B, nb, np.random.default_rng(B))
        outs.append(oracle.paged_attention(q, kp, vp, bt, np.asarray(lens), B))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_shared_prefix_equals_duplicated_prefix():
    """Two requests share their first three blocks (the prefix-sharing table example of P2
    "Prefix Sharing") vs each owning a private copy of the same prefix."""
    rng = np.random.default_rng(10)
    B, H, d = 4, 2, 8
    prefix = history(rng, 3 * B, H, d)
    tails = [history(rng, 2 * B - 1, H, d), history(rng, 2 * B, H, d)]
    hists = [(np.concatenate([prefix[0], t[0]]), np.concatenate([prefix[1], t[1]]))
             for t in tails]
    lens = np.asarray([h[0].shape[0] for h in hists])
    q = rng.standard_normal((2, H, d))
    # duplicated: every block private
    kp, vp, bt = build_pool(hists, B, 16, rng)
    dup = oracle.paged_attention(q, kp, vp, bt, lens, B)
    # shared: blocks 0..2 identical in both tables, tails private
    shared_tab = np.asarray([[9, 4, 12, 1, 7, -1], [9, 4, 12, 3, 14, -1]], dtype=np.int32)
    kp2, vp2, _ = build_pool(hists, B, 16, rng, tables=shared_tab)
    sh = oracle.paged_attention(q, kp2, vp2, shared_tab, lens, B)
    assert np.array_equal(sh, dup)


def test_decode_invariant_under_token_permutation():
    rng = np.random.default_rng(12)
    K, V = history(rng, 45, 3, 8)
    q = rng.standard_normal((3, 8))
    perm = rng.permutation(45)
    assert rel_err(_decode_one(K[perm], V[perm], q), _decode_one(K, V, q)) < 1e-12


def test_causal_query_ignores_later_keys():
    rng = np.random.default_rng(13)
    B, H, d, L, n = 8, 2, 8, 30, 10
    K, V = history(rng, L, H, d)
    q = rng.standard_normal((n, H, d))
    qsl = np.asarray([0, n])
    kp, vp, bt = build_pool([(K, V)], B, 8, rng)
    ref = oracle.paged_attention(q, kp, vp, bt, np.asarray([L]), B, q_start_loc=qsl)
    # change every key/value after position L-n+4: rows 0..4 must not move
    K2, V2 = K.copy(), V.copy()
    K2[L - n + 5:] = 1e3
    V2[L - n + 5:] = np.nan
    kp2, vp2, _ = build_pool([(K2, V2)], B, 8, rng, tables=bt)
    out = oracle.paged_attention(q, kp2, vp2, bt, np.asarray([L]), B, q_start_loc=qsl)
    assert np.array_equal(out[:5], ref[:5])
    assert np.isnan(out[5:]).all()


def test_unfilled_slots_and_padding_never_read():
    rng = np.random.default_rng(14)
    hist, kp, vp, bt, lens, qsl, q = mixed_batch(rng, 16)
    out = oracle.paged_attention(q, kp, vp, bt, lens, 16, q_start_loc=qsl)   # pool is NaN-poisoned
    assert np.isfinite(out).all()


def test_rejects_more_queries_than_context():
    rng = np.random.default_rng(15)
    hist, kp, vp, bt, lens, qsl, q = mixed_batch(rng, 16)
    with pytest.raises(ValueError):
        oracle.paged_attention(q, kp, vp, bt, np.asarray([1, 2, 16, 17, 33]), 16, q_start_loc=qsl)


# ------------------------------------------------- the pins have teeth --

_attend = oatt.attend
_gather = oatt.gather_context

def _mut_attend_scale_d(q, keys, values, positions, window=0, alibi_slopes=None):
    q, keys, values = (np.asarray(a, np.float64) for a in (q, keys, values))
    d = q.shape[-1]
    out = np.empty(q.shape)
    for r, p in enumerate(positions):
        k, v = keys[:p + 1], values[:p + 1]
        x = np.einsum("hd,jhd->hj", q[r], k) / d                      # planted: 1/d
        w = np.exp(x - x.max(axis=1, keepdims=True))
        out[r] = np.einsum("hj,jhd->hd", w / w.sum(axis=1, keepdims=True), v)
    return out


def _mut_attend_excludes_self(q, keys, values, positions, window=0, alibi_slopes=None):
    q, keys, values = (np.asarray(a, np.float64) for a in (q, keys, values))
    d = q.shape[-1]
    out = np.empty(q.shape)
    for r, p in enumerate(positions):
        n = max(1, int(p))                                            # planted: keys 0..p-1
        k, v = keys[:n], values[:n]
        x = np.einsum("hd,jhd->hj", q[r], k) / np.sqrt(d)
        w = np.exp(x - x.max(axis=1, keepdims=True))
        out[r] = np.einsum("hj,jhd->hd", w / w.sum(axis=1, keepdims=True), v)
    return out


def _mut_attend_norm_over_heads(q, keys, values, positions, window=0, alibi_slopes=None):
    q, keys, values = (np.asarray(a, np.float64) for a in (q, keys, values))
    d = q.shape[-1]
    out = np.empty(q.shape)
    for r, p in enumerate(positions):
        k, v = keys[:p + 1], values[:p + 1]
        x = np.einsum("hd,jhd->hj", q[r], k) / np.sqrt(d)
        w = np.exp(x - x.max())
        out[r] = np.einsum("hj,jhd->hd", w / w.sum(axis=0, keepdims=True), v)   # planted: axis
    return out


def _mut_attend_keys_as_values(q, keys, values, positions, window=0, alibi_slopes=None):
    return _attend(q, keys, keys, positions, window, alibi_slopes)    # planted: swapped operand


def _mut_gather_slot(pool, table_row, length, block_size):
    out = np.empty((length,) + pool.shape[2:])
    for j in range(length):
        out[j] = pool[int(table_row[j // block_size]), (j + 1) % block_size]   # planted: slot + 1
    return out


def _mut_gather_entry(pool, table_row, length, block_size):
    out = np.empty((length,) + pool.shape[2:])
    for j in range(length):
        out[j] = pool[int(table_row[j % block_size % len(table_row)]), j // block_size % block_size]
    return out


def _mut_positions_shift(q_rows, k_pool, v_pool, table_row, context_len, block_size, heads=None,
                         window=0, alibi_slopes=None):
    n = q_rows.shape[0]
    keys = _gather(k_pool, table_row, context_len, block_size)
    values = _gather(v_pool, table_row, context_len, block_size)
    return _attend(q_rows, keys, values, np.arange(context_len - n - 1, context_len - 1).clip(0))


def _pins_pass():
    """Run the brute-force and SDPA pins; True when the (possibly mutated) oracle passes them."""
    try:
        for B in (1, 4, 16):
            test_matches_brute_force_mixed_batch(B)
        test_matches_torch_sdpa(0)
        test_single_token_gives_its_value_exactly()
        test_dominant_key_selects_its_value()
    except (AssertionError, ValueError, IndexError, FloatingPointError):
        return False
    return True


MUTANTS = [
    ("attend", _mut_attend_scale_d),
    ("attend", _mut_attend_excludes_self),
    ("attend", _mut_attend_norm_over_heads),
    ("attend", _mut_attend_keys_as_values),
    ("gather_context", _mut_gather_slot),
    ("gather_context", _mut_gather_entry),
    ("paged_attention_seq", _mut_positions_shift),
]


def test_unmutated_oracle_passes_pins():
    assert _pins_pass()


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, name, mutant):
    monkeypatch.setattr(oatt, name, mutant)
    assert not _pins_pass()
