"""Pins for the oracle's sliding-window and ALiBi variants (no GPU).

Readings (oracle/attention.py): with window W the query at position p sees keys
p-W+1..p; ALiBi adds slope_h * (j - p) to the score of key j.  Pinned by
  * brute force (pure Python loops, math.exp, no max subtraction);
  * torch scaled_dot_product_attention with an additive float mask (the bias,
    and -inf outside the window), fp64 on the CPU;
  * reductions to the plain case: a window at least as long as the context
    gives bit-identical results, all-zero slopes the same results to rounding;
  * window = 1 returns the query's own value row exactly;
  * a windowed query equals plain attention over only the last W tokens of its
    history (a different route: truncate the history, rebuild the pool);
  * a very large slope leaves only the nearest key;
  * planted mistakes (bias sign, window off by one) fail these pins.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from test_oracle_attention import build_pool, history, max_abs, rel_err


def brute(q, K, V, p, window=0, slopes=None):
    H, d = len(q), len(q[0])
    lo = max(0, p - window + 1) if window > 0 else 0
    out = [[0.0] * d for _ in range(H)]
    for h in range(H):
        w = []
        for j in range(lo, p + 1):
            dot = sum(q[h][e] * K[j][h][e] for e in range(d)) / math.sqrt(d)
            if slopes is not None:
                dot += slopes[h] * (j - p)
            w.append(math.exp(dot))
        den = sum(w)
        for e in range(d):
            out[h][e] = sum(w[j - lo] * V[j][h][e] for j in range(lo, p + 1)) / den
    return out


def batch(rng, B=4, H=3, d=8, lens=(1, 6, 17, 40), qlens=(1, 2, 5, 9)):
    hist = [history(rng, L, H, d) for L in lens]
    NB = sum(-(-L // B) for L in lens) + 3
    kp, vp, bt = build_pool(hist, B, NB, rng)
    qsl = np.concatenate([[0], np.cumsum(qlens)])
    q = rng.standard_normal((int(qsl[-1]), H, d))
    return hist, kp, vp, bt, np.asarray(lens), qsl, q


@pytest.mark.parametrize("window,use_slopes", [(0, True), (3, False), (7, True), (1, True)])
def test_brute_force(window, use_slopes):
    rng = np.random.default_rng(window + 10 * use_slopes)
    hist, kp, vp, bt, lens, qsl, q = batch(rng)
    slopes = np.asarray([0.5, 0.125, 0.03125]) if use_slopes else None
    out = oracle.paged_attention(q, kp, vp, bt, lens, 4, q_start_loc=qsl, window=window,
                                 alibi_slopes=slopes)
    for s, (K, V) in enumerate(hist):
        n, L = qsl[s + 1] - qsl[s], lens[s]
        for r in range(qsl[s], qsl[s + 1]):
            p = int(L - n + (r - qsl[s]))
            ref = brute(q[r].tolist(), K.tolist(), V.tolist(), p, window,
                        None if slopes is None else slopes.tolist())
            assert rel_err(out[r], ref) < 1e-12


def test_sdpa_with_bias_mask():
    rng = np.random.default_rng(3)
    H, d, L, n, W = 4, 32, 90, 12, 25
    K, V = history(rng, L, H, d)
    q = rng.standard_normal((n, H, d))
    slopes = 2.0 ** -np.arange(1, H + 1)
    kp, vp, bt = build_pool([(K, V)], 16, 10, rng)
    out = oracle.paged_attention(q, kp, vp, bt, np.asarray([L]), 16, q_start_loc=np.asarray([0, n]),
                                 window=W, alibi_slopes=slopes)
    pos = np.arange(L - n, L)
    j = np.arange(L)
    bias = slopes[:, None, None] * (j[None, None, :] - pos[None, :, None])       # [H][n][L]
    visible = (j[None, :] <= pos[:, None]) & (j[None, :] > pos[:, None] - W)
    mask = torch.from_numpy(np.where(visible[None], bias, -np.inf))
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[None])
    assert max_abs(out, ref[0].numpy().transpose(1, 0, 2)) < 1e-12


def test_reductions_to_plain_are_bit_identical():
    rng = np.random.default_rng(4)
    hist, kp, vp, bt, lens, qsl, q = batch(rng)
    plain = oracle.paged_attention(q, kp, vp, bt, lens, 4, q_start_loc=qsl)
    long_window = oracle.paged_attention(q, kp, vp, bt, lens, 4, q_start_loc=qsl,
                                         window=int(lens.max()))
    zero_slopes = oracle.paged_attention(q, kp, vp, bt, lens, 4, q_start_loc=qsl,
                                         alibi_slopes=np.zeros(3))
    assert np.array_equal(long_window, plain)          # same key slices, same arithmetic
    # adding 0 * (j - p) is exact; the product with V is recomputed on a new buffer, and NumPy's
    # reduction kernels may order a sum differently by buffer alignment, hence a rounding bound
    assert max_abs(zero_slopes, plain) < 1e-14


def test_window_one_returns_own_value():
    rng = np.random.default_rng(5)
    hist, kp, vp, bt, lens, qsl, q = batch(rng)
    out = oracle.paged_attention(q, kp, vp, bt, lens, 4, q_start_loc=qsl, window=1,
                                 alibi_slopes=np.asarray([1.0, 2.0, 3.0]))
    for s, (K, V) in enumerate(hist):
        n, L = qsl[s + 1] - qsl[s], lens[s]
        for r in range(qsl[s], qsl[s + 1]):
            assert np.array_equal(out[r], V[L - n + (r - qsl[s])])


@pytest.mark.parametrize("use_slopes", [False, True])
def test_window_equals_truncated_history(use_slopes):
    """Decode over a long context with window W == plain decode over the last W tokens."""
    rng = np.random.default_rng(6 + use_slopes)
    H, d, W = 2, 16, 37
    lens = [5, 37, 38, 100, 257]
    hist = [history(rng, L, H, d) for L in lens]
    q = rng.standard_normal((len(lens), H, d))
    slopes = np.asarray([0.25, 0.0625]) if use_slopes else None
    kp, vp, bt = build_pool(hist, 8, sum(-(-L // 8) for L in lens) + 2, rng)
    win = oracle.paged_attention(q, kp, vp, bt, np.asarray(lens), 8, window=W,
                                 alibi_slopes=slopes)
    cut = [(K[-W:], V[-W:]) for K, V in hist]
    kp2, vp2, bt2 = build_pool(cut, 16, sum(-(-min(L, W) // 16) for L in lens) + 2,
                               np.random.default_rng(99))
    ref = oracle.paged_attention(q, kp2, vp2, bt2, np.asarray([min(L, W) for L in lens]), 16,
                                 alibi_slopes=slopes)
    assert rel_err(win, ref) < 1e-12


def test_large_slope_keeps_nearest_key():
    rng = np.random.default_rng(8)
    K, V = history(rng, 30, 2, 8)
    kp, vp, bt = build_pool([(K, V)], 4, 10, rng)
    q = rng.standard_normal((1, 2, 8))
    out = oracle.paged_attention(q, kp, vp, bt, np.asarray([30]), 4,
                                 alibi_slopes=np.asarray([200.0, 200.0]))
    assert max_abs(out[0], V[29]) < 1e-12


# ------------------------------------------------- the pins have teeth --

_attend = oatt.attend


def _mut_bias_sign(q, keys, values, positions, window=0, alibi_slopes=None):
    flipped = None if alibi_slopes is None else -np.asarray(alibi_slopes)
    return _attend(q, keys, values, positions, window, flipped)          # planted: sign


def _mut_window_off_by_one(q, keys, values, positions, window=0, alibi_slopes=None):
    return _attend(q, keys, values, positions, window + 1 if window else 0, alibi_slopes)


@pytest.mark.parametrize("mutant", [_mut_bias_sign, _mut_window_off_by_one])
def test_pins_catch_planted_mistake(monkeypatch, mutant):
    monkeypatch.setattr(oatt, "attend", mutant)
    caught = False
    for window, use_slopes in ((3, False), (7, True), (0, True)):
        try:
            test_brute_force(window, use_slopes)
        except AssertionError:
            caught = True
    assert caught
