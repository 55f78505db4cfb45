"""GPU parity of the sliding-window and ALiBi variants (pa_decode_ext) vs the fp64 oracle.

Readings under test (oracle/attention.py): with window W the query at position
p attends to tokens p-W+1 .. p; ALiBi adds slope_h * (j - p) to the score of
token j.  Slopes are the geometric sequence 2^(-8(h+1)/H) of the ALiBi paper;
the pages name the method without values, and any positive slopes take the
same code path.  Tolerances as in the plain tests (paged_harness.TOL).
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_40_amd import api
from workloads import make_config, make_custom_decode, make_custom_mixed
from paged_harness import (FULL_CHECK_POOL_BYTES, assert_bits_equal, assert_close,
                           every_sequence_check, host_copy, log, oracle_step, oracle_sub,
                           pick_sequences, pool_bytes, run_library, snapshot_for)

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 255, 256, 257, 511, 512, 513, 1000, 2049]


def geometric_slopes(H):
    return (2.0 ** (-8.0 * (np.arange(H) + 1) / H)).astype(np.float32)


def variant_check(w, window, alibi, note=""):
    log(f"[case] {w.name} W={window} alibi={alibi is not None} S={w.num_seqs} "
        f"H={w.num_heads} d={w.head_dim} B={w.block_size} {w.dtype} {note}")
    t = w.device_tensors("cuda")
    h = host_copy(t)
    out = run_library(w, t, window=window, alibi=alibi)
    torch.cuda.synchronize()
    ref, kp, vp = oracle_step(w, h, window=window, alibi=alibi)
    err = assert_close(out.cpu().numpy(), ref, w.dtype, f"{w.name} W={window}")
    assert_bits_equal(t["k_pool"].cpu().numpy(), kp, "k_pool")
    assert_bits_equal(t["v_pool"].cpu().numpy(), vp, "v_pool")
    log(f"[ok] max abs err {err:.3g}")


CASES = [(W, al) for W in (0, 1, 7, 16, 100, 300, 5000) for al in (False, True)
         if W or al]


@pytest.mark.parametrize("dtype,head_dim,block_size",
                         [("f16", 128, 16), ("f32", 64, 8), ("f16", 64, 32), ("f32", 128, 32)])
@pytest.mark.parametrize("window,use_alibi", CASES)
def test_window_alibi_edge_lengths(dtype, head_dim, block_size, window, use_alibi):
    """Windows shorter than a block, equal to one, spanning partitions and longer than every
    context, with and without ALiBi, over context lengths at block and partition edges; the
    step also appends one token per sequence."""
    w = make_custom_decode(50 + block_size, dtype, 3, head_dim, block_size, EDGE_LENS,
                           write_one=True, name=f"variant_{dtype}_d{head_dim}_B{block_size}")
    variant_check(w, window, geometric_slopes(3) if use_alibi else None)


def test_large_slopes_peaked():
    """Slopes large enough that only the newest few tokens carry weight."""
    w = make_custom_decode(61, "f16", 4, 128, 16, [3, 40, 600, 3000], name="alibi_steep")
    variant_check(w, 0, np.asarray([8.0, 2.0, 0.5, 0.125], np.float32))


def test_history_before_window_is_never_used():
    """Every slot older than the window holds NaN and the table entries of blocks wholly
    before the window are -1 (a sliding-window cache would have released them): the output
    must stay finite and equal the oracle's, which reads only the window."""
    H, D, B, W = 4, 128, 16, 100
    lens = [1, 50, 100, 101, 117, 300, 1000, 2500]
    w = make_custom_decode(62, "f16", H, D, B, lens, name="window_poisoned_history")
    log(f"[case] {w.name} W={W}")
    t = w.device_tensors("cuda")
    bt = t["block_tables"].cpu().numpy()
    blks, slots = [], []
    for s, L in enumerate(lens):
        lo = max(0, L - W)
        j = np.arange(lo)
        blks.append(bt[s, j // B])
        slots.append(j % B)
        bt[s, :lo // B] = -1
    blks = torch.from_numpy(np.concatenate(blks).astype(np.int64)).cuda()
    slots = torch.from_numpy(np.concatenate(slots).astype(np.int64)).cuda()
    t["k_pool"][blks, slots] = float("nan")
    t["v_pool"][blks, slots] = float("nan")
    t["block_tables"] = torch.from_numpy(bt).cuda()
    h = host_copy(t)
    slopes = geometric_slopes(H)
    out = run_library(w, t, window=W, alibi=slopes)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    ref, _, _ = oracle_step(w, h, window=W, alibi=slopes)
    assert_close(out.cpu().numpy(), ref, "f16", "poisoned history")
    log("[ok]")


def test_neutral_variants_bit_identical_to_plain():
    """A window at least as long as every context, and all-zero slopes, reproduce pa_decode's
    output bit for bit (same partitions, and adding 0 * (j - p) is exact)."""
    w = make_custom_decode(63, "f16", 8, 128, 16, [1, 17, 300, 2049, 4000, 6000], name="neutral")
    log(f"[case] {w.name}")
    t = w.device_tensors("cuda")
    plain = run_library(w, t)
    wide = run_library(w, t, window=int(w.context_lens.max()))
    zero = run_library(w, t, alibi=np.zeros(8, np.float32))
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), wide.view(torch.int16))
    assert torch.equal(plain.view(torch.int16), zero.view(torch.int16))
    log("[ok]")


# Windows long enough to span several context partitions of each size the launch picks; every
# sequence when the pools fit the host-side oracle comfortably, else sampled sequences.
@pytest.mark.parametrize("S,H,lo,hi,W", [
    (64, 40, 3000, 9000, 2500),    # 256-token partitions inside the window
    (256, 40, 1025, 4097, 4000),   # 2048-token partitions; short contexts end before W
    (256, 40, 1025, 4097, 1024),   # 1024-token partitions
])
def test_window_partitions(S, H, lo, hi, W):
    rng = np.random.default_rng(S + W)
    lens = rng.integers(lo, hi + 1, size=S)
    lens[0], lens[-1] = lo, hi
    w = make_custom_decode(64, "f16", H, 128, 16, lens, write_one=True,
                           name=f"window_{W}_S{S}")
    slopes = geometric_slopes(H)
    log(f"[case] {w.name} L=[{lo},{hi}] W={W} NB={w.num_blocks}")
    if pool_bytes(w) <= FULL_CHECK_POOL_BYTES:
        every_sequence_check(w, window=W, alibi=slopes)
        return
    t = w.device_tensors("cuda")
    seqs = pick_sequences(w, n=3, seed=S)
    sub = snapshot_for(w, t, seqs)
    out = run_library(w, t, window=W, alibi=slopes)
    torch.cuda.synchronize()
    refs, kp, _ = oracle_sub(w, sub, window=W, alibi=slopes)
    for i, s in enumerate(seqs):
        assert_close(out[s:s + 1].cpu().numpy(), refs[i], w.dtype, f"{w.name} seq {s}")
    idx_t = torch.tensor(sub["uniq"], dtype=torch.int64, device="cuda")
    assert_bits_equal(t["k_pool"].index_select(0, idx_t).cpu().numpy(), kp, "k_pool sampled")
    log("[ok]")


def test_full_size_large_batch_window_alibi_every_sequence():
    """The 256-sequence, 40-head large-batch decode (contexts 1025..4097) with a 1024-token
    window and ALiBi, as the benchmark's variant line runs it: every sequence and head
    against the oracle (in a pool of host processes), the pools bit for bit."""
    w = make_config(5)
    every_sequence_check(w, window=1024, alibi=geometric_slopes(w.num_heads))


# ------------------------------------------- chunked prefill (multi-query tile path) --

CHUNKS = [(0, 2), (0, 64), (17, 65), (300, 130), (1000, 257), (5, 33), (40, 384)]
CHUNK_CASES = [(1, False), (7, True), (32, False), (33, True), (100, True), (200, False),
               (5000, True), (0, True)]


@pytest.mark.parametrize("block_size", [8, 16, 32])
@pytest.mark.parametrize("window,use_alibi", CHUNK_CASES)
def test_chunk_window_alibi(block_size, window, use_alibi):
    """Chunks of 2..384 queries with short and long priors, mixed with decodes, under windows
    shorter than one step, at and past a step, shorter and longer than the chunks, and wider
    than every context; ALiBi alone and with a window."""
    w = make_custom_mixed(70 + block_size, 3, block_size, CHUNKS, [1, 16, 300, 1025],
                          name=f"chunks_W{window}_B{block_size}")
    variant_check(w, window, geometric_slopes(3) if use_alibi else None)


@pytest.mark.parametrize("window,use_alibi", [(7, True), (100, False), (0, True)])
def test_chunk_window_alibi_head_dim_64(window, use_alibi):
    w = make_custom_mixed(78, 3, 16, CHUNKS, [1, 300], name=f"chunks_d64_W{window}",
                          head_dim=64)
    variant_check(w, window, geometric_slopes(3) if use_alibi else None)


@pytest.mark.parametrize("window,use_alibi", [(700, False), (700, True), (2000, True),
                                              (0, True)])
def test_chunk_window_alibi_key_splits(window, use_alibi):
    """Long priors with 2 heads, so tiles are split over several workgroups: splits that
    start at the window's first step, windows spanning two to four splits, and ALiBi biases
    carried through the partial merge."""
    chunks = [(3000, 129), (6000, 40), (900, 300), (0, 70)]
    w = make_custom_mixed(79, 2, 16, chunks, [1, 4000], name=f"chunk_splits_W{window}")
    variant_check(w, window, geometric_slopes(2) if use_alibi else None)


def test_chunk_history_before_window_is_never_used():
    """Chunks whose keys older than the first query's window hold NaN, with the table entries
    of blocks wholly before it set to -1 (poisoned before any library call; this step's rows,
    written by each call, all lie inside the window): the tile path must not use them."""
    H, B, W = 3, 16, 70
    chunks = [(0, 100), (37, 40), (500, 200), (1000, 300)]
    w = make_custom_mixed(75, H, B, chunks, [900], name="chunks_window_poisoned")
    log(f"[case] {w.name} W={W}")
    t = w.device_tensors("cuda")
    bt = t["block_tables"].cpu().numpy()
    qsl = w.q_start_loc()
    blks, slots = [], []
    for s, L in enumerate(w.context_lens):
        n = int(qsl[s + 1] - qsl[s])
        lo = max(0, int(L) - n - W + 1)       # the first query's window start
        j = np.arange(lo)
        blks.append(bt[s, j // B])
        slots.append(j % B)
        bt[s, :lo // B] = -1
    blks = torch.from_numpy(np.concatenate(blks).astype(np.int64)).cuda()
    slots = torch.from_numpy(np.concatenate(slots).astype(np.int64)).cuda()
    t["k_pool"][blks, slots] = float("nan")
    t["v_pool"][blks, slots] = float("nan")
    t["block_tables"] = torch.from_numpy(bt).cuda()
    h = host_copy(t)
    slopes = geometric_slopes(H)
    for al in (None, slopes):
        out = run_library(w, t, window=W, alibi=al)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        ref, _, _ = oracle_step(w, h, window=W, alibi=al)
        assert_close(out.cpu().numpy(), ref, "f16", f"poisoned chunk history alibi={al is not None}")
    log("[ok]")


def test_chunk_neutral_variants_bit_identical_to_plain():
    """On the tile path too, a window at least as long as every context and all-zero slopes
    reproduce pa_decode bit for bit."""
    w = make_custom_mixed(76, 4, 16, [(0, 130), (700, 257), (33, 64)], [5, 600], name="chunk_neutral")
    t = w.device_tensors("cuda")
    plain = run_library(w, t)                 # each call rewrites the same slots first
    wide = run_library(w, t, window=int(w.context_lens.max()))
    zero = run_library(w, t, alibi=np.zeros(4, np.float32))
    torch.cuda.synchronize()
    p16 = plain.view(torch.int16)
    assert torch.equal(wide.view(torch.int16), p16)
    assert torch.equal(zero.view(torch.int16), p16)
