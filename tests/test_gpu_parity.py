"""GPU parity: the HIP library through its C ABI vs the fp64 oracle.

Every case generates its inputs from workloads/ and copies the oracle's inputs
to the host before the library runs.  Attention outputs must satisfy
|gpu - ref| <= atol + rtol*|ref| (fp32: 1e-5 + 0; fp16: 2e-3 + 1e-2*|ref|);
slot writes and block copies must match bit for bit over the whole pool
(NaN-poisoned unfilled slots included).
"""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_40_amd import api
from workloads import make_config, make_small, make_custom_decode, make_custom_mixed
from cases import long_chunk_marked, long_decode_marked, ordered_lens
from paged_harness import (FULL_CHECK_POOL_BYTES, assert_bits_equal, assert_close,
                           every_sequence_check, host_copy, log, oracle_step, oracle_sub,
                           pick_sequences, pool_bytes, run_library, snapshot_for)
from sensitivity import drop_block_margins, drop_last_token_margin

pytestmark = pytest.mark.gpu


def full_check(w, seed_note=""):
    log(f"[case] {w.name} seed={w.seed} S={w.num_seqs} H={w.num_heads} d={w.head_dim} "
        f"B={w.block_size} {w.dtype} {seed_note}")
    t = w.device_tensors("cuda")
    h = host_copy(t)
    out = run_library(w, t)
    torch.cuda.synchronize()
    ref, kp, vp = oracle_step(w, h)
    err = assert_close(out.cpu().numpy(), ref, w.dtype, w.name)
    assert_bits_equal(t["k_pool"].cpu().numpy(), kp, "k_pool")
    assert_bits_equal(t["v_pool"].cpu().numpy(), vp, "v_pool")
    log(f"[ok] max abs err {err:.3g}")
    return out


# ------------------------------------------------------------- configs --

@pytest.mark.parametrize("seed", [1, 2, 3])
def test_config1_tiny_fp32(seed):
    full_check(make_config(1, seed=seed))


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
@pytest.mark.parametrize("seed", [1, 2])
def test_small_variants(idx, seed):
    full_check(make_small(idx, seed=seed))


@pytest.mark.parametrize("q_scale", [4.0])
def test_small_config2_peaked(q_scale):
    full_check(make_small(2, seed=5, q_scale=q_scale), f"q_scale={q_scale}")


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_full_size_every_sequence(idx):
    every_sequence_check(make_config(idx))


def test_full_size_large_batch_marked():
    """The large batch with block-marked values and small keys (workloads.configs: v_mark,
    k_scale): every sequence against the oracle, on inputs where any one dropped block of any
    sequence would exceed the tolerance (shown on these inputs by the test itself)."""
    every_sequence_check(make_config(5, k_scale=0.125, v_mark=2048.0), margins=True)


def test_longest_first_order_with_ties():
    """600 sequences x 8 heads with a 5000-token bound (12 GB of K/V by the bound, above the
    4 GB at which pass 1 takes the sequences longest first): every sequence against the
    oracle, bit-identical to the shared-blocks launch, which keeps the given order, and
    captured in a HIP graph, bit-identical on every replay."""
    w = make_custom_decode(91, "f16", 8, 128, 16, ordered_lens(91, 600, 5000), write_one=True,
                           name="ordered_ties")
    assert w.num_seqs * w.num_heads * w.max_context_len * 2 * 128 * 2 >= 4e9
    every_sequence_check(w)
    t1 = w.device_tensors("cuda")
    plain = run_library(w, t1)
    t2 = w.device_tensors("cuda")
    hinted = run_library(w, t2, shared=True)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), hinted.view(torch.int16))
    log("[ok] bit-identical to the launch in the given order")
    # the same call captured in a HIP graph: the order is recomputed on every replay (the
    # workspace is zeroed before each one, which would send every grid row of the partition
    # pass to sequence 0 if it were not)
    need = api.pa_decode_workspace_bytes(w.num_queries, w.num_heads, w.head_dim,
                                         w.max_context_len)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t1["q"])

    def call():
        api.pa_decode(out, t1["q"], t1["k_pool"], t1["v_pool"], t1["block_tables"],
                      t1["context_lens"], max_context_len=w.max_context_len, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16)), "eager call"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        ws.zero_()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), plain.view(torch.int16)), f"replay {i}"
    log("[ok] 3 graph replays bit-identical")


def test_longest_first_order_in_a_mixed_batch():
    """Chunks of several queries among 400 decodes (8 heads, a 5,000-token bound): the order
    ranks every sequence, the partition pass skips the chunks and the tile path takes them;
    every sequence against the oracle."""
    lens = ordered_lens(94, 400, 5000)
    w = make_custom_mixed(94, 8, 16, [(0, 300), (2000, 128), (4800, 200)], list(lens),
                          name="ordered_mixed")
    assert w.num_seqs <= w.num_queries
    assert w.num_seqs * w.num_heads * w.max_context_len * 2 * 128 * 2 >= 4e9
    every_sequence_check(w)


@pytest.mark.parametrize("S", [1024, 1025])
def test_longest_first_order_at_the_sequence_limit(S):
    """1,024 sequences (the most the order kernel ranks) and 1,025 (the given order) x 8 heads
    with a 1,000-token bound (4.2 GB by the bound): every sequence against the oracle, and
    bit-identical to the shared-blocks launch."""
    w = make_custom_decode(92, "f16", 8, 128, 16, ordered_lens(92, S, 1000), write_one=True,
                           name=f"ordered_{S}")
    assert w.num_seqs * w.num_heads * w.max_context_len * 2 * 128 * 2 >= 4e9
    every_sequence_check(w)
    t1 = w.device_tensors("cuda")
    plain = run_library(w, t1)
    t2 = w.device_tensors("cuda")
    hinted = run_library(w, t2, shared=True)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), hinted.view(torch.int16))
    log("[ok] bit-identical to the launch in the given order")


# ------------------------------------------------------- layouts, edges --

EDGE_LENS = [1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 255, 256, 257, 511, 512, 513, 1000, 2049]


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("block_size", [8, 16, 32])
def test_layouts_and_edge_lengths(dtype, head_dim, block_size):
    w = make_custom_decode(11, dtype, 3, head_dim, block_size, EDGE_LENS,
                           name=f"edges_{dtype}_d{head_dim}_B{block_size}")
    full_check(w)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_write_then_decode_layouts(dtype):
    w = make_custom_decode(12, dtype, 5, 128, 16, [1, 16, 17, 256, 257, 700], write_one=True,
                           name=f"write_{dtype}")
    full_check(w)


def test_single_token_returns_its_value_exactly():
    w = make_custom_decode(13, "f16", 4, 128, 16, [1, 1, 1], name="single_token")
    log("[case] single token")
    t = w.device_tensors("cuda")
    out = run_library(w, t)
    torch.cuda.synchronize()
    for s in range(3):
        blk = int(w.block_tables[s, 0])
        assert torch.equal(out[s].view(torch.int16), t["v_pool"][blk, 0].view(torch.int16))


def _pool_from_histories(kh, vh, tables, NB, B, dtype):
    H, D = kh[0].shape[1:]
    kp = torch.full((NB, B, H, D), float("nan"), dtype=dtype)
    vp = torch.full((NB, B, H, D), float("nan"), dtype=dtype)
    for s in range(len(kh)):
        L = kh[s].shape[0]
        for b in range(-(-L // B)):
            lo, hi = b * B, min(L, (b + 1) * B)
            kp[tables[s][b], :hi - lo] = kh[s][lo:hi]
            vp[tables[s][b], :hi - lo] = vh[s][lo:hi]
    return kp.cuda(), vp.cuda()


def _histories(lens, H, D, seed, dtype=torch.float16):
    g = torch.Generator().manual_seed(seed)
    kh = [torch.randn(L, H, D, generator=g).to(dtype) for L in lens]
    vh = [torch.randn(L, H, D, generator=g).to(dtype) for L in lens]
    q = torch.randn(len(lens), H, D, generator=g).to(dtype)
    return kh, vh, q


def _decode(q, kp, vp, tables, lens):
    bt = torch.tensor(tables, dtype=torch.int32).cuda()
    cl = torch.tensor(lens, dtype=torch.int32).cuda()
    out = torch.empty_like(q)
    api.pa_decode(out, q, kp, vp, bt, cl, max_context_len=max(lens))
    torch.cuda.synchronize()
    return out


def _tables(rng, lens, B, NB, width=None):
    perm = rng.permutation(NB)
    need = [-(-L // B) for L in lens]
    width = width or max(need) + 1
    out, pos = [], 0
    for n in need:
        out.append(list(perm[pos:pos + n]) + [-1] * (width - n))
        pos += n
    return out


def test_block_permutation_bit_identical():
    """Same logical K/V under different physical placements: identical bits out
    (the reduction order depends only on token positions)."""
    log("[case] block permutation")
    lens, B, H, D = [1, 100, 257, 1500, 3000], 16, 4, 128
    kh, vh, q = _histories(lens, H, D, seed=21)
    q = q.cuda()
    NB = sum(-(-L // B) for L in lens) + 20
    outs = []
    for trial in range(3):
        tab = _tables(np.random.default_rng(trial), lens, B, NB)
        kp, vp = _pool_from_histories(kh, vh, tab, NB, B, torch.float16)
        outs.append(_decode(q, kp, vp, tab, lens))
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


def test_decode_token_permutation_invariant():
    """Decode attention is a sum over the context's tokens, so permuting a sequence's
    (k, v) rows jointly leaves it unchanged up to rounding: the GPU output of every
    permuted context stays within the fp16 tolerance of the unpermuted one, and both
    equal the oracle over their own token order.  Unlike a block permutation this
    changes the order of the kernel's sums (partitions, lanes, merges)."""
    log("[case] token permutation")
    lens, B, H, D = [2, 33, 257, 1500, 4100], 16, 4, 128
    kh, vh, q = _histories(lens, H, D, seed=23)
    NB = sum(-(-L // B) for L in lens) + 20
    tab = _tables(np.random.default_rng(3), lens, B, NB)
    qd = q.cuda()
    base = _decode(qd, *_pool_from_histories(kh, vh, tab, NB, B, torch.float16), tab, lens)
    for s, L in enumerate(lens):
        ref = oracle.attend(q[s:s + 1].numpy(), kh[s].numpy(), vh[s].numpy(), [L - 1])
        assert_close(base[s:s + 1].cpu().numpy(), ref, "f16", f"seq {s} unpermuted vs oracle")
    rng = np.random.default_rng(4)
    for trial in range(2):
        perms = [torch.from_numpy(rng.permutation(L)) for L in lens]
        khp = [k[p] for k, p in zip(kh, perms)]
        vhp = [v[p] for v, p in zip(vh, perms)]
        out = _decode(qd, *_pool_from_histories(khp, vhp, tab, NB, B, torch.float16), tab, lens)
        # each run is within the fp16 tolerance of the exact value, so within twice of each other
        o, b = out.cpu().numpy().astype(np.float64), base.cpu().numpy().astype(np.float64)
        assert (np.abs(o - b) <= 2 * (2e-3 + 1e-2 * np.abs(b))).all(), f"trial {trial}"
        for s, L in enumerate(lens):
            ref = oracle.attend(q[s:s + 1].numpy(), khp[s].numpy(), vhp[s].numpy(), [L - 1])
            assert_close(out[s:s + 1].cpu().numpy(), ref, "f16", f"seq {s} vs oracle")
    log("[ok]")


def _chunk_call(q, kp, vp, tables, lens, qlens):
    """pa_decode over sequences with qlens[s] query rows each (chunks and decodes)."""
    bt = torch.tensor(tables, dtype=torch.int32).cuda()
    cl = torch.tensor(lens, dtype=torch.int32).cuda()
    loc = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32).cuda()
    out = torch.empty_like(q)
    api.pa_decode(out, q, kp, vp, bt, cl, loc, max_context_len=max(lens),
                  max_query_len=max(qlens))
    torch.cuda.synchronize()
    return out


def test_closed_forms():
    """Results fixed by the attention formula alone, checked without the oracle: with every
    key of a sequence equal, the weights are uniform, so a decode returns the mean of its
    context's values and chunk query i the mean of values 0..p_i (prefix means); with every
    value equal to c the output is c.  Decodes of 1 to 5,000 tokens (up to three merged
    partitions) and chunks over 0 and 700 prior tokens, split into several workgroups."""
    log("[case] closed forms")
    B, H, D = 16, 2, 128
    g = torch.Generator().manual_seed(31)
    lens = [1, 100, 2049, 5000, 302, 1000]
    qlens = [1, 1, 1, 1, 300, 300]          # two chunks: priors 2 and 700
    NB = sum(-(-L // B) for L in lens) + 10
    tab = _tables(np.random.default_rng(5), lens, B, NB)
    krow = torch.randn(1, H, D, generator=g).half()
    kh = [krow.expand(L, H, D).clone() for L in lens]
    vh = [torch.randn(L, H, D, generator=g).half() for L in lens]
    q = torch.randn(sum(qlens), H, D, generator=g).half()
    out = _chunk_call(q.cuda(), *_pool_from_histories(kh, vh, tab, NB, B, torch.float16), tab,
                      lens, qlens).cpu().numpy().astype(np.float64)
    row = 0
    for s, (L, n) in enumerate(zip(lens, qlens)):
        v = vh[s].numpy().astype(np.float64)
        prefix_mean = np.cumsum(v, axis=0) / np.arange(1, L + 1)[:, None, None]
        want = prefix_mean[L - n:L]           # query i at position L-n+i
        got = out[row:row + n]
        assert np.abs(got - want).max() <= 2e-3 + 1e-2 * np.abs(want).max(), f"seq {s}"
        row += n
    # every value row equal to c: output c (for any keys)
    c = torch.randn(1, H, D, generator=g).half()
    kh = [torch.randn(L, H, D, generator=g).half() for L in lens]
    vh = [c.expand(L, H, D).clone() for L in lens]
    out = _chunk_call(q.cuda(), *_pool_from_histories(kh, vh, tab, NB, B, torch.float16), tab,
                      lens, qlens).cpu().numpy().astype(np.float64)
    want = np.broadcast_to(c.numpy().astype(np.float64), out.shape)
    assert np.abs(out - want).max() <= 2e-3 + 1e-2 * np.abs(want).max()
    log("[ok]")


def test_block_size_change_within_tolerance():
    """The same logical K/V laid out in blocks of 8, 16 and 32 tokens gives the same attention
    (each layout within the fp16 tolerance of the oracle, and of each other within twice it:
    the partition and load structure differ with the block size, so bits may too)."""
    log("[case] block size change")
    lens, H, D = [1, 31, 250, 2049, 4500], 4, 128
    kh, vh, q = _histories(lens, H, D, seed=27)
    qd = q.cuda()
    outs = []
    for B in (8, 16, 32):
        NB = sum(-(-L // B) for L in lens) + 10
        tab = _tables(np.random.default_rng(B), lens, B, NB)
        outs.append(_decode(qd, *_pool_from_histories(kh, vh, tab, NB, B, torch.float16), tab,
                            lens).cpu().numpy().astype(np.float64))
    for s, L in enumerate(lens):
        ref = oracle.attend(q[s:s + 1].numpy(), kh[s].numpy(), vh[s].numpy(), [L - 1])
        for o in outs:
            assert_close(o[s:s + 1], ref, "f16", f"seq {s}")
    for o in outs[1:]:
        assert (np.abs(o - outs[0]) <= 2 * (2e-3 + 1e-2 * np.abs(outs[0]))).all()
    log("[ok]")


def test_shared_prefix_bit_identical():
    """Prefix blocks shared by every sequence vs a private copy per sequence."""
    log("[case] shared vs duplicated prefix")
    B, H, D = 16, 4, 128
    g = torch.Generator().manual_seed(5)
    prefix_k = torch.randn(48, H, D, generator=g).half()
    prefix_v = torch.randn(48, H, D, generator=g).half()
    tails = [7, 16, 40, 300]
    kh = [torch.cat([prefix_k, torch.randn(n, H, D, generator=g).half()]) for n in tails]
    vh = [torch.cat([prefix_v, torch.randn(n, H, D, generator=g).half()]) for n in tails]
    lens = [k.shape[0] for k in kh]
    q = torch.randn(len(lens), H, D, generator=g).half().cuda()
    NB = 200
    dup = _tables(np.random.default_rng(1), lens, B, NB)
    out_dup = _decode(q, *_pool_from_histories(kh, vh, dup, NB, B, torch.float16), dup, lens)
    shared = [list(r) for r in dup]
    for r in shared[1:]:
        r[:3] = shared[0][:3]
    out_sh = _decode(q, *_pool_from_histories(kh, vh, shared, NB, B, torch.float16), shared, lens)
    assert torch.equal(out_sh.view(torch.int16), out_dup.view(torch.int16))


def test_copy_blocks_bit_exact_random_pairs():
    log("[case] copy blocks")
    import oracle
    rng = np.random.default_rng(3)
    for dtype, B, H, D in ((torch.float16, 16, 40, 128), (torch.float32, 32, 3, 64)):
        NB = 300
        kp = torch.randn(NB, B, H, D, dtype=torch.float32).to(dtype).cuda()
        vp = torch.randn(NB, B, H, D, dtype=torch.float32).to(dtype).cuda()
        kp[5, 3:] = float("nan")
        perm = rng.permutation(NB)
        pairs = np.stack([perm[:60], perm[60:120]], 1).astype(np.int32)
        pairs[0, 0] = 5
        hk, hv = kp.cpu().numpy(), vp.cpu().numpy()
        api.pa_copy_blocks(kp, vp, torch.from_numpy(pairs).cuda())
        torch.cuda.synchronize()
        ek, ev = oracle.copy_blocks(hk, hv, pairs)
        assert_bits_equal(kp.cpu().numpy(), ek, "k copy")
        assert_bits_equal(vp.cpu().numpy(), ev, "v copy")


def test_side_stream_and_reused_workspace():
    """Calls on a non-default stream with a caller-owned workspace reused across calls."""
    log("[case] side stream")
    w = make_small(5, seed=3)
    t = w.device_tensors("cuda")
    h = host_copy(t)
    need = api.pa_decode_workspace_bytes(w.num_queries, w.num_heads, w.head_dim,
                                         w.max_context_len)
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = run_library(w, t, stream=s, workspace=ws)
        out2 = torch.empty_like(out)
        api.pa_decode(out2, t["q"], t["k_pool"], t["v_pool"], t["block_tables"],
                      t["context_lens"], max_context_len=w.max_context_len, workspace=ws,
                      stream=s)
    s.synchronize()
    ref, _, _ = oracle_step(w, h)
    assert_close(out.cpu().numpy(), ref, w.dtype, "side stream")
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_graph_capture_replays():
    """A whole step (slot writes + mixed chunk/decode attention) captured in a HIP graph and
    replayed several times, with unrelated eager work and synchronisation between replays:
    every replay equals the eager step bit for bit, and the step equals the oracle.  The
    library only enqueues kernels (no allocation, no memset), so the step is capturable."""
    w = make_small(4, seed=1)
    log(f"[case] graph capture {w.name}")
    t = w.device_tensors("cuda")
    h = host_copy(t)
    need = api.pa_decode_workspace_bytes(w.num_queries, w.num_heads, w.head_dim,
                                         w.max_context_len)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])

    def step():
        api.pa_write_kv(t["k_pool"], t["v_pool"], t["k_new"], t["v_new"], t["block_tables"],
                        t["context_lens"], t["write_start_loc"])
        api.pa_decode_ext(out, t["q"], t["k_pool"], t["v_pool"], t["block_tables"],
                          t["context_lens"], t["q_start_loc"], max_context_len=w.max_context_len,
                          max_query_len=w.max_query_len, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                   # eager, on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.clone()
    ref, _, _ = oracle_step(w, h)
    assert_close(eager.cpu().numpy(), ref, w.dtype, "eager step")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    scratch = torch.randn(1 << 20, device="cuda")
    for i in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        scratch.mul_(0.5).add_(1.0)              # unrelated eager work between replays
        torch.cuda.synchronize()
    log("[ok] 4 replays bit-identical")


# Batch shapes that make the launch pick each context-partition size (the largest of
# 2048/1024/512/256 tokens that still gives >= 16384 waves), checked on every sequence when
# the pools fit the host-side oracle comfortably, else on sampled sequences.
@pytest.mark.parametrize("S,H,lo,hi,B,expect_p", [
    (64, 40, 3000, 4096, 16, 256),
    (128, 32, 2049, 4096, 16, 512),
    (128, 32, 3073, 4096, 32, 1024),
    (256, 40, 4097, 6000, 16, 2048),
    (192, 40, 2049, 4096, 8, 1024),
])
def test_partition_sizes(S, H, lo, hi, B, expect_p):
    rng = np.random.default_rng(S + H + B)
    lens = rng.integers(lo, hi + 1, size=S)
    lens[0], lens[-1] = lo, hi
    w = make_custom_decode(17, "f16", H, 128, B, lens, write_one=True,
                           name=f"partition_{expect_p}_B{B}")
    log(f"[case] {w.name} S={S} H={H} L=[{lo},{hi}] NB={w.num_blocks}")
    if pool_bytes(w) <= FULL_CHECK_POOL_BYTES:
        every_sequence_check(w)
        return
    t = w.device_tensors("cuda")
    seqs = pick_sequences(w, n=3, seed=S)
    sub = snapshot_for(w, t, seqs)
    out = run_library(w, t)
    torch.cuda.synchronize()
    refs, kp, _ = oracle_sub(w, sub)
    for i, s in enumerate(seqs):
        assert_close(out[s:s + 1].cpu().numpy(), refs[i], w.dtype, f"{w.name} seq {s}")
    idx_t = torch.tensor(sub["uniq"], dtype=torch.int64, device="cuda")
    assert_bits_equal(t["k_pool"].index_select(0, idx_t).cpu().numpy(), kp, "k_pool sampled")


# ------------------------------------------------ multi-query tile path --

@pytest.mark.parametrize("B", [8, 16, 32])
def test_chunk_tiles_edges(B):
    """Chunks of 2..130 queries (one short of, at and past the 64-query tile), with no prior
    context, a one-token prior and long priors, mixed with decodes in the same call."""
    chunks = [(0, 2), (0, 64), (1, 63), (17, 65), (300, 130), (1000, 16), (15, 33)]
    w = make_custom_mixed(30 + B, 4, B, chunks, [1, 16, 300, 1025], name=f"chunks_B{B}")
    full_check(w)


@pytest.mark.parametrize("B", [8, 16, 32])
def test_chunk_tiles_multi_tile(B):
    """Chunks spanning three to four 128-query tiles, with priors that end mid-block and
    mid-step, so the staged steps cross blocks at every offset and the last step of a tile
    holds the context's end."""
    chunks = [(37, 300), (1000, 257), (5, 511), (96, 384)]
    w = make_custom_mixed(50 + B, 2, B, chunks, [7, 129], name=f"chunks_multi_B{B}")
    full_check(w)


@pytest.mark.parametrize("B", [8, 16, 32])
def test_chunk_tiles_head_dim_64(B):
    """The tile path at head_dim 64: chunks of 2..511 queries over short and long priors
    (one to four 128-query tiles, contexts ending mid-block), mixed with decodes."""
    chunks = [(0, 2), (17, 65), (300, 130), (1000, 257), (5, 511), (40, 384)]
    w = make_custom_mixed(90 + B, 3, B, chunks, [1, 300, 1025], name=f"chunks_d64_B{B}",
                          head_dim=64)
    full_check(w)


@pytest.mark.parametrize("head_dim,B", [(128, 16), (64, 8), (128, 32)])
def test_chunk_key_splits(head_dim, B):
    """Few tile workgroups (2 heads, a handful of chunks), so the launch splits long tiles'
    keys over several workgroups and merges their partials: priors from 0 to 9,000 keys (one
    to ~18 splits, the last split shorter or a single step), chunks of 2..300 queries whose
    diagonal falls inside or across splits, next to decodes."""
    chunks = [(0, 2), (511, 2), (600, 40), (3000, 128), (9000, 129), (1537, 300)]
    w = make_custom_mixed(60 + B + head_dim, 2, B, chunks, [1, 2500, 9001],
                          name=f"chunk_splits_d{head_dim}_B{B}", head_dim=head_dim)
    full_check(w)


def test_chunk_tiles_peaked_scores():
    w = make_custom_mixed(41, 3, 16, [(200, 100), (0, 70)], [50], name="chunks_peaked",
                          q_scale=4.0)
    full_check(w, "q_scale=4")


def test_long_contexts():
    """Long contexts: a 100,000-token decode (about fifty 2048-token partitions merged), a
    65,537-token one (a one-token last partition) and a 300-query chunk over a 30,000-token
    prior, next to short ones, against the oracle over every head."""
    w = make_custom_decode(81, "f16", 4, 128, 16, [100000, 65537, 3, 700], write_one=True,
                           name="long_decode")
    full_check(w)
    w = make_custom_mixed(82, 2, 16, [(30000, 300), (5, 40)], [20000, 9], name="long_chunk")
    full_check(w)


def _sharpness(w, t_host_after, s, query_rows):
    """Smallest drop-one-block margin over the whole blocks each of sequence s's queries sees
    (and the appended token's margin for the last query), on the post-step host pools."""
    import oracle
    B = w.block_size
    L = int(w.context_lens[s])
    kp, vp = t_host_after
    keys = oracle.gather_context(kp, w.block_tables[s], L, B)
    vals = oracle.gather_context(vp, w.block_tables[s], L, B)
    n = len(query_rows)
    low = np.inf
    for i, qrow in enumerate(query_rows):
        p = L - n + i
        m = drop_block_margins(qrow, keys[:p + 1], vals[:p + 1], B, 2e-3, 1e-2)
        low = min(low, (m if n == 1 else m[:(p + 1) // B]).min())
    last = drop_last_token_margin(query_rows[-1], keys, vals, 2e-3, 1e-2)
    return low, last


def test_long_contexts_marked():
    """The long contexts on block-marked inputs (tests/cases.py): any one dropped block, the
    one-token last partition of the 65,537-token decode, or a misordered partition merge
    would break the tolerance - shown here on these very inputs before comparing."""
    for w in (long_decode_marked(), long_chunk_marked()):
        log(f"[case] {w.name}")
        t = w.device_tensors("cuda")
        h = host_copy(t)
        out = run_library(w, t)
        torch.cuda.synchronize()
        ref, kp, vp = oracle_step(w, h)
        assert_close(out.cpu().numpy(), ref, w.dtype, w.name)
        assert_bits_equal(t["k_pool"].cpu().numpy(), kp, "k_pool")
        assert_bits_equal(t["v_pool"].cpu().numpy(), vp, "v_pool")
        qsl = w.q_start_loc()
        for s in np.flatnonzero(w.context_lens >= 20000):
            a, b = (s, s + 1) if qsl is None else (int(qsl[s]), int(qsl[s + 1]))
            rows = h["q"][a:b].astype(np.float64)
            if b - a > 1:
                low, last = _sharpness(w, (kp, vp), s, rows)   # every query of the chunk
            else:
                low, last = _sharpness(w, (kp, vp), s, rows)
            log(f"[sharp] seq {s} L={int(w.context_lens[s])}: block margin {low:.1f}, "
                f"last token {last:.1f}")
            assert low >= 3.0 and (b - a > 1 or last >= 3.0)
        log("[ok]")


def test_chunk_only_batch():
    """Every sequence is a chunk (no decode units); the tile kernel alone writes the output."""
    w = make_custom_mixed(42, 2, 16, [(64, 64), (5, 128), (0, 256)], [], name="chunks_only")
    full_check(w)


@pytest.mark.parametrize("head_dim,B", [(128, 16), (128, 8), (64, 32), (64, 16)])
def test_mixed_batch_32_heads(head_dim, B):
    """Mixed batches large enough that the tile launch needs no key splits (32 heads, >= 2,000
    chunk rows): chunks over priors of 0..1,000 tokens ending mid-block, decodes of 1..3,000
    tokens; every sequence against the oracle."""
    chunks = [(0, 512), (300, 512), (1000, 520), (37, 600)]
    decodes = [1, 17, 256, 257, 1500, 2049, 3000]
    w = make_custom_mixed(70 + B + head_dim, 32, B, chunks, decodes,
                          name=f"mixed_32h_d{head_dim}_B{B}", head_dim=head_dim)
    every_sequence_check(w)
