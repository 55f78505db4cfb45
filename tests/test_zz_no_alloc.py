"""pa_decode_noalloc (the workspace in the library's own device array) through the C ABI
against pa_decode_ext with a caller workspace: the same kernels, so the same bits, on two
calls in a row - the second with a smaller batch - on a batch that also takes the
chunked-prefill tile path's key splits, and on one whose partition pass takes the sequences
longest first.  The first call is also checked against the oracle."""

import numpy as np
import pytest
import torch

from paged_harness import assert_close, host_copy, log, oracle_step
from paged_kv_cache_40_amd import _lib, api
from workloads import make_custom_decode, make_custom_mixed

pytestmark = pytest.mark.gpu


def _ext_and_noalloc(w, t, **kw):
    out_n = torch.full_like(t["q"], float("nan"))
    api.pa_decode_noalloc(out_n, t["q"], t["k_pool"], t["v_pool"], t["block_tables"],
                          t["context_lens"], t["q_start_loc"], max_context_len=w.max_context_len,
                          max_query_len=w.max_query_len, **kw)
    out_e = torch.full_like(t["q"], float("nan"))
    need = api.pa_decode_workspace_bytes(w.num_queries, w.num_heads, w.head_dim,
                                         w.max_context_len)
    ws = torch.full((max(need, 1),), 255, dtype=torch.uint8, device="cuda")
    api.pa_decode_ext(out_e, t["q"], t["k_pool"], t["v_pool"], t["block_tables"],
                      t["context_lens"], t["q_start_loc"], max_context_len=w.max_context_len,
                      max_query_len=w.max_query_len, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert need > 0, "the batch must use the workspace"
    return out_n, out_e


def _same_bits(a, b):
    itype = torch.int16 if a.dtype == torch.float16 else torch.int32
    return torch.equal(a.view(itype), b.view(itype))


def test_noalloc_equals_workspace_call_twice_then_smaller():
    first = make_custom_decode(91, "f16", 8, 128, 16, [9000, 1, 257, 4097, 2049, 700],
                               name="noalloc_first")
    second = make_custom_decode(92, "f32", 3, 64, 8, [600, 33, 2100], name="noalloc_second")
    for i, w in enumerate((first, second)):
        log(f"[case] call {i + 1}: {w.name} S={w.num_seqs} H={w.num_heads} {w.dtype}")
        t = w.device_tensors("cuda")
        h = host_copy(t)
        out_n, out_e = _ext_and_noalloc(w, t)
        assert _same_bits(out_n, out_e), f"call {i + 1}"
        ref, _, _ = oracle_step(w, h)
        assert_close(out_n.cpu().numpy(), ref, w.dtype, w.name)
    log("[ok]")


def test_noalloc_chunks_with_key_splits_and_variants():
    """A mixed batch whose few tile workgroups split their keys (partials in the array), then
    the grouped decode and a window with ALiBi slopes, each equal to the workspace call."""
    w = make_custom_mixed(93, 2, 16, [(3000, 128), (9000, 129), (0, 2)], [1, 2500],
                          name="noalloc_chunks")
    log(f"[case] {w.name}")
    t = w.device_tensors("cuda")
    out_n, out_e = _ext_and_noalloc(w, t)
    assert _same_bits(out_n, out_e)
    slopes = torch.tensor([0.25, 0.0625], dtype=torch.float32, device="cuda")
    out_n, out_e = _ext_and_noalloc(w, t, sliding_window=700, alibi_slopes=slopes)
    assert _same_bits(out_n, out_e)
    g = make_custom_decode(94, "f16", 4, 128, 16, [3000, 2990, 2500, 1800], name="noalloc_group")
    tg = g.device_tensors("cuda")
    out_n, out_e = _ext_and_noalloc(g, tg, group=2)
    assert _same_bits(out_n, out_e)
    log("[ok]")


def test_noalloc_longest_first_batch():
    """A batch large enough by its bound (600 sequences x 8 heads, 5,000-token bound) for the
    partition pass to take the sequences longest first: the order lives in the array too."""
    from cases import ordered_lens
    w = make_custom_decode(96, "f16", 8, 128, 16, ordered_lens(96, 600, 5000),
                           name="noalloc_ordered")
    assert w.num_seqs * w.num_heads * w.max_context_len * 2 * 128 * 2 >= 4e9
    log(f"[case] {w.name}")
    t = w.device_tensors("cuda")
    out_n, out_e = _ext_and_noalloc(w, t)
    assert _same_bits(out_n, out_e)
    log("[ok]")


def test_noalloc_rejects_a_batch_beyond_the_array():
    w = make_custom_decode(95, "f16", 40, 128, 16, [1, 2], name="noalloc_small")
    t = w.device_tensors("cuda")
    S, big = 256, 16384
    need = api.pa_decode_workspace_bytes(S, 40, 128, big)
    assert need > _lib.PA_NOALLOC_WORKSPACE_BYTES
    q = torch.zeros((S, 40, 128), dtype=torch.float16, device="cuda")
    bt = torch.zeros((S, big // 16), dtype=torch.int32, device="cuda")
    cl = torch.ones(S, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="workspace"):
        api.pa_decode_noalloc(torch.empty_like(q), q, t["k_pool"], t["v_pool"], bt, cl,
                              max_context_len=big)
