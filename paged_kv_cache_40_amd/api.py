"""Python binding of the C ABI (include/pa.h): same entry points, torch tensors in.

Argument marshalling only: shapes and dtypes are read from the tensors, device
pointers and the current HIP stream are passed through ctypes, and every step
of the computation runs in the HIP kernels of libpagedkv.so.  A nonzero status
raises RuntimeError with the library's message.

Debug mode (environment variable PA_DEBUG=1 at import, or set_debug(True)):
every call first runs the library's device-side precondition check for its
arguments (pa_check_attention / pa_check_write / pa_check_pairs), waits for it,
and raises PreconditionError instead of launching when a precondition fails.
The wait synchronizes the stream, so debug mode cannot run under HIP graph
capture (the C entry points pa_check_* only enqueue; the wrappers here wait
for the word).
"""

from __future__ import annotations

import os
from typing import Optional, Tuple

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.PA_F32, torch.float16: _lib.PA_F16}

_debug = os.environ.get("PA_DEBUG", "") not in ("", "0")


def set_debug(enabled: bool) -> None:
    """Check the device preconditions before every call (see the module docstring)."""
    global _debug
    _debug = bool(enabled)


def debug_enabled() -> bool:
    return _debug


class PreconditionError(RuntimeError):
    """A device-side precondition of a call does not hold: kind (a pa_check_kind name) and
    the lowest sequence or pair index showing it."""

    def __init__(self, what: str, kind: str, index: int):
        super().__init__(f"{what}: precondition {kind} violated at index {index}")
        self.kind, self.index = kind, index


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check_pool(k_pool: torch.Tensor, v_pool: torch.Tensor):
    _require(k_pool.dim() == 4 and k_pool.shape == v_pool.shape,
             "k_pool / v_pool must be [num_blocks][block_size][num_heads][head_dim] alike")
    _require(k_pool.dtype == v_pool.dtype and k_pool.dtype in _DTYPES, "pool dtype must be f32/f16")
    _require(k_pool.is_cuda and v_pool.is_cuda, "pools must be on the GPU")
    _require(k_pool.is_contiguous() and v_pool.is_contiguous(), "pools must be contiguous")
    nb, bs, h, d = k_pool.shape
    return nb, bs, h, d, _DTYPES[k_pool.dtype]


def _check_index(t: Optional[torch.Tensor], name: str, n: Optional[int] = None):
    if t is None:
        return
    _require(t.dtype == torch.int32 and t.is_cuda and t.is_contiguous(),
             f"{name} must be a contiguous int32 GPU tensor")
    if n is not None:
        _require(t.shape[0] == n, f"{name} must have {n} rows")


def _new_word(device) -> torch.Tensor:
    return torch.empty(1, dtype=torch.int64, device=device)


def _read_word(word: torch.Tensor, stream) -> Optional[Tuple[str, int]]:
    """Wait for the check on `stream`, then decode the word: None or (kind name, index)."""
    (torch.cuda.current_stream() if stream is None else stream).synchronize()
    w = int(word.item()) & 0xFFFFFFFFFFFFFFFF
    if w == _lib.PA_CHECK_OK:
        return None
    return _lib.CHECK_KINDS.get(w >> 32, f"kind {w >> 32}"), w & 0xFFFFFFFF


def pa_check_workspace_bytes(num_marks: int) -> int:
    return int(_lib.load().pa_check_workspace_bytes(int(num_marks)))


def pa_check_attention(k_pool, block_tables, context_lens, q_start_loc=None, num_tokens=None,
                       max_context_len: Optional[int] = None, max_query_len: int = 1,
                       sliding_window: int = 0, stream=None) -> Optional[Tuple[str, int]]:
    """Device preconditions of pa_decode(_ext) with these arguments.  Waits for the check and
    returns None when they hold, else (kind, lowest sequence index)."""
    nb, bs = k_pool.shape[0], k_pool.shape[1]
    S = context_lens.shape[0]
    _check_index(block_tables, "block_tables", S)
    _check_index(context_lens, "context_lens")
    _check_index(q_start_loc, "q_start_loc", S + 1)
    T = S if num_tokens is None else int(num_tokens)
    if max_context_len is None:
        max_context_len = int(context_lens.max().item())
    word = _new_word(context_lens.device)
    st = _lib.load().pa_check_attention(
        _ptr(word), nb, _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        _ptr(q_start_loc), S, T, int(max_context_len), int(max_query_len), bs,
        int(sliding_window), _stream(stream))
    _lib.check(st, "pa_check_attention")
    return _read_word(word, stream)


def pa_check_write(k_pool, block_tables, context_lens, write_start_loc=None, num_tokens=None,
                   stream=None) -> Optional[Tuple[str, int]]:
    """Device preconditions of pa_write_kv with these arguments (see pa_check_attention)."""
    nb, bs = k_pool.shape[0], k_pool.shape[1]
    S = context_lens.shape[0]
    _check_index(block_tables, "block_tables", S)
    _check_index(context_lens, "context_lens")
    _check_index(write_start_loc, "write_start_loc", S + 1)
    T = S if num_tokens is None else int(num_tokens)
    need = pa_check_workspace_bytes(nb * bs)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=context_lens.device)
    word = _new_word(context_lens.device)
    st = _lib.load().pa_check_write(
        _ptr(word), _ptr(ws), need, nb, _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), _ptr(write_start_loc), S, T, bs, _stream(stream))
    _lib.check(st, "pa_check_write")
    return _read_word(word, stream)


def pa_check_pairs(block_pairs, num_src_blocks: int, num_dst_blocks: int, same_pool: bool,
                   stream=None) -> Optional[Tuple[str, int]]:
    """Device preconditions of pa_copy_blocks (same_pool) or pa_swap_blocks; returns None or
    (kind, lowest pair index)."""
    _check_index(block_pairs, "block_pairs")
    _require(block_pairs.dim() == 2 and block_pairs.shape[1] == 2, "block_pairs must be [n][2]")
    need = pa_check_workspace_bytes(num_dst_blocks)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=block_pairs.device)
    word = _new_word(block_pairs.device)
    st = _lib.load().pa_check_pairs(_ptr(word), _ptr(ws), need, int(num_src_blocks),
                                    int(num_dst_blocks), _ptr(block_pairs),
                                    block_pairs.shape[0], 1 if same_pool else 0, _stream(stream))
    _lib.check(st, "pa_check_pairs")
    return _read_word(word, stream)


def _raise_if(found, what: str) -> None:
    if found is not None:
        raise PreconditionError(what, found[0], found[1])


def pa_decode_workspace_bytes(num_tokens: int, num_heads: int, head_dim: int,
                              max_context_len: int) -> int:
    return int(_lib.load().pa_decode_workspace_bytes(num_tokens, num_heads, head_dim,
                                                     max_context_len))


def pa_write_kv(k_pool, v_pool, k_new, v_new, block_tables, context_lens,
                write_start_loc=None, stream=None) -> None:
    nb, bs, h, d, dt = _check_pool(k_pool, v_pool)
    S = context_lens.shape[0]
    _check_index(block_tables, "block_tables", S)
    _check_index(context_lens, "context_lens")
    _check_index(write_start_loc, "write_start_loc", S + 1)
    T = k_new.shape[0]
    _require(k_new.shape == v_new.shape == (T, h, d), "k_new / v_new must be [T][H][d]")
    _require(k_new.dtype == v_new.dtype == k_pool.dtype, "k_new / v_new dtype must match the pool")
    _require(k_new.is_contiguous() and v_new.is_contiguous(), "k_new / v_new must be contiguous")
    if _debug:
        _raise_if(pa_check_write(k_pool, block_tables, context_lens, write_start_loc, T, stream),
                  "pa_write_kv")
    st = _lib.load().pa_write_kv(
        _ptr(k_pool), _ptr(v_pool), nb, _ptr(k_new), _ptr(v_new), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), _ptr(write_start_loc), S, T, h, d, bs, dt,
        _stream(stream))
    _lib.check(st, "pa_write_kv")


def pa_copy_blocks(k_pool, v_pool, block_pairs, stream=None) -> None:
    nb, bs, h, d, dt = _check_pool(k_pool, v_pool)
    _check_index(block_pairs, "block_pairs")
    _require(block_pairs.dim() == 2 and block_pairs.shape[1] == 2, "block_pairs must be [n][2]")
    if _debug:
        _raise_if(pa_check_pairs(block_pairs, nb, nb, True, stream), "pa_copy_blocks")
    st = _lib.load().pa_copy_blocks(_ptr(k_pool), _ptr(v_pool), nb, _ptr(block_pairs),
                                    block_pairs.shape[0], h, d, bs, dt, _stream(stream))
    _lib.check(st, "pa_copy_blocks")


def pa_swap_blocks(k_pool, v_pool, host_k, host_v, block_pairs, direction: str,
                   stream=None) -> None:
    """Move whole blocks between the device pools and a pinned host swap pool.

    direction "out": host[dst] = device[src]; "in": device[dst] = host[src], per row
    (src, dst) of block_pairs (int32 GPU tensor [n][2]).  host_k / host_v: CPU tensors of the
    pool layout allocated with pin_memory=True."""
    nb, bs, h, d, dt = _check_pool(k_pool, v_pool)
    _check_index(block_pairs, "block_pairs")
    _require(block_pairs.dim() == 2 and block_pairs.shape[1] == 2, "block_pairs must be [n][2]")
    _require(direction in ("out", "in"), "direction must be 'out' or 'in'")
    _require(host_k.dim() == 4 and host_k.shape == host_v.shape and
             tuple(host_k.shape[1:]) == (bs, h, d), "host pools must be [n][block_size][H][d]")
    _require(host_k.dtype == host_v.dtype == k_pool.dtype, "host pool dtype must match")
    _require(not host_k.is_cuda and not host_v.is_cuda and host_k.is_contiguous() and
             host_v.is_contiguous(), "host pools must be contiguous CPU tensors")
    _require(host_k.is_pinned() and host_v.is_pinned(), "host pools must be pinned memory")
    if _debug:
        nh = host_k.shape[0]
        src_n, dst_n = (nb, nh) if direction == "out" else (nh, nb)
        _raise_if(pa_check_pairs(block_pairs, src_n, dst_n, False, stream), "pa_swap_blocks")
    st = _lib.load().pa_swap_blocks(
        _ptr(k_pool), _ptr(v_pool), nb, _ptr(host_k), _ptr(host_v), host_k.shape[0],
        _ptr(block_pairs), block_pairs.shape[0],
        _lib.PA_SWAP_OUT if direction == "out" else _lib.PA_SWAP_IN, h, d, bs, dt,
        _stream(stream))
    _lib.check(st, "pa_swap_blocks")


def pa_decode(out, q, k_pool, v_pool, block_tables, context_lens, q_start_loc=None,
              max_context_len: Optional[int] = None, max_query_len: int = 1,
              workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Attention of q over the paged context; writes and returns `out`.

    max_context_len: host bound on context_lens (read from the device when omitted).
    workspace: a uint8 GPU tensor of at least pa_decode_workspace_bytes(...) bytes
    (allocated here when omitted).
    """
    return pa_decode_ext(out, q, k_pool, v_pool, block_tables, context_lens, q_start_loc,
                         max_context_len, max_query_len, workspace, 0, None, False, stream)


def pa_decode_ext(out, q, k_pool, v_pool, block_tables, context_lens, q_start_loc=None,
                  max_context_len: Optional[int] = None, max_query_len: int = 1,
                  workspace: Optional[torch.Tensor] = None, sliding_window: int = 0,
                  alibi_slopes: Optional[torch.Tensor] = None, shared_blocks: bool = False,
                  stream=None, group: int = 0) -> torch.Tensor:
    """pa_decode with a sliding window (0 = none), optional per-head ALiBi slopes (float32
    GPU tensor [num_heads]) and the shared-blocks scheduling hint (same results, faster when
    neighbouring sequences share blocks).  group = g in 2..6: sequences come in runs of g
    whose members may share leading blocks (samples of one prompt, beams of one search); rows
    every member of a run holds in the same blocks are read once for the run (fp16, one query
    per sequence, no window, not with shared_blocks; ALiBi slopes allowed)."""
    nb, bs, h, d, dt = _check_pool(k_pool, v_pool)
    S = context_lens.shape[0]
    T = q.shape[0]
    _check_index(block_tables, "block_tables", S)
    _check_index(context_lens, "context_lens")
    _check_index(q_start_loc, "q_start_loc", S + 1)
    _require(q.shape == (T, h, d) and out.shape == q.shape, "q / out must be [T][H][d]")
    _require(q.dtype == out.dtype == k_pool.dtype, "q / out dtype must match the pool")
    _require(q.is_contiguous() and out.is_contiguous(), "q / out must be contiguous")
    _require(0 <= int(group) <= 15, "group must be in 0..15 (2..6 are built)")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item())
    need = pa_decode_workspace_bytes(T, h, d, max_context_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if alibi_slopes is not None:
        _require(alibi_slopes.dtype == torch.float32 and alibi_slopes.is_cuda and
                 alibi_slopes.is_contiguous() and alibi_slopes.numel() == h,
                 "alibi_slopes must be a contiguous float32 GPU tensor [num_heads]")
    if _debug:
        _raise_if(pa_check_attention(k_pool, block_tables, context_lens, q_start_loc, T,
                                     max_context_len, max_query_len, sliding_window, stream),
                  "pa_decode")
    st = _lib.load().pa_decode_ext(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), nb, _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), _ptr(q_start_loc), S, T, int(max_context_len),
        int(max_query_len), h, d, bs, dt, _ptr(workspace), ws_bytes, int(sliding_window),
        _ptr(alibi_slopes),
        (_lib.PA_DECODE_SHARED_BLOCKS if shared_blocks else 0) |
        (int(group) << _lib.PA_DECODE_GROUP_SHIFT),
        _stream(stream))
    _lib.check(st, "pa_decode")
    return out


def pa_decode_noalloc(out, q, k_pool, v_pool, block_tables, context_lens, q_start_loc=None,
                      max_context_len: Optional[int] = None, max_query_len: int = 1,
                      sliding_window: int = 0, alibi_slopes: Optional[torch.Tensor] = None,
                      shared_blocks: bool = False, stream=None, group: int = 0) -> torch.Tensor:
    """pa_decode_ext without a workspace argument: the partial results live in the library's
    fixed device array (PA_NOALLOC_WORKSPACE_BYTES per device), so neither the library nor this
    wrapper allocates.  Calls that overlap on one device race on that array.
    max_context_len must be given (reading it from the device would synchronise)."""
    nb, bs, h, d, dt = _check_pool(k_pool, v_pool)
    S = context_lens.shape[0]
    T = q.shape[0]
    _check_index(block_tables, "block_tables", S)
    _check_index(context_lens, "context_lens")
    _check_index(q_start_loc, "q_start_loc", S + 1)
    _require(q.shape == (T, h, d) and out.shape == q.shape, "q / out must be [T][H][d]")
    _require(q.dtype == out.dtype == k_pool.dtype, "q / out dtype must match the pool")
    _require(q.is_contiguous() and out.is_contiguous(), "q / out must be contiguous")
    _require(0 <= int(group) <= 15, "group must be in 0..15 (2..6 are built)")
    _require(max_context_len is not None, "max_context_len is required")
    if alibi_slopes is not None:
        _require(alibi_slopes.dtype == torch.float32 and alibi_slopes.is_cuda and
                 alibi_slopes.is_contiguous() and alibi_slopes.numel() == h,
                 "alibi_slopes must be a contiguous float32 GPU tensor [num_heads]")
    st = _lib.load().pa_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), nb, _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), _ptr(q_start_loc), S, T, int(max_context_len),
        int(max_query_len), h, d, bs, dt, int(sliding_window), _ptr(alibi_slopes),
        (_lib.PA_DECODE_SHARED_BLOCKS if shared_blocks else 0) |
        (int(group) << _lib.PA_DECODE_GROUP_SHIFT),
        _stream(stream))
    _lib.check(st, "pa_decode_noalloc")
    return out


def pa_strerror(status: int) -> str:
    return _lib.strerror(status)
