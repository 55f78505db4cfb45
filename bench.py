#!/usr/bin/env python3
"""Throughput of the paged KV-cache hot path on one MI355X.

One step = the whole path over one batch: pa_write_kv appends this step's
token per sequence into its cache slot, then pa_decode (longest-first order,
context partitions + merge pass) computes paged attention for every (sequence,
head).  Default batch: 256 sequences x 40 heads, head_dim 128, block size 16,
fp16 K/V/q with fp32 accumulation, context lengths U{1024..4096} before the
append, a shared pool of 47,104 blocks (15.4 GB of K+V), synthetic seeded data
already resident in HBM.

Printed (one JSON line): K/V GB/s read = algorithmic K/V bytes of the step
(every valid K and V row of every sequence once) / wall time per step; plus
% of the 8 TB/s HBM peak, seq-heads/s, a roofline record for pa_decode timed
with HIP events on its stream, and the fp64 oracle timed on a bounded sample
of the same batch on the host cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode attention: K/V GB/s read & % of HBM peak; seq-heads/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pa_decode_traffic.json")
DECODE_SOURCES = ["paged_kv_cache_40_amd/csrc/pa_decode.hip",
                  "paged_kv_cache_40_amd/csrc/pa_common.hpp",
                  "paged_kv_cache_40_amd/csrc/pa_internal.hpp"]


def decode_source_hash() -> str:
    h = hashlib.sha256()
    for p in DECODE_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kv_bytes_unused=None):
    """HBM bytes per pa_decode launch from committed PMC counts, if they match the current
    kernel source; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("decode_source_sha") != decode_source_hash():
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------ hbm ceiling --

def hbm_stream_read_gbs(buf, reps: int = 5) -> float:
    """Median read bandwidth of the streaming-read probe over `buf` (a device tensor), GB/s."""
    import ctypes

    import numpy as np
    import torch

    from paged_kv_cache_40_amd.build import PROBE_LIB

    lib = ctypes.CDLL(PROBE_LIB)
    lib.pa_probe_stream_read.restype = ctypes.c_int
    lib.pa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_int32, ctypes.c_void_p]
    nbytes = (buf.numel() * buf.element_size()) // 16 * 16
    blocks = 2048  # 8 workgroups per CU, each streaming whole 256 KB chunks
    out = torch.empty(blocks * 256, dtype=torch.int32, device=buf.device)
    stream = torch.cuda.current_stream()
    times = []
    for i in range(reps + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        rc = lib.pa_probe_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), blocks,
                                      stream.cuda_stream)
        b.record(stream)
        if rc != 0:
            raise RuntimeError("HBM probe launch failed")
        torch.cuda.synchronize()
        if i:
            times.append(a.elapsed_time(b))
    return nbytes / (float(np.median(times)) * 1e-3) / 1e9


# ---------------------------------------------------------------- cpu leg --

# Oracle worker processes: every core the process may run on, at most 16 - one GPU's share of
# the host cores where this runs (os.cpu_count() reports the whole machine).  The record
# carries host_cores, available_cores and the workers actually used.
CPU_WORKER_CAP = 16


def default_cpu_workers() -> int:
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(CPU_WORKER_CAP, avail))


def _cpu_worker(args):
    shm, i = args
    import numpy as np
    import oracle
    z = np.load(os.path.join(shm, "sub.npz"))
    kp = np.load(os.path.join(shm, "k.npy"), mmap_mode="r")
    vp = np.load(os.path.join(shm, "v.npy"), mmap_mode="r")
    bt, cl, B = z["bt"], z["cl"], int(z["B"])
    # the oracle's slot write for this sequence's new token, then its attention
    kw, vw = oracle.write_kv(kp[bt[i, :(cl[i] + B - 1) // B]], vp[bt[i, :(cl[i] + B - 1) // B]],
                             z["kn"][i:i + 1], z["vn"][i:i + 1],
                             np.arange((cl[i] + B - 1) // B, dtype=np.int32)[None],
                             cl[i:i + 1], B)
    oracle.paged_attention_seq(z["q"][i:i + 1], kw, vw,
                               np.arange(kw.shape[0], dtype=np.int32), int(cl[i]), B)
    return i


def cpu_baseline(w, t, nseq: int, workers: int):
    """Time the oracle on the first `nseq` sequences of the batch (write + attention)."""
    import multiprocessing as mp

    import numpy as np
    import torch

    seqs = list(range(min(nseq, w.num_seqs)))
    B = w.block_size
    nb = -(-w.context_lens[seqs].astype(np.int64) // B)
    blocks = np.concatenate([w.block_tables[s, :nb[i]] for i, s in enumerate(seqs)])
    uniq, inv = np.unique(blocks, return_inverse=True)
    idx = torch.from_numpy(uniq.astype(np.int64)).cuda()
    shm = tempfile.mkdtemp(prefix="pa_cpu_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        np.save(os.path.join(shm, "k.npy"), t["k_pool"].index_select(0, idx).cpu().numpy())
        np.save(os.path.join(shm, "v.npy"), t["v_pool"].index_select(0, idx).cpu().numpy())
        bt = np.full((len(seqs), int(nb.max())), -1, np.int32)
        pos = 0
        for i in range(len(seqs)):
            bt[i, :nb[i]] = inv[pos:pos + nb[i]]
            pos += nb[i]
        rows = torch.tensor(seqs, device="cuda")
        np.savez(os.path.join(shm, "sub.npz"), bt=bt, cl=w.context_lens[seqs], B=B,
                 q=t["q"][rows].cpu().numpy(), kn=t["k_new"][rows].cpu().numpy(),
                 vn=t["v_new"][rows].cpu().numpy())
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers) as pool:
            pool.map(_cpu_worker, [(shm, 0)] * workers)      # warm the workers (imports)
            t0 = time.perf_counter()
            pool.map(_cpu_worker, [(shm, i) for i in range(len(seqs))], chunksize=1)
            dt = time.perf_counter() - t0
    finally:
        for f in os.listdir(shm):
            os.unlink(os.path.join(shm, f))
        os.rmdir(shm)
    kv = 2 * int(w.context_lens[seqs].astype(np.int64).sum()) * w.num_heads * w.head_dim * w.elt_bytes
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return {
        "value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
        "host_cores": os.cpu_count(), "available_cores": avail, "workers": workers,
        "worker_cap": CPU_WORKER_CAP,
        "seconds": round(dt, 3),
        "seq_heads_per_s": round(len(seqs) * w.num_heads / dt, 1),
        "sample": f"first {len(seqs)} of {w.num_seqs} sequences (all {w.num_heads} heads): the "
                  f"oracle's slot write + fp64 paged attention, one sequence per task over "
                  f"{workers} worker processes; {kv / 1e9:.3f} GB of fp16 K/V counted",
    }


# ------------------------------------------------------------ kv memory --

def kv_memory(w) -> dict:
    """KV-cache memory use of the batch as the block tables lay it out.

    paged_waste: slots allocated but not holding a token, over all distinct blocks the
    tables use (a block shared by several sequences counts once, filled as far as its
    fullest sharer).  reserved_waste: the same ratio if every sequence had reserved a
    contiguous region of the batch's longest context, as a fixed-reservation cache would.
    The pages quote under 4% for the paged layout and 60-80% for reservation-based systems."""
    import numpy as np

    B = w.block_size
    filled = {}
    for s, L in enumerate(w.context_lens.astype(int)):
        for b in range(-(-L // B)):
            blk = int(w.block_tables[s, b])
            filled[blk] = max(filled.get(blk, 0), min(B, L - b * B))
    alloc = len(filled) * B
    used = sum(filled.values())
    L = w.context_lens.astype(np.int64)
    reserved = len(L) * int(L.max())
    return {"paged_waste": round(1 - used / alloc, 4), "blocks": len(filled),
            "reserved_waste": round(1 - int(L.sum()) / reserved, 4),
            "reserved_len": int(L.max())}


# ---------------------------------------------------------------- gpu leg --

def _timed(fn, steps: int, warmup: int):
    import numpy as np
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return wall_ms, float(np.median([a.elapsed_time(b) for a, b in ev]))


def _timed_flushed(fn, steps: int, warmup: int, scratch):
    """Median event time of fn() when a buffer larger than every cache (scratch) is rewritten
    before each call, so no K/V row of the previous call is still cached."""
    import numpy as np
    import torch

    for _ in range(warmup):
        scratch.add_(1)
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        scratch.add_(1)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def bench_config(args) -> int:
    """One of the other batches: its whole step (copy-on-write copies, slot writes, attention)."""
    import numpy as np
    import torch

    from paged_kv_cache_40_amd import api
    from workloads import CONFIG_NAMES, make_config

    extra = {"num_heads": args.heads} if args.heads else {}
    w = make_config(args.config, seed=args.config if args.seed == 5 else args.seed, **extra)
    workload = CONFIG_NAMES[args.config]
    if args.heads:  # one GPU's share of a batch whose heads are split over several GPUs
        full = make_config(args.config, seed=args.config if args.seed == 5 else args.seed)
        workload += (f"; one GPU's share with the {full.num_heads} heads split "
                     f"{full.num_heads // args.heads} ways: {args.heads} heads")
    t = w.device_tensors("cuda")
    need = api.pa_decode_workspace_bytes(w.num_queries, w.num_heads, w.head_dim,
                                         w.max_context_len)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    # runs of neighbouring sequences that share blocks: the samples of one prompt
    group = args.group
    if group is None:
        runs = int(w.extra.get("samples", 0))
        group = runs if 2 <= runs <= 6 and w.dtype == "f16" and not (
            args.window or args.no_shared_hint) else 0
        # too few joint units to fill the chip (e.g. one GPU's share of the heads): the
        # shared-blocks hint is faster there (16 runs x 5 heads: 0.083 vs 0.107 ms per step)
        if group and -(-w.num_seqs // group) * w.num_heads * -(-w.max_context_len // 256) < 1536:
            group = 0
    shared = w.shares_blocks() and not args.no_shared_hint and not group
    slopes = None
    if args.alibi:  # the ALiBi paper's geometric slopes
        slopes = torch.tensor(2.0 ** (-8.0 * (np.arange(w.num_heads) + 1) / w.num_heads),
                              dtype=torch.float32, device="cuda")

    def step():
        if w.copy_pairs is not None and len(w.copy_pairs):
            api.pa_copy_blocks(t["k_pool"], t["v_pool"], t["copy_pairs"])
        if w.num_writes:
            api.pa_write_kv(t["k_pool"], t["v_pool"], t["k_new"], t["v_new"], t["block_tables"],
                            t["context_lens"], t["write_start_loc"])
        api.pa_decode_ext(out, t["q"], t["k_pool"], t["v_pool"], t["block_tables"],
                          t["context_lens"], t["q_start_loc"], max_context_len=w.max_context_len,
                          max_query_len=w.max_query_len, workspace=ws, shared_blocks=shared,
                          sliding_window=args.window, alibi_slopes=slopes, group=group)

    wall_ms, ev_ms = _timed(step, args.steps, args.warmup)

    def attend():  # the attention call alone, on the pools as the step leaves them
        api.pa_decode_ext(out, t["q"], t["k_pool"], t["v_pool"], t["block_tables"],
                          t["context_lens"], t["q_start_loc"], max_context_len=w.max_context_len,
                          max_query_len=w.max_query_len, workspace=ws, shared_blocks=shared,
                          sliding_window=args.window, alibi_slopes=slopes, group=group)

    _, attend_ms = _timed(attend, args.steps, args.warmup)
    # the same step after a 1 GiB buffer (4x the 256 MB last-level cache) is rewritten
    scratch = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
    flushed_ms = _timed_flushed(step, args.steps, args.warmup, scratch)
    del scratch
    kv = w.kv_bytes_read()
    if args.window:  # K and V rows inside each query row's window, counted once per sequence
        L = w.context_lens.astype(np.int64)
        n = w.query_lens.astype(np.int64)
        first = np.maximum(0, L - n - args.window + 1)
        kv = int(2 * (L - first).sum() * w.num_heads * w.head_dim * w.elt_bytes)
    B = w.block_size
    unique = w.unique_blocks_read() * 2 * B * w.num_heads * w.head_dim * w.elt_bytes
    rec = {
        "metric": METRIC, "value": round(kv / (wall_ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": workload, "num_seqs": w.num_seqs,
                   "num_heads": w.num_heads, "head_dim": w.head_dim, "block_size": B,
                   "num_blocks": w.num_blocks, "num_queries": w.num_queries,
                   "num_writes": w.num_writes,
                   "copy_pairs": 0 if w.copy_pairs is None else len(w.copy_pairs),
                   "shared_blocks_hint": shared, "group": group, "sliding_window": args.window,
                   "alibi": bool(args.alibi),
                   "kv_bytes_logical": kv, "kv_bytes_unique_blocks": unique},
        "event_ms_per_step": round(ev_ms, 4),
        "flushed_event_ms_per_step": round(flushed_ms, 4),
        "flushed_GBs": round(kv / (flushed_ms * 1e-3) / 1e9, 2),
        "pct_hbm_peak_logical": round(100 * kv / (wall_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "seq_heads_per_s": round(w.num_seqs * w.num_heads / (wall_ms * 1e-3), 1),
        "kv_memory": kv_memory(w),
        # pa_decode_ext alone (HIP events, median of back-to-back calls, so a batch smaller
        # than a few times the 256 MB last-level cache is partly served from it): the K/V
        # bytes of the distinct blocks read (a shared block counts once: what HBM must
        # deliver) over its time, against the 8 TB/s HBM peak; not given with a window,
        # where blocks are read only in part
        "attention": {"event_ms": round(attend_ms, 4),
                      "GBs_logical": round(kv / (attend_ms * 1e-3) / 1e9, 2),
                      "GBs_distinct_blocks": None if args.window else
                      round(unique / (attend_ms * 1e-3) / 1e9, 2),
                      "frac_hbm_peak_distinct_blocks": None if args.window else
                      round(unique / (attend_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if w.max_query_len > 1:
        qh = w.num_queries * w.num_heads
        rec["query_heads_per_s"] = round(qh / (wall_ms * 1e-3), 1)
    print(json.dumps(rec), flush=True)
    return 0


def bench_variant(args) -> int:
    """The large batch with a sliding window and/or ALiBi slopes (pa_decode_ext): write + decode
    per step; bytes = K and V rows inside each sequence's window."""
    import numpy as np
    import torch

    from paged_kv_cache_40_amd import api
    from workloads import make_config

    w = make_config(5, seed=args.seed)
    t = w.device_tensors("cuda")
    H, D = w.num_heads, w.head_dim
    W = args.window
    slopes = None
    if args.alibi:
        slopes = torch.tensor(2.0 ** (-8.0 * (np.arange(H) + 1) / H), dtype=torch.float32,
                              device="cuda")
    need = api.pa_decode_workspace_bytes(w.num_queries, H, D, w.max_context_len)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    stream = torch.cuda.current_stream()

    def write():
        api.pa_write_kv(t["k_pool"], t["v_pool"], t["k_new"], t["v_new"], t["block_tables"],
                        t["context_lens"], stream=stream)

    def decode():
        api.pa_decode_ext(out, t["q"], t["k_pool"], t["v_pool"], t["block_tables"],
                          t["context_lens"], max_context_len=w.max_context_len, workspace=ws,
                          sliding_window=W, alibi_slopes=slopes, stream=stream)

    def step():
        write()
        decode()

    wall_ms, _ = _timed(step, args.steps, args.warmup)
    _, decode_ms = _timed(decode, args.steps, args.warmup)
    L = w.context_lens.astype(np.int64)
    seen = np.minimum(L, W) if W > 0 else L
    kv = int(2 * seen.sum() * H * D * w.elt_bytes)
    rec = {
        "metric": METRIC, "value": round(kv / (wall_ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "large-batch decode + KV write (256 seqs x 40 heads, contexts "
                               "1025..4097) with a sliding window and/or ALiBi",
                   "sliding_window": W, "alibi": bool(args.alibi), "kv_bytes_in_window": kv},
        "decode_ms": round(decode_ms, 4),
        "decode_GBs": round(kv / (decode_ms * 1e-3) / 1e9, 1),
        "pct_hbm_peak_decode": round(100 * kv / (decode_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_swap(args) -> int:
    """Swap the K/V blocks of the first --swap-seqs sequences of the large batch out to a pinned
    host pool and back (pa_swap_blocks), against plain contiguous copies of the same byte count
    between device memory and pinned host memory (the host-link ceiling on this machine)."""
    import numpy as np
    import torch

    from paged_kv_cache_40_amd import api
    from workloads import make_config

    w = make_config(5, seed=args.seed)
    t = w.device_tensors("cuda")
    B = w.block_size
    n = min(args.swap_seqs, w.num_seqs)
    nb = -(-w.context_lens[:n].astype(np.int64) // B)
    blocks = np.concatenate([w.block_tables[s, :nb[s]] for s in range(n)]).astype(np.int32)
    NH = len(blocks)
    shape = (NH,) + tuple(t["k_pool"].shape[1:])
    hk = torch.empty(shape, dtype=torch.float16, pin_memory=True)
    hv = torch.empty(shape, dtype=torch.float16, pin_memory=True)
    host_ids = np.arange(NH, dtype=np.int32)
    out_pairs = torch.from_numpy(np.stack([blocks, host_ids], 1)).cuda()
    in_pairs = torch.from_numpy(np.stack([host_ids, blocks], 1)).cuda()
    stream = torch.cuda.current_stream()
    nbytes = 2 * NH * hk[0].numel() * hk.element_size()

    def swap_out():
        api.pa_swap_blocks(t["k_pool"], t["v_pool"], hk, hv, out_pairs, "out", stream=stream)

    def swap_in():
        api.pa_swap_blocks(t["k_pool"], t["v_pool"], hk, hv, in_pairs, "in", stream=stream)

    dev_buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    host_buf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)

    def d2h():
        host_buf.copy_(dev_buf, non_blocking=True)

    def h2d():
        dev_buf.copy_(host_buf, non_blocking=True)

    steps = max(3, args.steps // 3)
    res = {}
    for name, fn in (("swap_out", swap_out), ("swap_in", swap_in), ("copy_d2h", d2h),
                     ("copy_h2d", h2d)):
        _, ms = _timed(fn, steps, 2)
        res[name] = ms
    gbs = {k: nbytes / (v * 1e-3) / 1e9 for k, v in res.items()}
    value = 2 * nbytes / ((res["swap_out"] + res["swap_in"]) * 1e-3) / 1e9
    rec = {
        "metric": "KV block swap GB/s, device pool <-> pinned host pool (out + in)",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": 2,
        "ms_per_step": round(res["swap_out"] + res["swap_in"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"swap out and back in every K/V block of {n} sequences of the "
                               "large batch (256 x 40 heads, d=128, B=16, contexts 1025..4097)",
                   "blocks": NH, "bytes_each_way": nbytes},
        "swap_out_ms": round(res["swap_out"], 4), "swap_in_ms": round(res["swap_in"], 4),
        "swap_out_GBs": round(gbs["swap_out"], 2), "swap_in_GBs": round(gbs["swap_in"], 2),
        "contiguous_copy_d2h_GBs": round(gbs["copy_d2h"], 2),
        "contiguous_copy_h2d_GBs": round(gbs["copy_h2d"], 2),
        "frac_of_contiguous": {"out": round(gbs["swap_out"] / gbs["copy_d2h"], 4),
                               "in": round(gbs["swap_in"] / gbs["copy_h2d"], 4)},
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_beam(args) -> int:
    """Beam-search decoding on the large-batch shape: 64 requests (prompts U{1024..4096}) x width
    --beam candidates, 40 heads, d=128, B=16, fp16.  The block manager's steps (forks, prunes,
    copy-on-write pairs, slots, tables) are computed on the host first; the timed loop runs each
    step's pa_copy_blocks + pa_write_kv + pa_decode on the GPU."""
    import numpy as np
    import torch

    from paged_kv_cache_40_amd import BlockManager, api, tables_to_array
    from paged_kv_cache_40_amd.beam import BeamSearchKV, memory_saving
    from workloads.beam import beam_rows_torch, make_beam_tree

    W, H, D, B, R, steps = args.beam, 40, 128, 16, 64, args.beam_steps
    # a request's beams sit next to each other: runs of W for the grouped decode (2..6)
    group = args.group
    if group is None:
        group = W if 2 <= W <= 6 and not args.no_shared_hint else 0
    rng = np.random.default_rng(args.seed)
    prompts = rng.integers(1024, 4097, size=R)
    trees = [make_beam_tree(1000 + i, W, steps, int(P)) for i, P in enumerate(prompts)]
    NB = int(sum(W * (-(-(int(P) + steps) // B) + 1) for P in prompts))
    bm = BlockManager(NB, B)
    reqs = [BeamSearchKV(bm, tr.prompt_len) for tr in trees]
    prefill_tables = tables_to_array([r.beams[0] for r in reqs])
    plan, savings = [], []
    host_s = 0.0
    for t in range(steps):
        t0 = time.perf_counter()
        for r, tr in zip(reqs, trees):
            r.step(tr.parents[t])
        pairs = bm.take_copies()
        tables = [tb for r in reqs for tb in r.beams]
        lens = np.asarray([n for r in reqs for n in r.num_tokens()], np.int32)
        plan.append((pairs, tables_to_array(tables), lens))
        host_s += time.perf_counter() - t0
        savings.append(memory_saving(reqs))
    host_ms = host_s * 1e3 / steps
    print(f"[bench] beam plan: {steps} steps, host bookkeeping {host_ms:.2f} ms/step",
          file=sys.stderr, flush=True)

    kp = torch.empty((NB, B, H, D), dtype=torch.float16, device="cuda")
    vp = torch.empty_like(kp)
    gen = [beam_rows_torch(tr, H, D, torch.float16, "cuda") for tr in trees]
    wsl = torch.tensor(np.concatenate([[0], np.cumsum(prompts)]), dtype=torch.int32, device="cuda")
    api.pa_write_kv(kp, vp, torch.cat([g[0][:int(P)] for g, P in zip(gen, prompts)]),
                    torch.cat([g[1][:int(P)] for g, P in zip(gen, prompts)]),
                    torch.from_numpy(prefill_tables).cuda(),
                    torch.tensor(prompts, dtype=torch.int32, device="cuda"), wsl)
    dev = []
    for t, (pairs, bt, lens) in enumerate(plan):
        ids = [tr.token_id(t, b) for tr in trees for b in range(W)]
        req = [i for i in range(R) for _ in range(W)]
        kn = torch.stack([gen[i][0][j] for i, j in zip(req, ids)])
        vn = torch.stack([gen[i][1][j] for i, j in zip(req, ids)])
        q = torch.cat([g[2][t] for g in gen])
        dev.append(dict(pairs=torch.from_numpy(pairs).cuda() if len(pairs) else None,
                        bt=torch.from_numpy(bt).cuda(), cl=torch.from_numpy(lens).cuda(),
                        mcl=int(lens.max()), kn=kn, vn=vn, q=q))
    del gen
    mcl = max(d["mcl"] for d in dev)
    ws = torch.empty(max(api.pa_decode_workspace_bytes(R * W, H, D, mcl), 1), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((R * W, H, D), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()

    def run_step(d):
        if d["pairs"] is not None:
            api.pa_copy_blocks(kp, vp, d["pairs"])
        api.pa_write_kv(kp, vp, d["kn"], d["vn"], d["bt"], d["cl"])
        api.pa_decode_ext(out, d["q"], kp, vp, d["bt"], d["cl"], max_context_len=d["mcl"],
                          workspace=ws, shared_blocks=not (args.no_shared_hint or group),
                          group=group)

    kp0, vp0 = kp.clone(), vp.clone()  # the pools after the prefill, for the graph replays
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    t0 = time.perf_counter()
    for d in dev:
        run_step(d)
    ev1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ev_ms = ev0.elapsed_time(ev1) / steps
    # the same plan captured once in a HIP graph and replayed from the post-prefill pools
    # (pruned beams' blocks are reused by others, so a replay must start where the eager
    # pass started): the GPU time of the steps without the host issuing each call, and the
    # last step's output, which must equal the eager one bit for bit
    eager_last = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for d in dev:
            run_step(d)
    graph_times, graph_same = [], True
    for _ in range(2):
        kp.copy_(kp0)
        vp.copy_(vp0)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_times.append(g0.elapsed_time(g1) / steps)
        graph_same &= bool(torch.equal(out.view(torch.int16), eager_last.view(torch.int16)))
    graph_ms = min(graph_times)
    del graph, kp0, vp0
    logical = int(sum(2 * int(lens.astype(np.int64).sum()) * H * D * 2 for _, _, lens in plan))
    unique = int(sum(2 * held * B * H * D * 2 for held, _, _ in savings))
    copies = int(sum(len(p) for p, _, _ in plan))
    rec = {
        "metric": "beam-search decode step: K/V GB/s read (logical) and candidate tokens/s",
        "value": round(logical / steps / (ev_ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": 0, "ms_per_step": round(ev_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"beam search, 64 requests x width {W}, prompts U{{1024..4096}}, "
                               "40 heads, d=128, B=16, fp16, synthetic beam trees",
                   "width": W, "requests": R, "num_blocks": NB,
                   "shared_blocks_hint": not (args.no_shared_hint or group),
                   "group": group},
        "wall_ms_per_step": round(wall_ms, 4),
        "graph_ms_per_step": round(graph_ms, 4),
        "graph_output_equals_eager": graph_same,
        "candidate_tokens_per_s": round(R * W / (ev_ms * 1e-3), 1),
        "unique_block_GBs": round(unique / steps / (ev_ms * 1e-3) / 1e9, 2),
        "cow_copies_per_step": round(copies / steps, 2),
        "memory_saving_mean": round(float(np.mean([s for _, _, s in savings])), 4),
        "memory_saving_final": round(savings[-1][2], 4),
        "host_bookkeeping_ms_per_step": round(host_ms, 3),
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_prefix(args) -> int:
    """Shared-prefix prefill with the content-hash prefix cache: 64 requests = a --prefix-token
    shared prefix + a private suffix of U{16..128} tokens, 40 heads, d=128, B=16, fp16.
    Cold: every prompt token is written and attended (chunked-prefill tile path).  Warm: the
    prefix blocks come from the cache (one earlier request computed them), only the suffix is
    written and attended, over the whole context."""
    import numpy as np
    import torch

    from paged_kv_cache_40_amd import api, tables_to_array
    from paged_kv_cache_40_amd.prefix_cache import PrefixCachingAllocator
    from workloads.gen import normal_values_torch

    H, D, B, R, P = 40, 128, 16, 64, args.prefix
    rng = np.random.default_rng(args.seed)
    suffix = rng.integers(16, 129, size=R)
    prefix_tokens = list(range(P))
    prompts = [prefix_tokens + [10**6 + r * 1000 + j for j in range(int(n))]
               for r, n in enumerate(suffix)]
    lens = np.asarray([len(p) for p in prompts], np.int32)
    NB = int(sum(-(-int(L) // B) for L in lens)) + 64

    def rows(stream, n):
        t = torch.empty((n, H, D), dtype=torch.float16, device="cuda")
        normal_values_torch(args.seed, stream, t)
        return t

    pk, pv, pq = rows(31, P), rows(32, P), rows(33, P)
    sk, sv, sq = rows(34, int(suffix.sum())), rows(35, int(suffix.sum())), rows(36, int(suffix.sum()))
    soff = np.concatenate([[0], np.cumsum(suffix)])

    def prompt_rows(src_p, src_s, r, start):
        """Rows of prompt r from token `start` on."""
        parts = []
        if start < P:
            parts.append(src_p[start:])
        parts.append(src_s[int(soff[r]) + max(0, start - P):int(soff[r + 1])])
        return torch.cat(parts)

    def plan(alloc, warm):
        if warm:                                  # one earlier request computed the prefix
            t, _ = alloc.allocate(prefix_tokens + [0])
            alloc.commit(t, prefix_tokens + [0])
        tables, cached = [], []
        for p in prompts:
            t, c = alloc.allocate(p)
            tables.append(t)
            cached.append(c)
        nq = lens - np.asarray(cached, np.int32)
        loc = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
        kn = torch.cat([prompt_rows(pk, sk, r, c) for r, c in enumerate(cached)])
        vn = torch.cat([prompt_rows(pv, sv, r, c) for r, c in enumerate(cached)])
        q = torch.cat([prompt_rows(pq, sq, r, c) for r, c in enumerate(cached)])
        held = len({b for t in tables for b in t})
        return dict(bt=torch.from_numpy(tables_to_array(tables)).cuda(),
                    cl=torch.from_numpy(lens).cuda(), ql=torch.from_numpy(loc).cuda(),
                    kn=kn, vn=vn, q=q, out=torch.empty_like(q), mql=int(nq.max()),
                    queries=int(nq.sum()), cached=int(sum(cached)), held=held,
                    hits=alloc.hits, lookups=alloc.lookups)

    res = {}
    for name, warm in (("cold", False), ("warm", True)):
        alloc = PrefixCachingAllocator(NB, B)
        kp = torch.zeros((NB, B, H, D), dtype=torch.float16, device="cuda")
        vp = torch.zeros_like(kp)
        d = plan(alloc, warm)
        if warm:
            first = d["bt"][0, :P // B].long()
            kp[first] = pk[:P // B * B].view(-1, B, H, D)      # the cached prefix blocks
            vp[first] = pv[:P // B * B].view(-1, B, H, D)
        ws = torch.empty(max(api.pa_decode_workspace_bytes(d["queries"], H, D, int(lens.max())), 1),
                         dtype=torch.uint8, device="cuda")

        def step(d=d, kp=kp, vp=vp, ws=ws):
            api.pa_write_kv(kp, vp, d["kn"], d["vn"], d["bt"], d["cl"], d["ql"])
            api.pa_decode(d["out"], d["q"], kp, vp, d["bt"], d["cl"], d["ql"],
                          max_context_len=int(lens.max()), max_query_len=d["mql"], workspace=ws)

        _, ms = _timed(step, args.steps, args.warmup)
        res[name] = dict(ms=ms, d=d)
        del kp, vp
    warm = res["warm"]["d"]
    unshared = int(sum(-(-int(L) // B) for L in lens))
    rec = {
        "metric": "shared-prefix prefill: ms per batch, cold vs prefix-cached",
        "value": round(res["warm"]["ms"], 4), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(res["warm"]["ms"], 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"64 requests = {P}-token shared prefix + U{{16..128}}-token "
                               "suffix, 40 heads, d=128, B=16, fp16; content-hash prefix cache",
                   "prefix": P, "requests": R, "prompt_tokens": int(lens.sum())},
        "cold_ms": round(res["cold"]["ms"], 4), "warm_ms": round(res["warm"]["ms"], 4),
        "speedup": round(res["cold"]["ms"] / res["warm"]["ms"], 3),
        "queries_cold": res["cold"]["d"]["queries"], "queries_warm": warm["queries"],
        "cached_tokens": warm["cached"],
        "block_hit_rate": round(warm["hits"] / warm["lookups"], 4) if warm["lookups"] else 0.0,
        "blocks_held_warm": warm["held"], "blocks_unshared": unshared,
        "blocks_saved": round(1 - warm["held"] / unshared, 4),
    }
    print(json.dumps(rec), flush=True)
    return 0


def sweep_batch(w, t, args) -> None:
    """Decode latency vs batch size (first S sequences of the batch), with the batch's scattered
    block tables and with identity tables (each sequence's blocks contiguous in the pool)."""
    import numpy as np
    import torch

    from paged_kv_cache_40_amd import api

    B = w.block_size
    nb = -(-w.context_lens.astype(np.int64) // B)
    ident = np.full_like(w.block_tables, -1)
    pos = 0
    for s in range(w.num_seqs):
        ident[s, :nb[s]] = np.arange(pos, pos + nb[s])
        pos += nb[s]
    tables = {"scattered": t["block_tables"], "identity": torch.from_numpy(ident).cuda()}
    for S in (1, 8, 32, 64, 128, 256):
        if S > w.num_seqs:
            break
        kv = int(2 * w.context_lens[:S].astype(np.int64).sum() * w.num_heads * w.head_dim *
                 w.elt_bytes)
        mcl = int(w.context_lens[:S].max())
        need = api.pa_decode_workspace_bytes(S, w.num_heads, w.head_dim, mcl)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(t["q"][:S])
        for name, bt in tables.items():
            def dec(bt=bt):
                api.pa_decode(out, t["q"][:S], t["k_pool"], t["v_pool"], bt[:S],
                              t["context_lens"][:S], max_context_len=mcl, workspace=ws)
            _, ms = _timed(dec, max(5, args.steps // 2), 3)
            print(json.dumps({"sweep": "decode latency vs batch", "num_seqs": S, "table": name,
                              "decode_ms": round(ms, 4), "kv_bytes": kv,
                              "GBs": round(kv / (ms * 1e-3) / 1e9, 1)}), flush=True)



def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=5)
    ap.add_argument("--cpu-seqs", type=int, default=256, help="oracle sample size (0 = skip)")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="0 = every core this process may run on, at most CPU_WORKER_CAP")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (PMC byte calibration)")
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5],
                    help="batch to time (5 = the headline batch; 1-4 print their own line)")
    ap.add_argument("--sweep", action="store_true",
                    help="also print decode latency vs batch size, scattered vs identity tables")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window: the large batch's own variant line, or applied to "
                         "the batch of --config N")
    ap.add_argument("--alibi", action="store_true",
                    help="ALiBi slopes: the large batch's own variant line, or applied to the "
                         "batch of --config N")
    ap.add_argument("--swap", action="store_true",
                    help="time pa_swap_blocks out and in against plain host-link copies (own line)")
    ap.add_argument("--swap-seqs", type=int, default=64)
    ap.add_argument("--beam", type=int, default=0,
                    help="time beam-search decoding with this beam width instead (own line)")
    ap.add_argument("--beam-steps", type=int, default=64)
    ap.add_argument("--group", type=int, default=None,
                    help="grouped decode over runs of this many neighbouring sequences instead "
                         "of the shared-blocks hint; default: the batch's own runs (the samples "
                         "of one prompt, the beams of one request); 0: off")
    ap.add_argument("--no-shared-hint", action="store_true",
                    help="never pass the shared-blocks hint (for comparison)")
    ap.add_argument("--prefix", type=int, default=0,
                    help="time shared-prefix prefill, cold vs prefix-cached (own line)")
    ap.add_argument("--heads", type=int, default=0,
                    help="with --config 2-5: that batch with this many heads (one GPU's share "
                         "when the heads are split over several GPUs), own line")
    args = ap.parse_args(argv)
    if args.heads and args.config == 1:
        ap.error("--heads applies to --config 2-5 (the tiny batch has fixed shapes)")

    if args.gpus != 1:
        print(f"bench.py: the paged-attention path is measured on exactly one GPU; --gpus {args.gpus} is not "
              "supported (the path has no cross-GPU step to measure)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from paged_kv_cache_40_amd import _lib, api
    from workloads import make_config

    _lib.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.config != 5 or args.heads:
        return bench_config(args)
    if args.window or args.alibi:
        return bench_variant(args)
    if args.swap:
        return bench_swap(args)
    if args.beam:
        return bench_beam(args)
    if args.prefix:
        return bench_prefix(args)
    w = make_config(5, seed=args.seed)
    print(f"[bench] generating {w.name}: S={w.num_seqs} H={w.num_heads} NB={w.num_blocks}",
          file=sys.stderr, flush=True)
    t = w.device_tensors("cuda")
    T, H, D = w.num_queries, w.num_heads, w.head_dim
    need = api.pa_decode_workspace_bytes(T, H, D, w.max_context_len)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    stream = torch.cuda.current_stream()

    cpu = None
    if args.cpu_seqs > 0:
        workers = args.cpu_workers or default_cpu_workers()
        print(f"[bench] cpu baseline: {args.cpu_seqs} sequences on {workers} workers",
              file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, t, args.cpu_seqs, workers)

    def write():
        api.pa_write_kv(t["k_pool"], t["v_pool"], t["k_new"], t["v_new"], t["block_tables"],
                        t["context_lens"], stream=stream)

    def decode():
        api.pa_decode(out, t["q"], t["k_pool"], t["v_pool"], t["block_tables"],
                      t["context_lens"], max_context_len=w.max_context_len, workspace=ws,
                      stream=stream)

    for _ in range(args.warmup):
        write()
        decode()
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record(stream)
        write()
        e[1].record(stream)
        decode()
        e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    write_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    dec = np.asarray([b.elapsed_time(c) for _, b, c in ev])
    decode_ms = float(dec.mean())

    if args.calib_copy_mb:
        n = args.calib_copy_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    if args.sweep:
        sweep_batch(w, t, args)
    hbm = hbm_stream_read_gbs(t["k_pool"])

    kv = w.kv_bytes_read()
    ms_per_step = wall * 1e3 / args.steps
    value = kv / (ms_per_step * 1e-3) / 1e9
    achieved = kv / (decode_ms * 1e-3) / 1e9
    traffic = measured_traffic()
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "large-batch decode + KV write: 256 seqs x 40 heads, head_dim 128, "
                        "block_size 16, fp16 K/V/q (fp32 accumulation), context U{1024..4096} "
                        "+ 1 appended token, pool 47,104 blocks, random block placement",
            "num_seqs": w.num_seqs, "num_heads": H, "head_dim": D, "block_size": w.block_size,
            "num_blocks": w.num_blocks, "seed": args.seed,
            "kv_bytes_per_step": kv,
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_heads_per_s": round(w.num_seqs * H / (ms_per_step * 1e-3), 1),
        "kv_memory": kv_memory(w),
        "decode_ms": round(decode_ms, 4),
        "decode_ms_p10_p90": [round(float(np.percentile(dec, 10)), 4),
                              round(float(np.percentile(dec, 90)), 4)],
        "write_ms": round(write_ms, 4),
        "roofline": {
            "kernel": "pa_decode (order + partition pass + merge pass)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "measured_stream_read": round(hbm, 1),
            "frac_of_measured": round(achieved / hbm, 4),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
