#!/usr/bin/env python3
"""Throughput of the paged KV-cache hot path on one MI355X.

One step = the whole path over one batch: pa_write_kv appends this step's
token per sequence into its cache slot, then pa_decode (context partitions +
merge pass) computes paged attention for every (sequence, head).  Default
batch: 256 sequences x 40 heads, head_dim 128, block size 16, fp16 K/V/q with
fp32 accumulation, context lengths U{1024..4096} before the append, a shared
pool of 47,104 blocks (15.4 GB of K+V), synthetic seeded data already resident
in HBM.

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
                  "paged_kv_cache_40_amd/csrc/pa_common.hpp"]


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


# ---------------------------------------------------------------- cpu leg --

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
    return {
        "value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
        "seconds": round(dt, 3),
        "seq_heads_per_s": round(len(seqs) * w.num_heads / dt, 1),
        "sample": f"first {len(seqs)} of {w.num_seqs} sequences (all {w.num_heads} heads): the "
                  f"oracle's slot write + fp64 paged attention, one sequence per task over "
                  f"{workers} worker processes; {kv / 1e9:.3f} GB of fp16 K/V counted",
    }


# ---------------------------------------------------------------- gpu leg --

def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=5)
    ap.add_argument("--cpu-seqs", type=int, default=256, help="oracle sample size (0 = skip)")
    ap.add_argument("--cpu-workers", type=int, default=0, help="0 = min(16, host cores)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (PMC byte calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not "
              "supported (the path has no cross-GPU step to measure)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from paged_kv_cache_40_amd import _lib, api
    from workloads import make_config

    _lib.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
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
        workers = args.cpu_workers or min(16, os.cpu_count() or 1)
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
        "decode_ms": round(decode_ms, 4),
        "decode_ms_p10_p90": [round(float(np.percentile(dec, 10)), 4),
                              round(float(np.percentile(dec, 90)), 4)],
        "write_ms": round(write_ms, 4),
        "roofline": {
            "kernel": "pa_decode (partition pass + merge pass)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
