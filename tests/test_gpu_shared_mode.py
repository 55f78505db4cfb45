"""The shared-blocks scheduling hint of pa_decode_ext (cached loads, neighbouring sequences
grouped on one XCD) changes where and when work units run, never what they compute: outputs
must be bit-identical to the plain launch, on batches that share blocks and on batches that
do not, and still match the oracle."""

import numpy as np
import pytest
import torch

from workloads import make_config, make_small, make_custom_decode
from paged_harness import (assert_close, host_copy, log, oracle_step, oracle_sub,
                           pick_sequences, run_library, snapshot_for)

pytestmark = pytest.mark.gpu


def same_bits(a, b):
    return torch.equal(a.view(torch.int16 if a.dtype == torch.float16 else torch.int32),
                       b.view(torch.int16 if b.dtype == torch.float16 else torch.int32))


def twice(w, **kw):
    """Plain and hinted launches on identical fresh inputs."""
    t1 = w.device_tensors("cuda")
    plain = run_library(w, t1, **kw)
    t2 = w.device_tensors("cuda")
    hinted = run_library(w, t2, shared=True, **kw)
    torch.cuda.synchronize()
    return t1, plain, hinted


@pytest.mark.parametrize("idx", [3, 5, 2])
def test_small_configs_bit_identical_and_correct(idx):
    w = make_small(idx, seed=4)
    log(f"[case] shared hint small {w.name} shares={w.shares_blocks()}")
    t, plain, hinted = twice(w)
    assert same_bits(plain, hinted)
    h = host_copy(w.device_tensors("cuda"))
    ref, _, _ = oracle_step(w, h)
    assert_close(hinted.cpu().numpy(), ref, w.dtype, w.name)
    log("[ok]")


def test_full_parallel_sampling_batch():
    w = make_config(3)
    assert w.shares_blocks()
    log(f"[case] shared hint full {w.name}")
    t = w.device_tensors("cuda")
    seqs = pick_sequences(w, n=4, seed=3)
    sub = snapshot_for(w, t, seqs)
    hinted = run_library(w, t, shared=True)
    t2 = w.device_tensors("cuda")
    plain = run_library(w, t2)
    torch.cuda.synchronize()
    assert same_bits(plain, hinted)
    refs, _, _ = oracle_sub(w, sub)
    for i, s in enumerate(seqs):
        rows = torch.from_numpy(sub["q_rows"][i]).cuda()
        assert_close(hinted[rows].cpu().numpy(), refs[i], w.dtype, f"seq {s}")
    log("[ok]")


@pytest.mark.parametrize("dtype,B,window", [("f16", 16, 0), ("f32", 8, 300), ("f16", 32, 100)])
def test_layouts_windows_and_uneven_grids(dtype, B, window):
    """Grids whose size is not a multiple of the XCD rotation (8 x 128 units), several
    partition sizes, windows, fp32."""
    lens = [1, 17, 255, 256, 257, 1000, 2049, 4100, 33, 9000, 3]
    w = make_custom_decode(81, dtype, 5, 128 if dtype == "f16" else 64, B, lens,
                           name=f"shared_hint_{dtype}_B{B}")
    log(f"[case] {w.name} W={window}")
    t, plain, hinted = twice(w, window=window)
    assert same_bits(plain, hinted)
    h = host_copy(t)
    ref, _, _ = oracle_step(w, h, window=window)
    assert_close(hinted.cpu().numpy(), ref, w.dtype, w.name)
    log("[ok]")


def test_large_batch_without_sharing_bit_identical():
    w = make_config(5)
    log(f"[case] shared hint on {w.name} (no sharing)")
    t, plain, hinted = twice(w)
    assert same_bits(plain, hinted)
    log("[ok]")
