"""The full-batch oracle plumbing of the GPU tests, checked on the CPU (no GPU, no library call):
the process-pool oracle over a compact snapshot (copies and writes applied to the blocks involved
only) equals the oracle's whole-batch step, on small versions of every configuration."""

import numpy as np
import pytest

from paged_harness import host_copy, oracle_every_sequence, oracle_step, snapshot_for
from workloads import make_config, make_small


@pytest.mark.parametrize("idx", [1, 3, 4, 5])
def test_every_sequence_oracle_equals_whole_batch_step(idx):
    w = make_small(idx, seed=2) if idx != 1 else make_config(1, seed=2)
    t = w.device_tensors("cpu")
    h = host_copy(t)
    sub = snapshot_for(w, t, list(range(w.num_seqs)))
    refs, margins = oracle_every_sequence(w, sub, margins=True)
    ref, kp, vp = oracle_step(w, h)
    for i in range(w.num_seqs):
        assert np.array_equal(refs[i], ref[sub["q_rows"][i]]), i
    uniq = sub["uniq"]
    assert kp[uniq].tobytes() == sub["k_pool"][:-1].tobytes()
    assert vp[uniq].tobytes() == sub["v_pool"][:-1].tobytes()
    assert all(np.isfinite(v) for v in margins.values())
