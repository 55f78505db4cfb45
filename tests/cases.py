"""Batches shared by several tests: the marked long-context cases, shared by a GPU parity
test and the CPU test that shows how sharp it is (defined once here so the CPU side,
tests/test_sensitivity.py, reasons about exactly the inputs the GPU side,
tests/test_gpu_parity.py, runs), and the lengths of the longest-first dispatch cases.
"""

import numpy as np

from workloads import make_custom_decode, make_custom_mixed

# Block-marked values (workloads.configs: v_mark) with keys scaled by 1/8, so every token
# carries a similar softmax weight and every block a distinct, large value pattern.  The
# decode path keeps the softmax weights in fp32 and takes a large amplitude; the chunk (tile)
# path rounds them to fp16 for its matrix product with V, an error of about 2^-12 * |v| /
# sqrt(context) that must stay well inside the 2e-3 tolerance (about 7e-5 here), so its
# amplitude is small - still large enough that any one dropped full block exceeds the
# tolerance more than ten times.
LONG_MARK = dict(k_scale=0.125, v_mark=2048.0)
CHUNK_MARK = dict(k_scale=0.125, v_mark=64.0)


def long_decode_marked():
    """A 100,000-token decode (about fifty 2,048-token partitions merged), a 65,537-token one
    (its last partition and last block hold only the appended token), next to short ones."""
    return make_custom_decode(81, "f16", 4, 128, 16, [100000, 65537, 3, 700], write_one=True,
                              name="long_decode_marked", **LONG_MARK)


def long_chunk_marked():
    """A 300-query chunk over a 30,000-token prior and a short chunk, next to decodes."""
    return make_custom_mixed(82, 2, 16, [(30000, 300), (5, 40)], [20000, 9],
                             name="long_chunk_marked", **CHUNK_MARK)


def ordered_lens(seed, n, long_len):
    """Context lengths with many equal values and a few long ones: a batch whose bound
    (sequences x heads x longest context x K and V bytes) makes the library dispatch the
    sequences longest first, so that ties and the rank computation are exercised."""
    rng = np.random.default_rng(seed)
    lens = rng.choice([1, 2, 15, 16, 17, 255, 256, 257, 1000], size=n).astype(np.int32)
    lens[[3, n // 2, n - 1]] = long_len
    return lens
