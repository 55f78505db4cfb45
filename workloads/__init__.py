"""Seeded synthetic inputs for the paged KV-cache hot path.

This package is shared by both sides of every parity check (the HIP library
and the fp64 oracle).  It draws numbers and lays out the structure of a batch
(context lengths, which physical blocks each sequence owns, which blocks are
shared); it computes nothing of the attention, the slot write or the block
copy themselves.
"""

from .gen import normal_values, normal_values_torch, full_values, key_for  # noqa: F401
from .configs import (  # noqa: F401
    Workload,
    make_config,
    make_small,
    make_custom_decode,
    make_custom_mixed,
    CONFIG_NAMES,
)
