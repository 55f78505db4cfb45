"""fp64 CPU oracle for the paged KV-cache hot path — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check in __graft_entry__ and the `cpu_baseline` leg
of bench.py may import anything from this package.  The library under
paged_kv_cache_40_amd/ never does, and this package imports nothing from it:
the two share no code, headers, helpers or tables.  The only common inputs
come from the seeded generators in workloads/.

What it computes (plain definitions, written out; no blocking, fusion or
reordering beyond what the definitions state):
  * attention.py — softmax attention of each query over its sequence's keys,
    with the keys and values fetched token by token through the block table;
  * kv_ops.py    — the slot write of newly generated tokens, the
    copy-on-write whole-block copy and the block swap between the device
    pool and a host swap pool;
  * sizes.py     — the KV-cache byte formulas;
  * preconditions.py — the conditions the device-resident inputs (tables,
    lengths, start locations, block pairs) must meet, and the first one a
    batch breaks.

Sources (cited by key in every file):
  P1 = "Efficient Memory Management for Large Language Model Serving with
        PagedAttention" (paper review, urban-dandelion.tistory.com/4)
  P2 = "SOSP 2023論文解説: vLLM — PagedAttentionによるKVキャッシュメモリ管理の
        革新" (0h-n0.github.io/posts/conf-vllm-pagedattention)
  P3 = "연속 배치 처리 아키텍처" (Transformers docs, continuous batching
        architecture)

Every function here is pinned by the `-m "not gpu"` tests against something
other than itself (brute force, a library routine, closed forms, invariants,
the figures the pages print); see tests/test_oracle_*.py.
"""

from .attention import gather_context, attend, paged_attention, paged_attention_seq  # noqa: F401
from .kv_ops import write_kv, copy_blocks, swap_blocks  # noqa: F401
from .sizes import kv_bytes_per_token, block_bytes  # noqa: F401
from . import preconditions  # noqa: F401
