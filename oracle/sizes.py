"""Oracle: KV-cache byte counts — TEST INFRASTRUCTURE ONLY.

[P2 "LLM推論のメモリボトルネック"]: one token's cache holds a key and a value
vector for every layer and head, so it takes 2 * layers * heads * head_dim *
bytes-per-element bytes.
[P2 "PagedAttentionの仕組み", block structure]: a block of B tokens takes B
times that.
"""


def kv_bytes_per_token(num_layers: int, num_heads: int, head_dim: int, elt_bytes: int) -> int:
    return 2 * num_layers * num_heads * head_dim * elt_bytes


def block_bytes(num_layers: int, num_heads: int, head_dim: int, block_size: int,
                elt_bytes: int) -> int:
    return block_size * kv_bytes_per_token(num_layers, num_heads, head_dim, elt_bytes)
