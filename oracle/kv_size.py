"""KV-cache size closed form (oracle; test infrastructure only).

[Inside engines] "The KV Cache: Mathematical Formulation & Memory Footprint",
[KV essay] "What the cache costs", [KV management] (size formula) and
[InferScale] (per-fact storage cost) all state the same product: one K tensor
and one V tensor (the factor 2) per layer, per KV head, per head dimension, per
stored element byte, per token.
"""


def kv_bytes(n_layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int,
             n_tokens: int) -> int:
    """Exact byte count of K plus V for ``n_tokens`` tokens (Python ints)."""
    for v in (n_layers, n_kv_heads, head_dim, elem_bytes, n_tokens):
        if int(v) != v or v < 0:
            raise ValueError("kv_bytes takes non-negative integers")
    return 2 * int(n_layers) * int(n_kv_heads) * int(head_dim) * int(elem_bytes) * int(n_tokens)


def paged_pool_bytes(n_layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int,
                     n_tokens: int, block_tokens: int = 16) -> int:
    """Bytes a paged cache holds for one sequence of ``n_tokens``: whole blocks.

    [KV essay] "Paged attention": only the last block can be partly empty, so
    the sequence occupies ceil(n / block) blocks of ``block_tokens`` slots.
    """
    n_blocks = -(-int(n_tokens) // int(block_tokens))
    return kv_bytes(n_layers, n_kv_heads, head_dim, elem_bytes, n_blocks * int(block_tokens))
