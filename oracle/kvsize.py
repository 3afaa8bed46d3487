"""Closed-form KV-cache sizes (TEST INFRASTRUCTURE ONLY; see the package header).

Three pages write the same count three ways:

* [P2] §2 (estimating KV-cache memory): two tensors (K and V) times batch, sequence
  length, layers, KV heads, head dimension and bytes per element.
* [P1] §1 (KV Cache principle and memory analysis): two times layers, hidden size,
  sequence length and element size; for multi-head attention the hidden size is
  the number of KV heads times the head dimension.
* [P3] (bottleneck analysis section): two times layers, heads, head dimension,
  sequence length, batch and bytes.

All arithmetic is exact Python integers.
"""


def kv_cache_bytes(batch, seq_len, layers, kv_heads, head_dim, dtype_bytes):
    """Bytes of K plus V for ``batch`` sequences of ``seq_len`` tokens ([P2] §2)."""
    for v in (batch, seq_len, layers, kv_heads, head_dim, dtype_bytes):
        if int(v) != v or v < 0:
            raise ValueError("kv_cache_bytes takes non-negative integers")
    return 2 * int(batch) * int(seq_len) * int(layers) * int(kv_heads) * int(head_dim) \
        * int(dtype_bytes)


def kv_cache_bytes_hidden(layers, hidden_size, seq_len, dtype_bytes, batch=1):
    """The hidden-size spelling of the same count ([P1] §1), MHA only."""
    return 2 * int(layers) * int(hidden_size) * int(seq_len) * int(dtype_bytes) * int(batch)


def paged_pool_bytes(num_blocks, block_size, kv_heads, head_dim, dtype_bytes, layers=1):
    """Bytes of a paged K+V pool: ``num_blocks`` blocks of ``block_size`` token slots
    per KV head, for each layer ([P1] §2 and [P3]: the cache is cut into fixed-size
    blocks)."""
    return 2 * int(layers) * int(num_blocks) * int(block_size) * int(kv_heads) \
        * int(head_dim) * int(dtype_bytes)


def blocks_needed(seq_len, block_size):
    """Logical blocks a sequence of ``seq_len`` tokens occupies: the ceiling of the
    ratio, since blocks are fixed-size and allocated whole ([P3], paging section)."""
    return -(-int(seq_len) // int(block_size))
