"""Block-table arithmetic and gather (TEST INFRASTRUCTURE ONLY; see the package header).

[P1] §2 (PageAttention): the KV cache is cut into fixed-size blocks, a block
table records which physical block holds each logical block, and attention finds
the stored rows through that table.  [P3] (PagedAttention memory management
section) gives the worked case: 16-token blocks, sequence A on physical blocks
0, 3, 7 and sequence B on 1, 2, 5; the kernel indexes the physical blocks through
the table and stitches the scattered K/V back together before ordinary
attention.

Cache layout taken here (the pages' Block holds ``[block_size, hidden]`` per
block with heads side by side; splitting the hidden axis into heads gives the
same numbers): ``cache[physical_block][kv_head][offset_in_block][head_dim]``.
A *slot* numbers the token positions of the pool: ``slot = physical * bs + offset``.
"""

import numpy as np


def slot_of(block_table_row, position, block_size):
    """Pool slot holding logical ``position`` of a sequence."""
    logical = position // block_size
    physical = int(block_table_row[logical])
    return physical * block_size + position % block_size


def block_and_offset(slot, block_size):
    """Inverse of ``slot_of``: the physical block and the offset inside it."""
    return slot // block_size, slot % block_size


def gather(cache, block_table_row, ctx, block_size, kv_head):
    """Stitch the first ``ctx`` token rows of one KV head back into logical order.

    ``cache`` is ``[NB][Hkv][bs][...]``; the result is ``[ctx][...]`` with the
    same dtype.  One logical block at a time, as the table lists them.
    """
    tail = cache.shape[3:]
    out = np.empty((ctx,) + tail, dtype=cache.dtype)
    n_logical = -(-ctx // block_size)
    for j in range(n_logical):
        physical = int(block_table_row[j])
        first = j * block_size
        count = min(block_size, ctx - first)
        out[first:first + count] = cache[physical, kv_head, :count]
    return out


def gather_scales(scales, block_table_row, ctx, block_size, kv_head):
    """Same walk for a per-slot scale array ``[NB][Hkv][bs]``."""
    out = np.empty((ctx,), dtype=scales.dtype)
    n_logical = -(-ctx // block_size)
    for j in range(n_logical):
        physical = int(block_table_row[j])
        first = j * block_size
        count = min(block_size, ctx - first)
        out[first:first + count] = scales[physical, kv_head, :count]
    return out
