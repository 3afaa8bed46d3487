"""Multi-token queries over the paged cache (TEST INFRASTRUCTURE ONLY; see the package header).

A step that brings several new tokens per sequence at once — a chunk of a long
prompt (chunked prefill) or the draft tokens a verifier checks — attends
through the same block tables ([P3], PagedAttention section: the kernel finds
the physical blocks through the table and runs standard attention over the
stitched cache).  The pages show only the one-token decode; the reading taken
here is the usual causal one:

* the new tokens' K/V rows are written to the cache first, so ``context_lens[b]``
  counts them;
* query token ``j`` of the ``L_b`` new tokens of sequence ``b`` sits at position
  ``p = context_lens[b] - L_b + j`` and attends to positions ``0 .. p``
  (causal: a token never sees the tokens after it);
* query head ``h`` reads KV head ``h // G`` as in decode;
* a row with ``p < 0`` (more new tokens than cached ones, which callers must
  not send) attends to nothing and is defined as zeros.

Queries are packed: ``q[T][Hq][d]`` with sequence ``b``'s rows at
``q_start[b] .. q_start[b] + L_b``.
"""

import numpy as np

from . import paging, widen
from .attention import attend, kv_head_of, validate_tables


def _dequant(cache, scale, bt_row, ctx, bs, g, fmt):
    raw = paging.gather(cache, bt_row, ctx, bs, g)
    if fmt in ("i8", "i4"):
        s = paging.gather_scales(np.asarray(scale), bt_row, ctx, bs, g)
        return widen.widen_kv(raw, fmt, s)
    if fmt == "fp8":
        return widen.widen_kv(raw, "fp8", scale)
    return widen.widen_kv(raw, fmt)


def multi_query_attention(q, q_lens, k_cache, v_cache, block_tables, context_lens, scale,
                          block_size, kv_format, k_scale=None, v_scale=None, rows=None,
                          check_tables=True):
    """Output ``[T][Hq][d]`` (fp64).  ``q_lens[b]`` new tokens per sequence, packed in
    sequence order.  ``rows``: optional iterable of (token row, head) to compute (the
    rest stay NaN)."""
    q = np.asarray(q, dtype=np.float64)
    T, Hq, d = q.shape
    NB, Hkv, bs, dk = k_cache.shape
    if bs != block_size or dk * (2 if kv_format == "i4" else 1) != d:
        raise ValueError("cache shape does not match block_size / head_dim")
    lens = np.asarray(q_lens, dtype=np.int64)
    if lens.sum() != T or np.any(lens < 0):
        raise ValueError("q_lens must be non-negative and sum to the query rows")
    if check_tables:
        validate_tables(block_tables, context_lens, NB, block_size)
    bt = np.asarray(block_tables)
    ctx_all = np.asarray(context_lens)
    starts = np.concatenate([[0], np.cumsum(lens)])
    wanted = None if rows is None else set((int(r), int(h)) for r, h in rows)
    out = np.zeros((T, Hq, d)) if wanted is None else np.full((T, Hq, d), np.nan)
    for b in range(len(lens)):
        L, ctx = int(lens[b]), int(ctx_all[b])
        for g in range(Hkv):
            heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g]
            todo = [(j, h) for j in range(L) for h in heads
                    if wanted is None or (int(starts[b]) + j, h) in wanted]
            if not todo:
                continue
            K = _dequant(k_cache, k_scale, bt[b], ctx, block_size, g, kv_format) if ctx else None
            V = _dequant(v_cache, v_scale, bt[b], ctx, block_size, g, kv_format) if ctx else None
            for j, h in todo:
                r = int(starts[b]) + j
                p = ctx - L + j
                if p < 0:
                    out[r, h] = 0.0
                else:
                    out[r, h] = attend(q[r, h], K[:p + 1], V[:p + 1], scale)
    return out
