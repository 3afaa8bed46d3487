"""Paged decode attention, by definition (TEST INFRASTRUCTURE ONLY; see the package header).

What is computed, step by step, in the pages' order:

1. Check the block tables ([P1] §2, [P3] paging section): every logical block a
   sequence uses maps to a physical block of the pool, and no physical block is
   held by two live logical blocks.
2. Locate each sequence's rows through its block table and stitch them into a
   contiguous cache ([P3]: the kernel indexes the physical blocks through the
   table and stitches the scattered K/V together).
3. Dequantize the stitched rows to float64 (INT8 per [P1] §4, FP8 per [P2] §4 /
   [P3]; see ``widen``).
4. Run standard attention for the one new query token ([P3]: "standard
   attention" after the stitch).  The pages show the grouping but not the
   softmax: [P1] §3's group_query_attention example reshapes the query heads into
   ``n_heads // group_size`` groups of ``group_size`` and has no softmax or
   1/sqrt(d); taken here as scaled softmax attention where query head ``h`` reads
   KV head ``h // G`` (G = Hq / Hkv), so MHA (G = 1), GQA-g and MQA (Hkv = 1)
   are one rule.  ``scale`` is the caller's softmax scale (1/sqrt(d) in use).

A sequence with ``context_len == 0`` attends to nothing; its output is defined
as zeros (the pages never meet this case).
"""

import numpy as np

from . import paging, widen


def validate_tables(block_tables, context_lens, num_blocks, block_size):
    """Step 1.  Raises ValueError on a table the method cannot use."""
    bt = np.asarray(block_tables)
    ctx = np.asarray(context_lens)
    if bt.ndim != 2 or ctx.ndim != 1 or bt.shape[0] != ctx.shape[0]:
        raise ValueError("block_tables is [B][MB] and context_lens is [B]")
    max_tokens = bt.shape[1] * block_size
    seen = set()
    for b in range(bt.shape[0]):
        c = int(ctx[b])
        if c < 0 or c > max_tokens:
            raise ValueError(f"context_lens[{b}] = {c} outside [0, {max_tokens}]")
        for j in range(-(-c // block_size)):
            p = int(bt[b, j])
            if p < 0 or p >= num_blocks:
                raise ValueError(f"block_tables[{b}][{j}] = {p} not in [0, {num_blocks})")
            if p in seen:
                raise ValueError(f"physical block {p} is used twice")
            seen.add(p)


def kv_head_of(h, num_q_heads, num_kv_heads):
    """KV head read by query head ``h``: [P1] §3 views the query heads as
    ``num_q_heads // G`` consecutive groups of ``G = num_q_heads // num_kv_heads``."""
    return h // (num_q_heads // num_kv_heads)


def attend(q_vec, K, V, scale, return_weights=False):
    """Standard scaled softmax attention of one query row over ``K``/``V`` rows (fp64).

    z_t = scale * <q, K_t>;  w = softmax(z);  o = sum_t w_t V_t.
    """
    q_vec = np.asarray(q_vec, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    z = scale * (K @ q_vec)
    m = np.max(z)
    p = np.exp(z - m)
    w = p / np.sum(p)
    o = w @ V
    if return_weights:
        return o, w
    return o


def decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale,
                     block_size, kv_format, k_scale=None, v_scale=None,
                     check_tables=True, pairs=None, return_weights=False):
    """Output ``[B][Hq][d]`` (fp64) of one decode step.

    q            [B][Hq][d], any real dtype (widened exactly to fp64 by the caller
                 or here; pass bf16 already widened).
    k_cache      [NB][Hkv][bs][d] stored K: float32 / float16 / uint16 (bf16 bits)
                 / int8 / uint8 (fp8 codes), per ``kv_format``; for ``i4``
                 [NB][Hkv][bs][d/2] packed bytes; v_cache alike.
    k_scale      i8 / i4: float32 [NB][Hkv][bs] (127 or 7 over absmax per row);
                 fp8: one float.
    block_tables int [B][MB];  context_lens int [B].
    pairs        optional iterable of (b, h) to compute (the rest stay NaN), for
                 sampled checks of large cases.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    NB, Hkv, bs, dk = k_cache.shape
    if bs != block_size or dk * (2 if kv_format == "i4" else 1) != d:
        raise ValueError("cache shape does not match block_size / head_dim")
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    if check_tables:
        validate_tables(block_tables, context_lens, NB, block_size)
    bt = np.asarray(block_tables)
    ctx_all = np.asarray(context_lens)

    if pairs is None:
        out = np.zeros((B, Hq, d), dtype=np.float64)
        wanted = {(b, h) for b in range(B) for h in range(Hq)}
    else:
        out = np.full((B, Hq, d), np.nan, dtype=np.float64)
        wanted = set((int(b), int(h)) for b, h in pairs)
    weights = {}

    for b in range(B):
        ctx = int(ctx_all[b])
        for g in range(Hkv):
            heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g and (b, h) in wanted]
            if not heads:
                continue
            if ctx == 0:
                for h in heads:
                    out[b, h] = 0.0
                continue
            # Step 2: stitch through the block table.
            Kraw = paging.gather(k_cache, bt[b], ctx, block_size, g)
            Vraw = paging.gather(v_cache, bt[b], ctx, block_size, g)
            # Step 3: dequantize.
            if kv_format in ("i8", "i4"):
                ks = paging.gather_scales(np.asarray(k_scale), bt[b], ctx, block_size, g)
                vs = paging.gather_scales(np.asarray(v_scale), bt[b], ctx, block_size, g)
                K = widen.widen_kv(Kraw, kv_format, ks)
                V = widen.widen_kv(Vraw, kv_format, vs)
            elif kv_format == "fp8":
                K = widen.widen_kv(Kraw, "fp8", k_scale)
                V = widen.widen_kv(Vraw, "fp8", v_scale)
            else:
                K = widen.widen_kv(Kraw, kv_format)
                V = widen.widen_kv(Vraw, kv_format)
            # Step 4: query head h reads KV head h // G.
            for h in heads:
                if return_weights:
                    out[b, h], weights[(b, h)] = attend(q[b, h], K, V, scale, True)
                else:
                    out[b, h] = attend(q[b, h], K, V, scale)
    if return_weights:
        return out, weights
    return out


def contiguous_attention(q, K, V, scale):
    """Decode attention on an unpaged cache: K, V are ``[B][Hkv][T][d]`` with every
    sequence ``T`` long — the static layout paging replaces ([P1] §2, [P3])."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            out[b, h] = attend(q[b, h], K[b, kv_head_of(h, Hq, Hkv)], V[b, kv_head_of(h, Hq, Hkv)],
                               scale)
    return out
