"""Expected cache after appending new tokens (TEST INFRASTRUCTURE ONLY; see the package header).

[P3] (paging section): blocks are taken on demand and each new token's K/V row
goes to the slot its sequence's block table gives.  The new token of row ``i``
carries a pool slot ``slot[i] = physical * bs + offset``; a negative slot means
"no write".  Each KV head's row is written at ``cache[slot // bs][head][slot % bs]``,
converted to the cache's storage:

* same float format: copied;
* INT8 / INT4: quantized per row ([P1] §4; INT4 with 7 for 127, packed two
  per byte), its scale written at the same position of the scale array;
* FP8: encoded with the tensor's existing scale (saturating at +-448).

Everything else in the pool is left as it was, byte for byte.
"""

import numpy as np

from . import paging, quant, widen


def append_expected(k_cache, v_cache, k_new, v_new, slot_mapping, block_size,
                    kv_format, k_scale=None, v_scale=None, src_format=None):
    """Return ``(k_cache', v_cache', k_scale', v_scale')`` as new arrays.

    k_new, v_new: ``[T][Hkv][d]`` sources in ``src_format`` storage (float32,
    float16, or uint16 bf16 bits).  For a plain float cache the source must have
    the cache's storage dtype and is copied bit for bit.  For ``i8`` the scale
    arrays are ``[NB][Hkv][bs]``; for ``fp8`` they are scalars (read, returned
    unchanged).
    """
    if kv_format in ("i8", "fp8", "i4"):
        fmt = src_format or {np.dtype(np.float16): "f16", np.dtype(np.uint16): "bf16",
                             np.dtype(np.float32): "f32"}[np.asarray(k_new).dtype]
        k_new = widen.widen_plain(k_new, fmt).astype(np.float32)
        v_new = widen.widen_plain(v_new, fmt).astype(np.float32)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    ks = None if k_scale is None else np.array(k_scale, copy=True)
    vs = None if v_scale is None else np.array(v_scale, copy=True)
    T, Hkv, d = np.asarray(k_new).shape
    for i in range(T):
        slot = int(slot_mapping[i])
        if slot < 0:
            continue
        blk, off = paging.block_and_offset(slot, block_size)
        for g in range(Hkv):
            for src, cache, scales, given in ((k_new, kc, ks, k_scale), (v_new, vc, vs, v_scale)):
                row = np.asarray(src)[i, g]
                if kv_format == "i8":
                    q, s = quant.quantize_int8_rows(row[None, :])
                    cache[blk, g, off] = q[0]
                    scales[blk, g, off] = s[0]
                elif kv_format == "i4":
                    q, s = quant.quantize_int4_rows(row[None, :])
                    cache[blk, g, off] = quant.pack_int4(q)[0]
                    scales[blk, g, off] = s[0]
                elif kv_format == "fp8":
                    codes, _ = quant.quantize_fp8(row, scale=given)
                    cache[blk, g, off] = codes
                else:
                    if row.dtype != cache.dtype:
                        raise TypeError("plain-format append copies the cache's own dtype")
                    cache[blk, g, off] = row
    return kc, vc, ks, vs
