"""Storage order of the cache pools (TEST INFRASTRUCTURE ONLY; see the package header).

The pools keep the ``[NB][Hkv][bs][d]`` shape, and the oracle reasons about
them in that logical order: row ``t`` of block ``b``, head ``g`` is token ``t``'s
vector.  The library stores each group of 16 consecutive rows of a (block,
head) tile in a different order of the same bytes (its format definition,
``include/pagedkv.h``); the functions here turn stored pools back into the
logical order (and the reverse), written from that definition with numpy
reshapes.  They move bytes only.

Inside one 16-row group, with ``eb`` bytes per element and rows of ``d``
elements:

* K: the row of token ``t`` is cut into 16-byte chunks; chunk ``c`` of token
  ``t`` is stored at byte ``(c * 16 + t) * 16``.
* V: element ``(t, d)`` with ``n = d // 16``, ``r = d % 16``, ``c = t // 4``,
  ``i = t % 4`` and ``G = 4 // eb`` is stored at byte
  ``((n // G) * 64 + c * 16 + r) * 16 + ((n % G) * 4 + i) * eb``.
"""

import numpy as np


def _groups(stored):
    """View a pool ``[NB][Hkv][bs][d]`` as ``[NB][Hkv][bs/16][16 * d]`` elements."""
    a = np.asarray(stored)
    NB, Hkv, bs, d = a.shape
    if bs % 16:
        raise ValueError("block_size must be a multiple of 16")
    return a.reshape(NB, Hkv, bs // 16, 16 * d), (NB, Hkv, bs, d)


def k_from_stored(stored):
    """Stored K pool -> logical ``[NB][Hkv][bs][d]`` (same dtype)."""
    g, (NB, Hkv, bs, d) = _groups(stored)
    eb = g.dtype.itemsize
    per_chunk = 16 // eb
    x = g.reshape(NB, Hkv, bs // 16, (d * eb) // 16, 16, per_chunk)   # [chunk][token][elem]
    x = x.transpose(0, 1, 2, 4, 3, 5)                                 # [token][chunk][elem]
    return np.ascontiguousarray(x).reshape(NB, Hkv, bs, d)


def v_from_stored(stored):
    """Stored V pool -> logical ``[NB][Hkv][bs][d]`` (same dtype)."""
    g, (NB, Hkv, bs, d) = _groups(stored)
    eb = g.dtype.itemsize
    G = 4 // eb
    # element index = (((n // G) * 4 + c) * 16 + r) * (4 G) + (n % G) * 4 + i
    x = g.reshape(NB, Hkv, bs // 16, d // (16 * G), 4, 16, G, 4)      # [nq][c][r][nm][i]
    x = x.transpose(0, 1, 2, 4, 7, 3, 6, 5)                           # [c][i][nq][nm][r]
    return np.ascontiguousarray(x).reshape(NB, Hkv, bs, d)


def k_to_stored(logical):
    """Logical K pool -> stored order (inverse of ``k_from_stored``)."""
    g, (NB, Hkv, bs, d) = _groups(logical)
    eb = g.dtype.itemsize
    per_chunk = 16 // eb
    x = g.reshape(NB, Hkv, bs // 16, 16, (d * eb) // 16, per_chunk).transpose(0, 1, 2, 4, 3, 5)
    return np.ascontiguousarray(x).reshape(NB, Hkv, bs, d)


def v_to_stored(logical):
    """Logical V pool -> stored order (inverse of ``v_from_stored``)."""
    g, (NB, Hkv, bs, d) = _groups(logical)
    eb = g.dtype.itemsize
    G = 4 // eb
    x = g.reshape(NB, Hkv, bs // 16, 4, 4, d // (16 * G), G, 16)     # [c][i][nq][nm][r]
    x = x.transpose(0, 1, 2, 5, 3, 7, 6, 4)                           # [nq][c][r][nm][i]
    return np.ascontiguousarray(x).reshape(NB, Hkv, bs, d)


# ---------------------------------------------------------------------------
# INT4 pools hold packed bytes ``[NB][Hkv][bs][d/2]`` (logical order: element
# 2k of a row in the low nibble of byte k, 2k+1 in the high nibble).
#
# * K: the packed row is cut into 16-byte chunks exactly as above (the
#   functions above apply to the packed uint8 array unchanged).
# * V: nibbles move, not just bytes.  With ``n = d // 16``, ``r = d % 16``,
#   ``c = t // 4``, ``i = t % 4``, element ``(t, d)`` sits in byte
#   ``((n // 8) * 64 + c * 16 + r) * 16 + ((n % 8) // 2) * 4 + i`` of the group,
#   low nibble for even ``n``, high for odd: each stored byte holds token
#   ``t``'s elements ``d`` and ``d + 16``.  ``d`` must be a multiple of 128.
# ---------------------------------------------------------------------------
def _nibbles(packed):
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2], out[..., 1::2] = b & 0xF, b >> 4
    return out


def _pack(nibbles):
    n = np.asarray(nibbles, dtype=np.uint8)
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def _v4_shape(packed):
    a = np.asarray(packed)
    if a.dtype != np.uint8:
        raise TypeError("int4 pools are packed uint8")
    NB, Hkv, bs, half = a.shape
    d = 2 * half
    if bs % 16 or d % 128:
        raise ValueError("int4 V needs block_size % 16 == 0 and head_dim % 128 == 0")
    return NB, Hkv, bs, d


def v4_from_stored(stored):
    """Stored INT4 V pool -> logical packed ``[NB][Hkv][bs][d/2]``."""
    NB, Hkv, bs, d = _v4_shape(stored)
    # nibble index in a group = (((nq*4 + c)*16 + r)*16 + nw*4 + i)*2 + np,
    # with n = 8*nq + 2*nw + np
    x = _nibbles(stored).reshape(NB, Hkv, bs // 16, d // 128, 4, 16, 4, 4, 2)  # nq c r nw i np
    x = x.transpose(0, 1, 2, 4, 7, 3, 6, 8, 5)                                # c i nq nw np r
    return _pack(np.ascontiguousarray(x).reshape(NB, Hkv, bs, d))


def v4_to_stored(logical):
    """Logical packed INT4 V pool -> stored order (inverse of ``v4_from_stored``)."""
    NB, Hkv, bs, d = _v4_shape(logical)
    x = _nibbles(logical).reshape(NB, Hkv, bs // 16, 4, 4, d // 128, 4, 2, 16)  # c i nq nw np r
    x = x.transpose(0, 1, 2, 5, 3, 8, 6, 4, 7)                                 # nq c r nw i np
    return _pack(np.ascontiguousarray(x).reshape(NB, Hkv, bs, d))
