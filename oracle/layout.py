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
