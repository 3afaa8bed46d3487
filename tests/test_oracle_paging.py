"""Pins for oracle.paging: the worked block tables of [P3] (tests/golden/block_table_example.json)."""
import json
import os

import numpy as np

from oracle import paging

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_table_example.json")


def _example():
    with open(GOLDEN) as f:
        return json.load(f)


def test_slots_of_worked_tables():
    ex = _example()
    bs = ex["block_size"]
    for s in ex["slots"]:
        row = ex["block_tables"][s["seq"]]
        assert paging.slot_of(row, s["position"], bs) == s["slot"]
        assert paging.block_and_offset(s["slot"], bs) == (s["physical"], s["offset"])


def _tagged_pool(num_blocks, kv_heads, bs, width):
    """Pool whose every element encodes (physical block, head, offset, lane)."""
    pool = np.zeros((num_blocks, kv_heads, bs, width), dtype=np.float64)
    for p in range(num_blocks):
        for g in range(kv_heads):
            for o in range(bs):
                pool[p, g, o] = p * 1e6 + g * 1e4 + o * 1e2 + np.arange(width)
    return pool


def test_gather_walks_the_table_in_logical_order():
    ex = _example()
    bs = ex["block_size"]
    pool = _tagged_pool(8, 2, bs, 3)
    for name, row in ex["block_tables"].items():
        ctx = 3 * bs - 5  # ragged last block
        for g in range(2):
            got = paging.gather(pool, row, ctx, bs, g)
            assert got.shape == (ctx, 3)
            for pos in range(ctx):
                phys, off = row[pos // bs], pos % bs
                assert got[pos, 0] == phys * 1e6 + g * 1e4 + off * 1e2


def test_gather_scales_matches_gather():
    rng = np.random.default_rng(0)
    scales = rng.standard_normal((8, 2, 16)).astype(np.float32)
    row = [5, 1, 6]
    for ctx in (1, 16, 17, 40):
        a = paging.gather_scales(scales, row, ctx, 16, 1)
        b = paging.gather(scales[..., None], row, ctx, 16, 1)[:, 0]
        assert np.array_equal(a, b)


def test_two_sequences_never_share_a_physical_block():
    ex = _example()
    a, b = ex["block_tables"]["A"], ex["block_tables"]["B"]
    assert not set(a) & set(b)
