"""Pins for oracle.kvsize: the KV-size figures the pages print (tests/golden/kv_size_points.json)."""
import json
import os

import pytest

from oracle import kvsize

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_size_points.json")


def _points():
    with open(GOLDEN) as f:
        return json.load(f)


def test_exact_points():
    for p in _points()["exact"]:
        got = kvsize.kv_cache_bytes(p["batch"], p["seq_len"], p["layers"], p["kv_heads"],
                                    p["head_dim"], p["dtype_bytes"])
        assert got == p["bytes"], p["cite"]
        assert round(got / 1e9, 2) == p["printed_gb"], p["cite"]


def test_lower_bounds():
    for p in _points()["lower_bounds"]:
        got = kvsize.kv_cache_bytes(p["batch"], p["seq_len"], p["layers"], p["kv_heads"],
                                    p["head_dim"], p["dtype_bytes"])
        assert got >= p["bytes_at_least"], p["cite"]
    # MHA (64 KV heads) is exactly 8x the GQA-8 figure.
    assert kvsize.kv_cache_bytes(1, 32768, 80, 64, 128, 2) == 8 * 10737418240 == 85899345920


def test_rounded_points():
    pts = _points()["rounded"]
    single = pts[0]
    got = kvsize.kv_cache_bytes_hidden(single["layers"], single["hidden_size"], single["seq_len"],
                                       single["dtype_bytes"], single["batch"])
    assert got == 2 ** 31
    assert round(got / 1e9, single["decimals"]) == single["printed_gb"]
    batch8 = pts[1]
    got8 = kvsize.kv_cache_bytes_hidden(batch8["layers"], batch8["hidden_size"], batch8["seq_len"],
                                        batch8["dtype_bytes"], batch8["batch"])
    assert got8 == 8 * got == 17179869184
    assert round(batch8["batch"] * batch8["printed_as_multiple_of_rounded"], 6) == batch8["printed_gb"]


def test_spellings_agree():
    # [P1] §1's hidden-size form equals [P2] §2's head form when hidden = kv_heads * head_dim (MHA).
    for layers, heads, d, seq, nbytes, batch in [(32, 32, 128, 4096, 2, 1), (40, 40, 128, 2048, 2, 32),
                                                 (80, 64, 128, 32768, 1, 3)]:
        assert kvsize.kv_cache_bytes_hidden(layers, heads * d, seq, nbytes, batch) == \
            kvsize.kv_cache_bytes(batch, seq, layers, heads, d, nbytes)


def test_paged_pool_has_no_tail_waste_when_blocks_divide():
    # The 70B / 32K sequence in 16-token or 256-token blocks occupies exactly the closed form.
    for bs in (16, 256):
        nb = kvsize.blocks_needed(32768, bs)
        assert nb * bs == 32768
        assert kvsize.paged_pool_bytes(nb, bs, 8, 128, 2, layers=80) == 10737418240


def test_blocks_needed_is_ceiling():
    assert kvsize.blocks_needed(37, 16) == 3
    assert kvsize.blocks_needed(64, 16) == 4
    assert kvsize.blocks_needed(2049, 16) == 129
    assert kvsize.blocks_needed(0, 16) == 0
    assert kvsize.blocks_needed(1, 256) == 1


def test_rejects_non_integers():
    with pytest.raises(ValueError):
        kvsize.kv_cache_bytes(1, 2.5, 1, 1, 1, 1)
