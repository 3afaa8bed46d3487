"""Host logic of the input generator: block tables, slots and poison masks
(checked against oracle.paging, which shares no code with it)."""
import numpy as np
import torch
import pytest

from oracle import kvsize, paging
from harness import workloads as W


@pytest.mark.parametrize("name", W.NAMES)
def test_tables_are_valid_and_disjoint(name):
    w = W.make(name)
    used = []
    for b in range(w.batch):
        n = kvsize.blocks_needed(int(w.context_lens[b]), w.block_size)
        row = w.block_tables[b]
        assert np.all(row[:n] >= 0) and np.all(row[:n] < w.num_blocks)
        assert np.all(row[n:] == -1)
        used.extend(row[:n].tolist())
    assert len(used) == len(set(used))
    assert w.num_blocks >= len(used)


def test_published_shapes():
    w = W.make("llama70b_gqa8")
    assert (w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size) == (32, 64, 8, 128, 16)
    assert w.context_lens.min() >= 512 and w.context_lens.max() <= 32768
    assert int(w.context_lens.sum()) == 560359 and w.num_blocks == 43798
    assert w.kv_bytes_per_layer() == 2 * 560359 * 8 * 128 * 2
    c = W.make("llama13b_int8")
    assert np.all(c.context_lens == 2049) and c.num_blocks == 5160
    f = W.make("llama70b_fp8")
    assert f.layers == 80 and f.context_lens.min() >= 128 and f.context_lens.max() <= 32768
    assert W.make("llama70b_fp8", block_size=256).num_blocks == 2087
    i4 = W.make("llama70b_int4")
    assert i4.kv_format == "i4" and np.array_equal(i4.context_lens, w.context_lens)
    # packed nibbles plus one float32 scale per row
    assert i4.kv_bytes_per_layer() == 2 * 560359 * 8 * (128 // 2 + 4)
    assert W.make("llama13b_int4").kv_format == "i4"
    # every context at 32K: 2048 blocks per sequence, a pool past 2**31 bytes per cache
    f = W.make("llama70b_gqa8_32k")
    assert np.all(f.context_lens == 32768) and f.num_blocks == 81920
    assert f.num_blocks * f.num_kv_heads * f.block_size * f.head_dim * 2 > 2**31
    assert f.kv_bytes_per_layer() == 2 * 32 * 32768 * 8 * 128 * 2 == 4 * 2**30


@pytest.mark.parametrize("name", W.NAMES)
def test_every_workload_names_a_known_format(name):
    from oracle import widen
    assert W.make(name).kv_format in widen.FORMATS


@pytest.mark.parametrize("name", ["llama7b_bf16", "llama13b_int8", "llama70b_fp8"])
def test_append_slots_match_oracle_slot_arithmetic(name):
    w = W.make(name)
    got = w.append_slots()
    for b in range(w.batch):
        assert got[b] == paging.slot_of(w.block_tables[b], int(w.context_lens[b]) - 1, w.block_size)


def test_empty_sequences_append_nowhere():
    """An empty sequence's append slot is -1 and poisons no pool slot.  Two empty
    and two 48-token sequences fill a pool of exactly 6 blocks, so the poisoned
    slots are the two appended ones and nothing else (a -1 taken as an index
    would poison slot 15 of the pool's last block, a live middle block here)."""
    from harness.device_cache import poison_mask
    w = W.custom(torch.float16, "i4", [0, 48, 0, 48], 2, 1, 128, 16,
                 pool_factor=1.0, perm_seed=1, appends=True)
    assert w.num_blocks == 6 and w.block_tables[3, 1] == w.num_blocks - 1
    slots = w.append_slots()
    assert slots[0] == -1 and slots[2] == -1 and np.all(slots[[1, 3]] >= 0)
    m = poison_mask(w)
    assert m.sum() == 2 and m[slots[1] // 16, slots[1] % 16] and m[slots[3] // 16, slots[3] % 16]


def test_unused_mask_counts_live_slots():
    w = W.make("tiny_fp32")
    m = W.unused_slot_mask(w)
    assert (~m).sum() == int(w.context_lens.sum())
    for b in range(w.batch):
        for pos in range(int(w.context_lens[b])):
            blk, off = paging.block_and_offset(paging.slot_of(w.block_tables[b], pos, 16), 16)
            assert not m[blk, off]


def test_pool_too_small_is_refused():
    with pytest.raises(ValueError):
        W.deal_blocks([64, 64], 16, 7)
