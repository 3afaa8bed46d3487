"""Pins for oracle.append (CPU only): rows land at the slots of [P3]'s worked
table, converted as the cache format says, and nothing else in the pool moves."""
import json
import os

import numpy as np

from oracle import append, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_table_example.json")


def _example():
    with open(GOLDEN) as f:
        return json.load(f)


def test_rows_land_on_worked_slots_and_nothing_else_changes():
    ex = _example()
    bs = ex["block_size"]
    rng = np.random.default_rng(0)
    NB, Hkv, d = 8, 2, 4
    kc = rng.standard_normal((NB, Hkv, bs, d)).astype(np.float16)
    vc = rng.standard_normal((NB, Hkv, bs, d)).astype(np.float16)
    slots = np.array([s["slot"] for s in ex["slots"]] + [-1], dtype=np.int64)
    T = len(slots)
    kn = rng.standard_normal((T, Hkv, d)).astype(np.float16)
    vn = rng.standard_normal((T, Hkv, d)).astype(np.float16)
    k2, v2, _, _ = append.append_expected(kc, vc, kn, vn, slots, bs, "f16")
    touched = np.zeros((NB, bs), dtype=bool)
    for i, s in enumerate(ex["slots"]):
        assert np.array_equal(k2[s["physical"], :, s["offset"]], kn[i])
        assert np.array_equal(v2[s["physical"], :, s["offset"]], vn[i])
        touched[s["physical"], s["offset"]] = True
    by_slot = lambda a: a.transpose(0, 2, 1, 3)   # [NB][bs][Hkv][d]
    assert np.array_equal(by_slot(k2)[~touched], by_slot(kc)[~touched])   # the -1 slot wrote nothing
    assert np.array_equal(by_slot(v2)[~touched], by_slot(vc)[~touched])


def test_int8_append_quantizes_each_row_and_writes_its_scale():
    rng = np.random.default_rng(1)
    NB, Hkv, bs, d = 4, 3, 16, 32
    kc = rng.integers(-128, 128, (NB, Hkv, bs, d)).astype(np.int8)
    vc = rng.integers(-128, 128, (NB, Hkv, bs, d)).astype(np.int8)
    ks = rng.standard_normal((NB, Hkv, bs)).astype(np.float32)
    vs = rng.standard_normal((NB, Hkv, bs)).astype(np.float32)
    kn = rng.standard_normal((2, Hkv, d)).astype(np.float16)
    vn = rng.standard_normal((2, Hkv, d)).astype(np.float16)
    slots = np.array([2 * bs + 5, 0], dtype=np.int64)
    k2, v2, ks2, vs2 = append.append_expected(kc, vc, kn, vn, slots, bs, "i8", ks, vs)
    for i, (blk, off) in enumerate([(2, 5), (0, 0)]):
        q, s = quant.quantize_int8_rows(kn[i].astype(np.float32))
        assert np.array_equal(k2[blk, :, off], q) and np.array_equal(ks2[blk, :, off], s)
        q, s = quant.quantize_int8_rows(vn[i].astype(np.float32))
        assert np.array_equal(v2[blk, :, off], q) and np.array_equal(vs2[blk, :, off], s)
    mask = np.ones((NB, bs), dtype=bool)
    mask[2, 5] = mask[0, 0] = False
    assert np.array_equal(k2.transpose(0, 2, 1, 3)[mask], kc.transpose(0, 2, 1, 3)[mask])
    assert np.array_equal(ks2.transpose(0, 2, 1)[mask], ks.transpose(0, 2, 1)[mask])


def test_fp8_append_uses_the_given_tensor_scale():
    rng = np.random.default_rng(2)
    NB, Hkv, bs, d = 2, 1, 16, 16
    kc = np.zeros((NB, Hkv, bs, d), dtype=np.uint8)
    vc = np.zeros((NB, Hkv, bs, d), dtype=np.uint8)
    kn = (rng.standard_normal((1, Hkv, d)) * 4).astype(np.float32)
    vn = (rng.standard_normal((1, Hkv, d)) * 4).astype(np.float32)
    s = np.float32(0.01)   # small: most values saturate at 448
    k2, v2, _, _ = append.append_expected(kc, vc, kn, vn, [17], bs, "fp8", s, s)
    want, _ = quant.quantize_fp8(kn[0, 0], scale=s)
    assert np.array_equal(k2[1, 0, 1], want)
    assert np.any((want & 0x7F) == 0x7E)


def test_int4_append_quantizes_packs_and_writes_the_scale():
    rng = np.random.default_rng(3)
    NB, Hkv, bs, d = 3, 2, 16, 32
    kc = rng.integers(0, 256, (NB, Hkv, bs, d // 2)).astype(np.uint8)
    vc = rng.integers(0, 256, (NB, Hkv, bs, d // 2)).astype(np.uint8)
    ks = rng.standard_normal((NB, Hkv, bs)).astype(np.float32)
    vs = rng.standard_normal((NB, Hkv, bs)).astype(np.float32)
    kn = rng.standard_normal((1, Hkv, d)).astype(np.float16)
    vn = rng.standard_normal((1, Hkv, d)).astype(np.float16)
    k2, v2, ks2, vs2 = append.append_expected(kc, vc, kn, vn, [bs + 9], bs, "i4", ks, vs)
    q, s = quant.quantize_int4_rows(kn[0].astype(np.float32))
    assert np.array_equal(k2[1, :, 9], quant.pack_int4(q)) and np.array_equal(ks2[1, :, 9], s)
    q, s = quant.quantize_int4_rows(vn[0].astype(np.float32))
    assert np.array_equal(v2[1, :, 9], quant.pack_int4(q)) and np.array_equal(vs2[1, :, 9], s)
    mask = np.ones((NB, bs), dtype=bool)
    mask[1, 9] = False
    assert np.array_equal(k2.transpose(0, 2, 1, 3)[mask], kc.transpose(0, 2, 1, 3)[mask])
