"""Each pin must be able to fail.  These tests plant one plausible mistake at a
time in the oracle (on the CPU, through monkeypatch) and check that the pins in
the other oracle test files catch it."""
import numpy as np
import pytest

import oracle.attention as attention
import oracle.paging as paging
import oracle.quant as quant
import oracle.widen as widen
from tests import test_oracle_attention as TA
from tests import test_oracle_quant as TQ
from tests import test_oracle_paging as TP


def _fails(fn, *args):
    with pytest.raises((AssertionError, ValueError, IndexError)):
        fn(*args)


def test_wrong_grouping_is_caught(monkeypatch):
    # Interleaved grouping (h mod Hkv) instead of consecutive groups.
    monkeypatch.setattr(attention, "kv_head_of", lambda h, hq, hkv: h % hkv)
    _fails(TA.test_matches_torch_sdpa, 8, 2, 16)


def test_dropped_scale_is_caught(monkeypatch):
    orig = attention.attend
    monkeypatch.setattr(attention, "attend", lambda q, K, V, s, rw=False: orig(q, K, V, 1.0, rw))
    _fails(TA.test_matches_torch_sdpa, 4, 4, 16)


def test_unnormalised_softmax_is_caught(monkeypatch):
    def bad(q, K, V, s, rw=False):
        z = s * (np.asarray(K) @ np.asarray(q))
        w = np.exp(z - z.max())
        return (w @ np.asarray(V), w) if rw else w @ np.asarray(V)
    monkeypatch.setattr(attention, "attend", bad)
    _fails(TA.test_weights_sum_to_one)


def test_off_by_one_gather_is_caught(monkeypatch):
    def bad(cache, row, ctx, bs, g):
        out = np.empty((ctx,) + cache.shape[3:], dtype=cache.dtype)
        for pos in range(ctx):
            p = pos + 1 if pos + 1 < ctx else pos
            out[pos] = cache[int(row[p // bs]), g, p % bs]
        return out
    monkeypatch.setattr(paging, "gather", bad)
    _fails(TA.test_needles_pick_out_their_rows)


def test_transposed_block_offset_is_caught(monkeypatch):
    monkeypatch.setattr(paging, "slot_of", lambda row, pos, bs: int(row[pos % bs]) * bs + pos // bs)
    _fails(TP.test_slots_of_worked_tables)


def test_multiplying_dequant_is_caught(monkeypatch):
    orig = widen.widen_kv

    def bad(x, fmt, scale=None):
        if fmt == "i8":
            return np.asarray(x).astype(np.float64) * np.asarray(scale, dtype=np.float64)[..., None]
        return orig(x, fmt, scale)
    monkeypatch.setattr(widen, "widen_kv", bad)
    _fails(TA.test_int8_cache_stays_within_quantization_error)


def test_round_half_away_is_caught(monkeypatch):
    monkeypatch.setattr(np, "rint", lambda y: np.sign(y) * np.floor(np.abs(y) + 0.5))
    _fails(TQ.test_int8_matches_page_code_bit_for_bit, 0)


def test_true_division_scale_is_caught(monkeypatch):
    def bad(x):
        x32 = np.asarray(x).astype(np.float32)
        s = (np.float32(127.0) / np.max(np.abs(x32), axis=-1)).astype(np.float32)
        return np.clip(np.rint(x32 * s[..., None]), -128, 127).astype(np.int8), s
    monkeypatch.setattr(quant, "quantize_int8_rows", bad)
    _fails(TQ.test_int8_matches_page_code_bit_for_bit, 0)


def test_fp8_ties_away_is_caught(monkeypatch):
    pos = widen.E4M3FN_TABLE[:0x7F]

    def bad(y):
        y = np.asarray(y, dtype=np.float64)
        mag = np.abs(y)
        hi = np.minimum(np.searchsorted(pos, mag, side="left"), len(pos) - 1)
        lo = np.maximum(hi - 1, 0)
        pick = (pos[hi] - mag) <= (mag - pos[lo])
        code = np.where(pick, hi, lo)
        return (code | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)
    monkeypatch.setattr(quant, "encode_e4m3fn", bad)
    _fails(TQ.test_e4m3fn_encoder_ties_and_random_values_match_torch)


def test_fp8_wrong_bias_is_caught(monkeypatch):
    table = np.array([widen.e4m3fn_value(c) * 2.0 for c in range(256)])
    monkeypatch.setattr(widen, "E4M3FN_TABLE", table)
    _fails(TQ.test_e4m3fn_decoder_matches_torch_on_all_codes)


def test_int4_wrong_range_is_caught(monkeypatch):
    def bad(x):   # 15 levels per side instead of 7
        x32 = np.asarray(x).astype(np.float32)
        a = np.max(np.abs(x32), axis=-1)
        s = ((np.float32(1) / a).astype(np.float32) * np.float32(15)).astype(np.float32)
        return np.clip(np.rint(x32 * s[..., None]), -16, 15).astype(np.int8), s
    monkeypatch.setattr(quant, "quantize_int4_rows", bad)
    _fails(TQ.test_int4_hand_worked_row)


def test_int4_swapped_nibbles_are_caught(monkeypatch):
    def bad(codes):
        c = np.asarray(codes).astype(np.int64) & 0xF
        return (c[..., 1::2] | (c[..., 0::2] << 4)).astype(np.uint8)
    monkeypatch.setattr(quant, "pack_int4", bad)
    _fails(TQ.test_int4_packing_by_hand_and_round_trip)


def test_int4_unsigned_widening_is_caught(monkeypatch):
    orig = widen.widen_kv

    def bad(x, fmt, scale=None):
        if fmt == "i4":
            b = np.asarray(x).astype(np.int64)
            codes = np.stack([b & 0xF, b >> 4], axis=-1).reshape(b.shape[:-1] + (-1,))
            return codes / np.asarray(scale, dtype=np.float64)[..., None]
        return orig(x, fmt, scale)
    monkeypatch.setattr(widen, "widen_kv", bad)
    _fails(TQ.test_int4_widening_divides_by_the_row_scale)


def test_causal_off_by_one_is_caught(monkeypatch):
    from oracle import multi
    from tests import test_oracle_multi as TM
    orig = multi.attend

    def bad(q_vec, K, V, scale, return_weights=False):   # sees one row fewer than its position
        return orig(q_vec, K[:-1] if len(K) > 1 else K, V[:-1] if len(V) > 1 else V, scale)
    monkeypatch.setattr(multi, "attend", bad)
    _fails(TM.test_whole_prompt_is_causal_sdpa, 4, 4)
