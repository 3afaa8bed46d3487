"""Pins for oracle.quant and the FP8 decoder in oracle.widen (CPU only).

INT8: the page's quantize_tensor ([P1] §4) run literally through torch in float32
on the CPU is a library routine independent of the oracle's numpy code, so the
codes must agree bit for bit; plus the properties the definition implies.
FP8: torch's float8_e4m3fn dtype (a library implementation of the OCP format)
checks the decoder on all 256 codes and the encoder on every tie and on random
values; every finite code round-trips.
"""
import numpy as np
import pytest
import torch

from oracle import quant, widen


def page_quantize_tensor(x):
    """[P1] §4 quantize_tensor, executed by torch (float32, CPU)."""
    x = torch.as_tensor(x, dtype=torch.float32)
    scale = 127.0 / x.abs().max(dim=-1, keepdim=True)[0]
    q_x = (x * scale).round().clamp(-128, 127)
    return q_x, scale


def _rows(seed, n=4000, d=128, outliers=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, d, generator=g)
    if outliers:
        mask = torch.rand(n, d, generator=g) < 0.01
        x = torch.where(mask, x * 8, x)
    return x.to(torch.float16).to(torch.float32).numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_int8_matches_page_code_bit_for_bit(seed):
    x = _rows(seed)
    q, s = quant.quantize_int8_rows(x)
    tq, ts = page_quantize_tensor(x)
    assert np.array_equal(q.astype(np.int64), tq.numpy().astype(np.int64))
    assert np.array_equal(s, ts[:, 0].numpy())


def test_int8_bf16_and_f32_sources():
    g = torch.Generator().manual_seed(3)
    for dt in (torch.bfloat16, torch.float32):
        x = (torch.randn(500, 64, generator=g) * 3).to(dt).to(torch.float32).numpy()
        q, s = quant.quantize_int8_rows(x)
        tq, ts = page_quantize_tensor(x)
        assert np.array_equal(q.astype(np.int64), tq.numpy().astype(np.int64))


def test_int8_absmax_maps_to_127():
    x = _rows(4)
    q, s = quant.quantize_int8_rows(x)
    idx = np.argmax(np.abs(x), axis=-1)
    picked = q[np.arange(len(q)), idx].astype(np.int64)
    sign = np.sign(x[np.arange(len(q)), idx])
    assert np.array_equal(np.abs(picked), np.full(len(q), 127))
    assert np.array_equal(np.sign(picked), sign)
    assert q.min() >= -127   # -128 is never reached (|x * 127/a| <= 127 + rounding)


def test_int8_error_bound():
    x = _rows(5)
    q, s = quant.quantize_int8_rows(x)
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) / s[:, None].astype(np.float64))
    bound = (0.5 + 127 * 2.0 ** -23) / s[:, None].astype(np.float64)
    assert np.all(err <= bound)


def test_int8_odd_symmetry_and_power_of_two_scaling():
    x = _rows(6)
    q, s = quant.quantize_int8_rows(x)
    qn, sn = quant.quantize_int8_rows(-x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for k in (-3, 1, 5):
        q2, s2 = quant.quantize_int8_rows(x * np.float32(2.0 ** k))
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, (s * np.float32(2.0 ** -k)).astype(np.float32))


def test_int8_zero_row():
    x = np.zeros((3, 16), dtype=np.float32)
    x[1, 3] = 2.5
    q, s = quant.quantize_int8_rows(x)
    assert np.all(q[0] == 0) and s[0] == np.float32(1.0)
    assert np.all(q[2] == 0) and s[2] == np.float32(1.0)
    assert q[1, 3] == 127 and s[1] == (np.float32(1.0) / np.float32(2.5)) * np.float32(127.0)


def test_e4m3fn_decoder_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = widen.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.nanmax(mine) == 448.0
    assert np.sum(np.isnan(mine)) == 2          # 0x7F and 0xFF
    assert mine[1] == 2.0 ** -9                 # smallest subnormal


def test_e4m3fn_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = widen.e4m3fn_to_f64(codes)
    back = quant.encode_e4m3fn(vals)
    assert np.array_equal(back, codes)          # includes -0.0 -> 0x80


def _torch_encode(y):
    t = torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3fn_encoder_ties_and_random_values_match_torch():
    pos = widen.E4M3FN_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)   # exact in float32
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    for y in (mids, -mids):
        assert np.array_equal(quant.encode_e4m3fn(y), _torch_encode(y))
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01,
                        rng.standard_normal(20000) * 30]).astype(np.float32)
    y = np.clip(y, -448, 448)
    assert np.array_equal(quant.encode_e4m3fn(y), _torch_encode(y))


def test_fp8_tensor_quantizer():
    x = _rows(7, n=500)
    codes, s = quant.quantize_fp8(x)
    a = np.float32(np.max(np.abs(x)))
    assert s == np.float32(a / np.float32(448))
    # The largest magnitude lands on 448 (code 0x7E / 0xFE).
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert codes[i] & 0x7F == 0x7E
    # Relative round-trip error in the normal range is at most 2^-4.
    deq = widen.widen_kv(codes, "fp8", s)
    normal = np.abs(x) / s >= 2.0 ** -6
    rel = np.abs(deq[normal] - x[normal]) / np.abs(x[normal])
    assert rel.max() <= 2.0 ** -4
    # Saturation with a given scale: values past 448 * s clamp to the largest code.
    big = np.array([1e6, -1e6, 464.0, 480.0], dtype=np.float32)
    c2, _ = quant.quantize_fp8(big, scale=np.float32(1.0))
    assert list(c2) == [0x7E, 0xFE, 0x7E, 0x7E]
    zc, zs = quant.quantize_fp8(np.zeros(8, dtype=np.float32))
    assert zs == np.float32(1.0) and np.all(zc == 0)
