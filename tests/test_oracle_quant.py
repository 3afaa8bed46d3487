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
    """The INT8 rule of [P1] «LLM推理显存优化：KV Cache管理3大策略实测，节省60%显存开销»
    §4 (quantize_tensor), carried out by torch in float32 on the CPU: per row,
    the largest magnitude a; the scale is the number 127 divided by the tensor
    of those maxima (torch's scalar-by-tensor division, the operation the page
    applies); codes are the rows times their scale, rounded half to even and
    limited to [-128, 127].  Returns (codes, scales [n][1])."""
    rows = torch.as_tensor(x, dtype=torch.float32)
    absmax = torch.amax(torch.abs(rows), dim=1, keepdim=True)
    scales = torch.Tensor.__rtruediv__(absmax, 127.0)
    codes = torch.clamp(torch.round(torch.mul(rows, scales)), min=-128, max=127)
    return codes, scales


def test_torch_scalar_by_tensor_division_is_reciprocal_times_scalar():
    """(Why the oracle forms the scale as fl32(fl32(1/a) * 127): that is what
    torch computes for the page's scalar-by-tensor division.)"""
    a = torch.from_numpy(np.abs(_rows(9, n=20000, outliers=False)).max(axis=1))
    assert torch.equal(torch.Tensor.__rtruediv__(a, 127.0), torch.reciprocal(a) * 127.0)


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


# ---------------------------------------------------------------------------
# INT4: [P1] §4 lists an INT4 cache only by its size and speed; the quantizer
# read here is the page's INT8 rule with 7 for 127 and [-8, 7] for the clamp.
# Pins: a hand-worked row, the nearest-code definition checked by brute force
# over all 16 codes, the sign/absmax properties, the nibble order by hand.
# ---------------------------------------------------------------------------
def test_int4_hand_worked_row():
    # a = 1, s = fl32(1/1) * 7 = 7: codes rint(3.5) = 4 (half to even),
    # rint(-7) = -7, rint(1.75) = 2, 0; rint(-0.35) = -0.
    q, s = quant.quantize_int4_rows(np.array([[0.5, -1.0, 0.25, 0.0, -0.05]], np.float32))
    assert s[0] == np.float32(7.0)
    assert q[0].tolist() == [4, -7, 2, 0, 0]
    # a = 0.75: s = fl32(fl32(1/0.75) * 7); 0.1 * s = 0.9333.. -> 1, -0.375 * s = -3.5 -> -4
    q, s = quant.quantize_int4_rows(np.array([[0.1, -0.375, 0.75]], np.float32))
    assert s[0] == np.float32(np.float32(np.float32(1) / np.float32(0.75)) * np.float32(7))
    assert q[0].tolist() == [1, -4, 7]


@pytest.mark.parametrize("seed", [0, 1])
def test_int4_codes_are_the_nearest_of_all_sixteen(seed):
    """Brute force: for every element, the code is the one of -8..7 closest to
    fl32(x * s), ties to the even code."""
    x = _rows(seed, n=600, d=64)
    q, s = quant.quantize_int4_rows(x)
    y = (x * s[:, None]).astype(np.float32).astype(np.float64)
    codes = np.arange(-8, 8, dtype=np.float64)
    dist = np.abs(y[..., None] - codes)
    best = dist.min(axis=-1, keepdims=True)
    ties = dist == best
    # among tied codes pick the even one
    pick = np.where(ties.sum(-1) > 1, np.argmax(ties & (codes % 2 == 0), axis=-1), np.argmin(dist, -1))
    assert np.array_equal(q.astype(np.int64), (pick - 8).astype(np.int64))


def test_int4_absmax_maps_to_seven_and_zero_rows():
    x = _rows(5, n=500, d=128)
    x[7] = 0.0
    q, s = quant.quantize_int4_rows(x)
    idx = np.argmax(np.abs(x), axis=-1)
    picked = q[np.arange(len(q)), idx].astype(np.int64)
    live = np.arange(len(q)) != 7
    assert np.all(np.abs(picked[live]) == 7)
    assert np.array_equal(np.sign(picked[live]), np.sign(x[np.arange(len(q)), idx][live]))
    assert q.min() >= -7 and q.max() <= 7 and np.all(q[7] == 0) and s[7] == 1.0
    # error bound: |x - q/s| <= 0.5/s (+ one rounding of x*s)
    err = np.abs(x.astype(np.float64) - q / s[:, None].astype(np.float64))
    assert np.all(err[live] <= (0.5 + 1e-5) / s[live, None])


def test_int4_odd_symmetry_and_power_of_two_scaling():
    x = _rows(6, n=300, d=64)
    q, s = quant.quantize_int4_rows(x)
    qn, sn = quant.quantize_int4_rows(-x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    q4, s4 = quant.quantize_int4_rows(x * 4)
    assert np.array_equal(q4, q) and np.array_equal(s4, s / 4)


def test_int4_packing_by_hand_and_round_trip():
    assert quant.pack_int4(np.array([1, -2, 7, -8], np.int8)).tolist() == [0xE1, 0x87]
    assert quant.unpack_int4(np.array([0xE1, 0x87], np.uint8)).tolist() == [1, -2, 7, -8]
    rng = np.random.default_rng(7)
    c = rng.integers(-8, 8, size=(5, 3, 64)).astype(np.int8)
    assert np.array_equal(quant.unpack_int4(quant.pack_int4(c)), c)


def test_int4_widening_divides_by_the_row_scale():
    packed = quant.pack_int4(np.array([[3, -8, 0, 7]], np.int8))
    got = widen.widen_kv(packed, "i4", np.array([2.0], np.float32))
    assert got.tolist() == [[1.5, -4.0, 0.0, 3.5]]
