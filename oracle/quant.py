"""KV quantizers (TEST INFRASTRUCTURE ONLY; see the package header).

(INT4, per row, and its nibble packing: see ``quantize_int4_rows``.)

INT8, per row — [P1] §4 (INT8 quantization, quantize_tensor): the scale is 127
divided by the row's largest magnitude (``dim=-1``, one scale per row), the row
is multiplied by it, rounded and clamped to [-128, 127].  Readings taken:

* precision: float32, the dtype the page's tensors carry; numpy's float32
  division and multiplication are IEEE correctly rounded;
* the scale: the page writes the scalar 127 divided by the absmax tensor in
  PyTorch, and PyTorch evaluates a scalar divided by a tensor as the tensor's
  reciprocal times the scalar.  So the scale the page's code produces is
  ``fl32(fl32(1 / a) * 127)``, one float32 ulp away from a true division in about
  a quarter of rows; that executed form is the definition used here;
* rounding: the page calls torch's ``round``, which rounds half to even, so
  ``np.rint``;
* granularity: one scale per (token, KV head) row over head_dim — the code's
  ``dim=-1``, where the prose says "per block of K/V data";
* a zero row (the page's formula divides by zero): codes 0 and stored scale 1.0.

FP8, per tensor — [P2] §4 (``--kv-cache-dtype fp8``) and [P3] (KV quantization
section) name an FP8 KV cache with no format or scale rule.  Readings taken:
OCP E4M3FN; one float32 scale per tensor ``s = max|x| / 448`` (448 = the largest
finite E4M3FN value), codes ``encode(clamp(x / s, -448, 448))`` with x / s in
float32 and round-to-nearest, ties to the even code; dequantized value
``decode(code) * s``.  A zero tensor takes ``s = 1.0``.
"""

import numpy as np

from .widen import E4M3FN_TABLE

E4M3FN_MAX = 448.0


def quantize_int8_rows(x):
    """Per-row INT8 quantization.  ``x``: float array (f16/f32 exact, or bf16
    already widened to float32), rows along the last axis.  Returns
    ``(codes int8, scale float32)`` with ``scale`` shaped like ``x`` minus its last axis."""
    x32 = np.asarray(x).astype(np.float32)
    absmax = np.max(np.abs(x32), axis=-1)
    zero = absmax == 0
    safe = np.where(zero, np.float32(1.0), absmax).astype(np.float32)
    recip = (np.float32(1.0) / safe).astype(np.float32)
    scale = (recip * np.float32(127.0)).astype(np.float32)
    scale = np.where(zero, np.float32(1.0), scale).astype(np.float32)
    y = (x32 * scale[..., None]).astype(np.float32)
    q = np.clip(np.rint(y), -128, 127)
    q = np.where(zero[..., None], 0, q)
    return q.astype(np.int8), scale


def quantize_int4_rows(x):
    """Per-row INT4 quantization: [P1] §4's rule with the 4-bit range — the
    pages report an INT4 cache ([P1] §4, quantization-effect table) but give
    its quantizer only for INT8; the reading taken keeps every step and puts
    7 = 2**3 - 1 where the INT8 code has 127: ``s = fl32(fl32(1/a) * 7)``,
    ``q = clamp(rint(fl32(x * s)), -8, 7)``, a zero row gives codes 0 and scale
    1.0.  Returns ``(codes int8 in [-8, 7], scale float32)``."""
    x32 = np.asarray(x).astype(np.float32)
    absmax = np.max(np.abs(x32), axis=-1)
    zero = absmax == 0
    safe = np.where(zero, np.float32(1.0), absmax).astype(np.float32)
    recip = (np.float32(1.0) / safe).astype(np.float32)
    scale = (recip * np.float32(7.0)).astype(np.float32)
    scale = np.where(zero, np.float32(1.0), scale).astype(np.float32)
    y = (x32 * scale[..., None]).astype(np.float32)
    q = np.clip(np.rint(y), -8, 7)
    q = np.where(zero[..., None], 0, q)
    return q.astype(np.int8), scale


def pack_int4(codes):
    """INT4 codes ``[..., d]`` (int8 in [-8, 7]) -> bytes ``[..., d/2]``: element
    2k in the low nibble of byte k, element 2k+1 in the high nibble, two's
    complement."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed):
    """Inverse of ``pack_int4``: bytes ``[..., d/2]`` -> int8 codes ``[..., d]``."""
    b = np.asarray(packed).astype(np.int64)
    lo, hi = b & 0xF, b >> 4
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int64)
    out[..., 0::2], out[..., 1::2] = lo, hi
    return np.where(out >= 8, out - 16, out).astype(np.int8)


def fp8_tensor_scale(x):
    """Per-tensor FP8 scale ``max|x| / 448`` in float32 (1.0 for an all-zero tensor)."""
    x32 = np.asarray(x).astype(np.float32)
    a = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    if a == 0:
        return np.float32(1.0)
    return np.float32(a / np.float32(E4M3FN_MAX))


# Non-negative finite E4M3FN magnitudes, ascending with the code (0x00..0x7E).
_POS_VALUES = E4M3FN_TABLE[:0x7F]


def encode_e4m3fn(y):
    """Nearest E4M3FN code to each float ``y`` (|y| <= 448 expected), ties to the
    code with an even mantissa; the sign bit follows the sign of ``y`` (so -0.0
    and small negatives that round to zero give 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    mag = np.abs(y)
    if np.any(mag > E4M3FN_MAX) or np.any(np.isnan(y)):
        raise ValueError("encode_e4m3fn expects finite values clamped to +-448")
    hi = np.searchsorted(_POS_VALUES, mag, side="left")        # first value >= mag
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag == _POS_VALUES[hi], hi, code)
    sign = np.signbit(y).astype(np.int64) << 7
    return (code.astype(np.int64) | sign).astype(np.uint8)


def quantize_fp8(x, scale=None):
    """Per-tensor FP8 E4M3FN quantization.  Returns ``(codes uint8, scale float32)``;
    if ``scale`` is given it is used as is."""
    x32 = np.asarray(x).astype(np.float32)
    s = fp8_tensor_scale(x32) if scale is None else np.float32(scale)
    y = (x32 / s).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3FN_MAX), np.float32(E4M3FN_MAX))
    return encode_e4m3fn(y), np.float32(s)
