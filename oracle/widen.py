"""Stored KV bytes -> float64 (TEST INFRASTRUCTURE ONLY; see the package header).

Each decoder is written from the format's definition, not from a library cast:

* f32 / f16: IEEE binary32 / binary16, widened exactly by numpy.
* bf16: the upper 16 bits of an IEEE binary32 (held here as uint16 bit patterns,
  since numpy has no bfloat16); widening = shift into the high half.
* INT8 with a per-row scale: the quantizer of [P1] §4 (quantize_tensor) stores
  ``q = round(x * s)`` with ``s = 127 / max|x|``, so the value it stands for is
  ``q / s``.  (The page's dequant_matmul multiplies by the scales instead; that
  contradicts its own quantizer, and the quantizer's definition is followed.)
* FP8 E4M3FN (the OCP 8-bit float with 4 exponent bits, bias 7, 3 mantissa bits,
  subnormals, no infinities, NaN only at S.1111.111, largest finite 448) with a
  per-tensor scale: the stored code stands for ``decode(code) * s``.  The pages
  name only "fp8" for the KV cache ([P2] §4 ``--kv-cache-dtype fp8``; [P3] KV
  quantization section); E4M3FN is the reading taken.
"""

import numpy as np

FORMATS = ("f32", "f16", "bf16", "i8", "fp8", "i4")


def bf16_bits_to_f64(bits):
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("bf16 values are passed as uint16 bit patterns")
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_value(code):
    """Value of one FP8 E4M3FN code (0..255) from the format definition."""
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


# One entry per code; built from the definition above, code by code.
E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e4m3fn_to_f64(codes):
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("fp8 values are passed as uint8 codes")
    return E4M3FN_TABLE[codes]


def widen_plain(x, fmt):
    """f32 / f16 / bf16 storage -> float64 (exact)."""
    if fmt == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if fmt == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if fmt == "bf16":
        return bf16_bits_to_f64(x)
    raise ValueError(f"not a plain float format: {fmt}")


def widen_kv(x, fmt, scale=None):
    """Dequantize stored KV rows to float64.

    ``x`` has the row dimension last.  For ``i8``, ``scale`` has the shape of ``x``
    without its last axis (one float32 per row); for ``fp8`` it is one scalar.
    """
    if fmt in ("f32", "f16", "bf16"):
        return widen_plain(x, fmt)
    if fmt == "i8":
        x = np.asarray(x)
        if x.dtype != np.int8:
            raise TypeError("int8 cache must be int8")
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        return x.astype(np.float64) / s[..., None]
    if fmt == "fp8":
        return e4m3fn_to_f64(x) * float(np.float32(scale))
    if fmt == "i4":
        # Two's-complement nibbles, two per byte (element 2k low, 2k+1 high),
        # value code / scale like INT8.
        b = np.asarray(x)
        if b.dtype != np.uint8:
            raise TypeError("int4 cache rows are packed uint8")
        lo, hi = b.astype(np.int64) & 0xF, b.astype(np.int64) >> 4
        codes = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.float64)
        codes[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
        codes[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        return codes / s[..., None]
    raise ValueError(f"unknown KV format {fmt}")
