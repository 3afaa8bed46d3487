// pkv_common.h — shared device helpers for the paged-KV kernels (gfx950).
//
// Storage formats: IEEE f32 / f16, bfloat16 (upper half of an f32), INT8 and
// INT4 (two's-complement nibbles, two per byte) with a per-row scale, and OCP
// FP8 E4M3FN (bias 7, 3 mantissa bits, max 448).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

// Wavefront width on CDNA.
constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int64_t i64x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
// Round to nearest even (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return bitsf((uint32_t)h << 16); }
// Round to nearest even; inputs here are finite.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = fbits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// FP8 E4M3FN code -> f32, from the format definition (exact for every finite
// code; the NaN code 0x7F/0xFF decodes to 480 here and is only ever met in slots
// the kernels never use).
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t code) {
  const uint32_t sign = (code & 0x80u) << 24;
  const uint32_t e = (code >> 3) & 0xFu;
  const uint32_t m = code & 0x7u;
  const float sub = (float)m * 0.001953125f;               // m * 2^-9
  const float nrm = bitsf(((e + 120u) << 23) | (m << 20));  // 2^(e-7) * (1 + m/8)
  return bitsf(fbits(e == 0 ? sub : nrm) | sign);
}

// f32 (finite, |y| <= 448) -> nearest E4M3FN code, ties to even; sign from y.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float y) {
  const uint32_t u = fbits(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __builtin_fabsf(y);
  uint32_t code;
  if (a < 0.015625f) {                    // below 2^-6: the subnormal grid m * 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);   // exact scaling, RNE; 8 -> 2^-6
  } else {
    const uint32_t ua = fbits(a);
    int32_t e = (int32_t)(ua >> 23) - 127;            // -6 .. 8
    uint32_t m3 = (ua >> 20) & 7u;
    const uint32_t rem = ua & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
    if (m3 == 8u) { m3 = 0; ++e; }
    code = ((uint32_t)(e + 7) << 3) | m3;
  }
  return sign | code;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Element size of a storage type (INT4: two elements per byte; use
// dtype_bits or row_bytes for it).
__host__ __device__ constexpr int dtype_bytes(int dt) {
  return dt == PKV_F32 ? 4 : (dt == PKV_F16 || dt == PKV_BF16) ? 2 : 1;
}
__host__ __device__ constexpr int dtype_bits(int dt) { return dt == PKV_I4 ? 4 : 8 * dtype_bytes(dt); }
// Bytes of one stored row of d elements.
__host__ __device__ constexpr int64_t row_bytes_of(int dt, int64_t d) { return d * dtype_bits(dt) / 8; }
// Storage types with one float32 scale per stored row.
__host__ __device__ constexpr bool row_scaled(int dt) { return dt == PKV_I8 || dt == PKV_I4; }

// ---------------------------------------------------------------------------
// Storage order inside a group of 16 consecutive token rows of one (block,
// KV head) tile (the pool keeps the [NB][Hkv][bs][d] shape; only the order of
// the 16 * d elements of each 16-row group changes).  eb = element bytes.
//
// K: the row of token t is cut into 16-byte chunks; chunk c of token t sits at
//    byte (c * 16 + t) * 16.  A wave reading 16 bytes per lane at lane * 16
//    (+1 KB per instruction) gets chunk (j * 4 + lane / 16) of token lane % 16:
//    the A operand of a 16x16xK MFMA with tokens as rows.
// V: element (t, d) with nc = d / 16, r = d % 16, c = t / 4, i = t % 4 and
//    G = 4 / eb column blocks per 16 bytes sits at byte
//    ((nc / G) * 64 + c * 16 + r) * 16 + ((nc % G) * 4 + i) * eb.
//    Lane 16 c + r of instruction j then holds, for d = 16 nc + r with
//    nc in [j G, j G + G), the values of tokens 4c .. 4c + 3: the A operand of
//    O^T += V^T P^T.
// ---------------------------------------------------------------------------
//
// INT4 (rows of d / 2 packed bytes, element 2k in the low nibble of byte k):
// K groups chunk the packed rows as above (k_group_offset(t, d / 2, 1), the
// nibble of element d being d & 1).  V groups move nibbles: element (t, d),
// n = d / 16, sits at nibble v4_group_nibble(t, d) of the group, i.e. byte
// ((n / 8) * 64 + (t / 4) * 16 + d % 16) * 16 + ((n % 8) / 2) * 4 + t % 4,
// low nibble for even n.  Lane 16 c + r of a 16-byte load then holds, in word
// w, tokens 4c .. 4c + 3 of columns 16 (2w) + r (low nibbles) and
// 16 (2w + 1) + r (high nibbles); a byte holds one token's d and d + 16.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int k_group_offset(int t, int d, int eb) {
  return (((d * eb) >> 4) * 16 + t) * 16 + ((d * eb) & 15);
}
__host__ __device__ constexpr int v_group_offset(int t, int d, int eb) {
  return (((d >> 4) / (4 / eb)) * 64 + (t >> 2) * 16 + (d & 15)) * 16 +
         (((d >> 4) % (4 / eb)) * 4 + (t & 3)) * eb;
}
__host__ __device__ constexpr int v4_group_nibble(int t, int d) {
  return ((((d >> 4) >> 3) * 64 + (t >> 2) * 16 + (d & 15)) * 16 + (((d >> 4) & 7) >> 1) * 4 +
          (t & 3)) * 2 + ((d >> 4) & 1);
}

}  // namespace pkv
