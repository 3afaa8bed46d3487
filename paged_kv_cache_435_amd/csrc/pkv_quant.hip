// pkv_quant.hip — KV quantization and cache append, hand-written for gfx950.
//
// INT8 ([P1] «LLM推理显存优化：KV Cache管理3大策略实测，节省60%显存开销» §4,
// quantize_tensor): per row a = max|x|, s = fl32(fl32(1/a) * 127) — the form
// PyTorch evaluates for the page's scalar-over-tensor 127 / absmax — then
// q = clamp(rint(fl32(x * s)), -128, 127).  Division is IEEE (no fast-math),
// rint is round-half-even, so codes and scales are bit-exact.
//
// INT4: the same rule with 7 for 127 and codes clamped to [-8, 7], packed two
// per byte (see int4_row_scale).
//
// FP8 E4M3FN, one scale per tensor ([P2] «生产级 LLM 推理的 KV 缓存优化» §4
// --kv-cache-dtype fp8; [P3] KV-quantization section): s = fl32(max|x| / 448),
// codes = RNE(clamp(fl32(x / s), -448, 448)).
//
// Append ([P3] PagedAttention section: each new token's row goes to the slot
// its block table names): one wave per (token, KV head); the row is copied or
// quantized on the fly.
#include "pkv_common.h"
#include "pkv_internal.h"

namespace pkv {

template <int XT>
__device__ __forceinline__ float load_f32(const void* x, int64_t i) {
  if constexpr (XT == PKV_F32) return static_cast<const float*>(x)[i];
  else if constexpr (XT == PKV_F16) return f16_to_f32(static_cast<const uint16_t*>(x)[i]);
  else return bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
}

// Row scale of the INT8 quantizer; 0 marks an all-zero row.
__device__ __forceinline__ float int8_row_scale(float absmax) {
  if (absmax == 0.0f) return 0.0f;
  const float r = 1.0f / absmax;   // IEEE correctly rounded
  return r * 127.0f;
}

__device__ __forceinline__ int8_t int8_code(float x, float s) {
  const float y = x * s;
  float q = __builtin_rintf(y);
  q = q < -128.0f ? -128.0f : (q > 127.0f ? 127.0f : q);
  return (int8_t)(int)q;
}

// INT4 ([P1] §4 lists an INT4 cache without its quantizer; the rule here is
// the INT8 one with 7 for 127): s = fl32(fl32(1/a) * 7), codes in [-8, 7]
// (|x * s| <= 7 up to rounding, so -8 is never produced).
__device__ __forceinline__ float int4_row_scale(float absmax) {
  if (absmax == 0.0f) return 0.0f;
  const float r = 1.0f / absmax;
  return r * 7.0f;
}

__device__ __forceinline__ uint32_t int4_nibble(float x, float s) {
  if (s == 0.0f) return 0u;
  float q = __builtin_rintf(x * s);
  q = q < -8.0f ? -8.0f : (q > 7.0f ? 7.0f : q);
  return (uint32_t)(int)q & 0xFu;
}

__device__ __forceinline__ uint8_t fp8_code(float x, float s) {
  float y = x / s;                 // IEEE correctly rounded
  if (y != y) return (uint8_t)(0x7Fu | ((fbits(y) >> 24) & 0x80u));   // NaN stays NaN
  y = y < -448.0f ? -448.0f : (y > 448.0f ? 448.0f : y);
  return (uint8_t)f32_to_e4m3fn(y);
}

// ---------------------------------------------------------------------------
// INT8 rows: one wave per row, four rows per workgroup.
// ---------------------------------------------------------------------------
template <int XT>
__global__ __launch_bounds__(256) void quantize_int8_kernel(const void* __restrict__ x,
                                                            int8_t* __restrict__ out,
                                                            float* __restrict__ scale,
                                                            int64_t n_rows, int row_len) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  const int64_t base = row * row_len;
  float a = 0.0f;
  for (int i = lane; i < row_len; i += kWave) a = fmaxf(a, __builtin_fabsf(load_f32<XT>(x, base + i)));
  a = wave_max(a);
  const float s = int8_row_scale(a);
  for (int i = lane; i < row_len; i += kWave)
    out[base + i] = s == 0.0f ? (int8_t)0 : int8_code(load_f32<XT>(x, base + i), s);
  if (lane == 0) scale[row] = s == 0.0f ? 1.0f : s;
}

// INT4 rows: one wave per row, four rows per workgroup; lane i packs elements
// 2i and 2i + 1 into byte i (low nibble first).
template <int XT>
__global__ __launch_bounds__(256) void quantize_int4_kernel(const void* __restrict__ x,
                                                            uint8_t* __restrict__ out,
                                                            float* __restrict__ scale,
                                                            int64_t n_rows, int row_len) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  const int64_t base = row * row_len;
  float a = 0.0f;
  for (int i = lane; i < row_len; i += kWave) a = fmaxf(a, __builtin_fabsf(load_f32<XT>(x, base + i)));
  a = wave_max(a);
  const float s = int4_row_scale(a);
  const int half = row_len / 2;
  for (int i = lane; i < half; i += kWave) {
    const uint32_t lo = int4_nibble(load_f32<XT>(x, base + 2 * i), s);
    const uint32_t hi = int4_nibble(load_f32<XT>(x, base + 2 * i + 1), s);
    out[row * half + i] = (uint8_t)(lo | (hi << 4));
  }
  if (lane == 0) scale[row] = s == 0.0f ? 1.0f : s;
}

// ---------------------------------------------------------------------------
// FP8 per tensor: absmax (atomic max on the bit pattern of non-negative
// floats, accumulated in scale[0]), finalize, encode.
// ---------------------------------------------------------------------------
__global__ void fp8_scale_init_kernel(float* scale) {
  if (threadIdx.x == 0) reinterpret_cast<uint32_t*>(scale)[0] = 0u;
}

template <int XT>
__global__ __launch_bounds__(256) void fp8_absmax_kernel(const void* __restrict__ x, int64_t n,
                                                         float* scale) {
  float a = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    a = fmaxf(a, __builtin_fabsf(load_f32<XT>(x, i)));
  a = wave_max(a);
  if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned int*>(scale), fbits(a));
}

__global__ void fp8_scale_finalize_kernel(float* scale) {
  if (threadIdx.x == 0) {
    const float a = bitsf(reinterpret_cast<uint32_t*>(scale)[0]);
    scale[0] = a == 0.0f ? 1.0f : a / 448.0f;
  }
}

template <int XT>
__global__ __launch_bounds__(256) void fp8_encode_kernel(const void* __restrict__ x, int64_t n,
                                                         const float* __restrict__ scale,
                                                         uint8_t* __restrict__ out) {
  const float s = scale[0];
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = fp8_code(load_f32<XT>(x, i), s);
}

template <int XT>
static hipError_t quantize_t(const void* x, int64_t n_rows, int row_len, int out_dtype, void* out,
                             float* scale, int scale_given, hipStream_t st) {
  if (out_dtype == PKV_I8 || out_dtype == PKV_I4) {
    if (n_rows == 0) return hipSuccess;
    const int64_t blocks = (n_rows + 3) / 4;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (out_dtype == PKV_I8)
      hipLaunchKernelGGL((quantize_int8_kernel<XT>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                         static_cast<int8_t*>(out), scale, n_rows, row_len);
    else
      hipLaunchKernelGGL((quantize_int4_kernel<XT>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                         static_cast<uint8_t*>(out), scale, n_rows, row_len);
    return hipGetLastError();
  }
  const int64_t n = n_rows * (int64_t)row_len;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  if (!scale_given) {
    hipLaunchKernelGGL(fp8_scale_init_kernel, dim3(1), dim3(64), 0, st, scale);
    if (n > 0)
      hipLaunchKernelGGL((fp8_absmax_kernel<XT>), dim3((unsigned)blocks), dim3(256), 0, st, x, n,
                         scale);
    hipLaunchKernelGGL(fp8_scale_finalize_kernel, dim3(1), dim3(64), 0, st, scale);
  }
  if (n > 0)
    hipLaunchKernelGGL((fp8_encode_kernel<XT>), dim3((unsigned)blocks), dim3(256), 0, st, x, n,
                       (const float*)scale, static_cast<uint8_t*>(out));
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int x_dtype, int64_t n_rows, int row_len, int out_dtype,
                           void* out, float* scale, int scale_given, hipStream_t st) {
  switch (x_dtype) {
    case PKV_F32: return quantize_t<PKV_F32>(x, n_rows, row_len, out_dtype, out, scale, scale_given, st);
    case PKV_F16: return quantize_t<PKV_F16>(x, n_rows, row_len, out_dtype, out, scale, scale_given, st);
    default: return quantize_t<PKV_BF16>(x, n_rows, row_len, out_dtype, out, scale, scale_given, st);
  }
}

// ---------------------------------------------------------------------------
// Append: one wave per (token, KV head) row, four rows per workgroup.  Each
// lane takes D/64 consecutive elements of the row and stores them at their
// place in the row's 16-token group (k_group_offset / v_group_offset).
// ---------------------------------------------------------------------------
template <int ST, int CT, int D>
__global__ __launch_bounds__(256) void append_kernel(const void* __restrict__ k,
                                                     const void* __restrict__ v,
                                                     const int64_t* __restrict__ slots,
                                                     void* __restrict__ k_cache,
                                                     void* __restrict__ v_cache,
                                                     float* __restrict__ k_scale,
                                                     float* __restrict__ v_scale, int64_t rows,
                                                     int num_blocks, int block_size,
                                                     int num_kv_heads) {
  constexpr int PER = D / kWave;   // elements per lane
  constexpr int eb = dtype_bytes(CT);
  constexpr int R = (int)row_bytes_of(CT, D);   // bytes per stored row
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int64_t t = row / num_kv_heads;
  const int g = (int)(row % num_kv_heads);
  const int64_t src_row = t * num_kv_heads + g;
  // The slot and the row's source values are loaded together (the source
  // addresses do not depend on the slot); the slot is checked after.
  const int64_t slot = slots[t];

  if constexpr (CT == PKV_I4) {
    // Lane i holds two elements that share a stored byte: K elements 2i, 2i+1;
    // V elements d and d + 16 with d = 32 (i / 16) + i % 16.
    static_assert(D == 128, "INT4 rows are 128 elements");
    float x[2][2];
    int d0[2];
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const void* src = which == 0 ? k : v;
      d0[which] = which == 0 ? 2 * lane : 32 * (lane >> 4) + (lane & 15);
      const int d1 = which == 0 ? d0[which] + 1 : d0[which] + 16;
      x[which][0] = load_f32<ST>(src, src_row * D + d0[which]);
      x[which][1] = load_f32<ST>(src, src_row * D + d1);
    }
    if (slot < 0 || slot >= (int64_t)num_blocks * block_size) return;
    const int64_t blk = slot / block_size;
    const int off = (int)(slot % block_size);
    const int t16 = off & 15;
    const int64_t dst_row = (blk * num_kv_heads + g) * block_size + off;   // scale index
    const int64_t group_byte = (dst_row - t16) * R;                      // first byte of the group
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      uint8_t* cache = static_cast<uint8_t*>(which == 0 ? k_cache : v_cache) + group_byte;
      float* sc = which == 0 ? k_scale : v_scale;
      const float a = wave_max(fmaxf(__builtin_fabsf(x[which][0]), __builtin_fabsf(x[which][1])));
      const float s = int4_row_scale(a);
      const uint32_t bits = int4_nibble(x[which][0], s) | (int4_nibble(x[which][1], s) << 4);
      const int pos = which == 0 ? k_group_offset(t16, lane, 1) : v4_group_nibble(t16, d0[which]) >> 1;
      cache[pos] = (uint8_t)bits;
      if (lane == 0) sc[dst_row] = s == 0.0f ? 1.0f : s;
    }
    return;
  }
  // Same type: the stored bits; otherwise the values as f32.
  uint32_t raw[2][PER];
  float xv[2][PER];
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const void* src = which == 0 ? k : v;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int64_t i = src_row * D + lane * PER + e;
      if constexpr (CT == ST) {
        if constexpr (eb == 4)
          raw[which][e] = static_cast<const uint32_t*>(src)[i];
        else
          raw[which][e] = static_cast<const uint16_t*>(src)[i];
      } else {
        xv[which][e] = load_f32<ST>(src, i);
      }
    }
  }
  if (slot < 0 || slot >= (int64_t)num_blocks * block_size) return;
  const int64_t blk = slot / block_size;
  const int off = (int)(slot % block_size);
  const int t16 = off & 15;
  const int64_t dst_row = (blk * num_kv_heads + g) * block_size + off;   // scale index
  const int64_t group_byte = (dst_row - t16) * R;                      // first byte of the group
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    uint8_t* cache = static_cast<uint8_t*>(which == 0 ? k_cache : v_cache) + group_byte;
    float* sc = which == 0 ? k_scale : v_scale;
    int pos[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int d = lane * PER + e;
      pos[e] = which == 0 ? k_group_offset(t16, d, eb) : v_group_offset(t16, d, eb);
    }
    if constexpr (CT == ST) {
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        if constexpr (eb == 4)
          *reinterpret_cast<uint32_t*>(cache + pos[e]) = raw[which][e];
        else
          *reinterpret_cast<uint16_t*>(cache + pos[e]) = (uint16_t)raw[which][e];
      }
    } else if constexpr (CT == PKV_I8) {
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < PER; ++e) a = fmaxf(a, __builtin_fabsf(xv[which][e]));
      a = wave_max(a);
      const float s = int8_row_scale(a);
#pragma unroll
      for (int e = 0; e < PER; ++e)
        cache[pos[e]] = (uint8_t)(s == 0.0f ? (int8_t)0 : int8_code(xv[which][e], s));
      if (lane == 0) sc[dst_row] = s == 0.0f ? 1.0f : s;
    } else {  // FP8 with the tensor's scale
      const float s = sc[0];
#pragma unroll
      for (int e = 0; e < PER; ++e) cache[pos[e]] = fp8_code(xv[which][e], s);
    }
  }
}

template <int ST, int CT>
static hipError_t append_t(const void* k, const void* v, int num_tokens, const int64_t* slots,
                           void* kc, void* vc, float* ks, float* vs, int nb, int bs, int hkv,
                           int d, hipStream_t st) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t rows = (int64_t)num_tokens * hkv;
  const int64_t blocks = (rows + 3) / 4;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if constexpr (CT == PKV_I4) {
    if (d != 128) return hipErrorInvalidValue;
  } else if (d == 64) {
    hipLaunchKernelGGL((append_kernel<ST, CT, 64>), dim3((unsigned)blocks), dim3(256), 0, st, k, v,
                       slots, kc, vc, ks, vs, rows, nb, bs, hkv);
    return hipGetLastError();
  }
    hipLaunchKernelGGL((append_kernel<ST, CT, 128>), dim3((unsigned)blocks), dim3(256), 0, st, k,
                       v, slots, kc, vc, ks, vs, rows, nb, bs, hkv);
  return hipGetLastError();
}

template <int ST>
static hipError_t append_s(int ct, const void* k, const void* v, int n, const int64_t* slots,
                           void* kc, void* vc, float* ks, float* vs, int nb, int bs, int hkv,
                           int d, hipStream_t st) {
  switch (ct) {
    case PKV_I8: return append_t<ST, PKV_I8>(k, v, n, slots, kc, vc, ks, vs, nb, bs, hkv, d, st);
    case PKV_I4: return append_t<ST, PKV_I4>(k, v, n, slots, kc, vc, ks, vs, nb, bs, hkv, d, st);
    case PKV_FP8_E4M3FN:
      return append_t<ST, PKV_FP8_E4M3FN>(k, v, n, slots, kc, vc, ks, vs, nb, bs, hkv, d, st);
    default: return append_t<ST, ST>(k, v, n, slots, kc, vc, ks, vs, nb, bs, hkv, d, st);
  }
}

hipError_t launch_append(const void* k, const void* v, int src_dtype, int num_tokens,
                         const int64_t* slots, void* k_cache, void* v_cache, float* k_scale,
                         float* v_scale, int num_blocks, int block_size, int num_kv_heads,
                         int head_dim, int cache_dtype, hipStream_t st) {
  switch (src_dtype) {
    case PKV_F32:
      return append_s<PKV_F32>(cache_dtype, k, v, num_tokens, slots, k_cache, v_cache, k_scale,
                               v_scale, num_blocks, block_size, num_kv_heads, head_dim, st);
    case PKV_F16:
      return append_s<PKV_F16>(cache_dtype, k, v, num_tokens, slots, k_cache, v_cache, k_scale,
                               v_scale, num_blocks, block_size, num_kv_heads, head_dim, st);
    default:
      return append_s<PKV_BF16>(cache_dtype, k, v, num_tokens, slots, k_cache, v_cache, k_scale,
                                v_scale, num_blocks, block_size, num_kv_heads, head_dim, st);
  }
}

}  // namespace pkv
