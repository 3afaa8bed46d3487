// pkv_kernel.h — device code shared by the attention kernels (gfx950): MFMA
// element types, stored-byte conversions, query/output element access, and
// the work plan every wave of a launch computes from the device-resident
// context lengths.
#pragma once

#include "pkv_common.h"
#include "pkv_internal.h"

namespace pkv {

enum { MT_F32 = 0, MT_F16 = 1, MT_BF16 = 2 };

template <int QT>
struct MfmaOf {
  static constexpr int value = QT == PKV_F32 ? MT_F32 : (QT == PKV_F16 ? MT_F16 : MT_BF16);
};

// ---------------------------------------------------------------------------
// Stored KV bytes -> MFMA input elements.
//
// Each call converts one 16-byte chunk.  For 16-bit MFMA types the result is
// packed two elements per 32-bit word; for f32 it is one float per word.
// FP8 -> f16/bf16/f32 uses gfx950's E4M3 conversions (exact).  INT8 -> f16
// gives offset subnormals (q + 128) 2^-24, corrected after the products.
// INT4 (8 nibbles per word) takes nibble pairs
// 16 bits apart, so word w of the output holds nibbles (w, w + 4) of the
// input word (an order the query operand is loaded in to match): -> f16 as
// offset subnormals (q + 8) 2^-24 / 2^-20, corrected after the products;
// -> bf16 exactly, through f32 (2^23 + u - (2^23 + 8)); -> f32 exactly, one
// element per word in the nibbles' own order.
// ---------------------------------------------------------------------------
template <int KV, int MT>
struct Cvt {
  static constexpr int in_elems = 128 / dtype_bits(KV);             // per 16 B chunk
  static constexpr int out_words = MT == MT_F32 ? in_elems : in_elems / 2;
  static constexpr int word_out = out_words / 4;                     // outputs per input word

  // One 32-bit word of stored bytes -> word_out MFMA words.
  __device__ __forceinline__ static void word(const uint32_t raw, uint32_t* w) {
    if constexpr ((KV == PKV_F16 && MT == MT_F16) || (KV == PKV_BF16 && MT == MT_BF16) ||
                  (KV == PKV_F32 && MT == MT_F32)) {
      w[0] = raw;
    } else if constexpr (KV == PKV_I8 && MT == MT_F16) {
      // Offset codes as f16 subnormals (q + 128) 2^-24: the bytes of
      // raw ^ 0x80 moved to the low byte of each half (see OffsetCodes).
      const uint32_t t = raw ^ 0x80808080u;
      w[0] = __builtin_amdgcn_perm(0u, t, 0x04010400u);
      w[1] = __builtin_amdgcn_perm(0u, t, 0x04030402u);
    } else if constexpr (KV == PKV_I4 && MT == MT_F16) {
      // Offset codes as f16 subnormals, one bit operation per word:
      // (raw & mask) ^ 8 puts u ^ 8 = q + 8 (u = the stored two's-complement
      // nibble) in the low mantissa bits, i.e. (q + 8) 2^-24 for the low nibble
      // of a byte pair and (q + 8) 2^-20 for the high one.  The kernel takes
      // the offset and the powers of two back out (see OffsetCodes); the MFMA
      // multiplies f16 subnormals exactly.
      const uint32_t x8 = raw >> 8;
      w[0] = (raw & 0x000F000Fu) ^ 0x00080008u;
      w[1] = (raw & 0x00F000F0u) ^ 0x00800080u;
      w[2] = (x8 & 0x000F000Fu) ^ 0x00080008u;
      w[3] = (x8 & 0x00F000F0u) ^ 0x00800080u;
    } else if constexpr (KV == PKV_I4 && MT == MT_F32) {
      // Exact: nibble e of the word (element 8 i + e of the chunk's word i),
      // sign-extended.
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = fbits((float)((int32_t)(raw << (28 - 4 * e)) >> 28));
    } else if constexpr (KV == PKV_I4 && MT == MT_BF16) {
      const uint32_t x = raw ^ 0x88888888u;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lo = bitsf(0x4B000000u | ((x >> (4 * k)) & 0xFu)) - 8388616.0f;
        const float hi = bitsf(0x4B000000u | ((x >> (4 * k + 16)) & 0xFu)) - 8388616.0f;
        w[k] = __builtin_amdgcn_perm(fbits(hi), fbits(lo), 0x07060302u);   // exact: truncation
      }
    } else if constexpr (KV == PKV_FP8_E4M3FN && MT == MT_F16) {
      // gfx950 converts OCP E4M3 pairs to f16 (exact; scale 1).
      w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw, 1.0f, false));
      w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw, 1.0f, true));
    } else if constexpr (KV == PKV_FP8_E4M3FN && MT == MT_BF16) {
      w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw, 1.0f, false));
      w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw, 1.0f, true));
    } else if constexpr (KV == PKV_FP8_E4M3FN && MT == MT_F32) {
      const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw, 1.0f, false);
      const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw, 1.0f, true);
      w[0] = fbits(lo[0]);
      w[1] = fbits(lo[1]);
      w[2] = fbits(hi[0]);
      w[3] = fbits(hi[1]);
    } else {
      // Generic: through f32 (exact for every pair built here).
      static_assert(KV != PKV_I4, "INT4 converts to f16 or bf16 only");
      constexpr int eb = dtype_bytes(KV);
      constexpr int per = 4 / eb;   // elements in the word
      float f[per];
#pragma unroll
      for (int e = 0; e < per; ++e) {
        const int sh = e * eb * 8;
        if constexpr (KV == PKV_I8) {
          f[e] = (float)(int8_t)((raw >> sh) & 0xFFu);
        } else if constexpr (KV == PKV_FP8_E4M3FN) {
          f[e] = e4m3fn_to_f32((raw >> sh) & 0xFFu);
        } else if constexpr (KV == PKV_F16) {
          f[e] = f16_to_f32((uint16_t)((raw >> sh) & 0xFFFFu));
        } else if constexpr (KV == PKV_BF16) {
          f[e] = bf16_to_f32((uint16_t)((raw >> sh) & 0xFFFFu));
        } else {
          f[e] = bitsf(raw);
        }
      }
#pragma unroll
      for (int o = 0; o < word_out; ++o) {
        if constexpr (MT == MT_F32) {
          w[o] = fbits(f[o]);
        } else if constexpr (MT == MT_F16) {
          w[o] = (uint32_t)f32_to_f16(f[2 * o]) | ((uint32_t)f32_to_f16(f[2 * o + 1]) << 16);
        } else {  // bf16: every value converted here is exact in bf16, so truncate
          w[o] = (fbits(f[2 * o]) >> 16) | (fbits(f[2 * o + 1]) & 0xFFFF0000u);
        }
      }
    }
  }

  // One 16-byte chunk -> out_words MFMA words.
  __device__ __forceinline__ static void run(const u32x4 raw, uint32_t* w) {
#pragma unroll
    for (int i = 0; i < 4; ++i) word(raw[i], w + i * word_out);
  }
};

// Extra factor the conversion above leaves in the value (none: every
// conversion is exact).
template <int KV, int MT>
__host__ __device__ constexpr float cvt_gain() {
  return 1.0f;
}

// One query element (stored as QT) as an MFMA element (16-bit pattern or f32 bits).
template <int QT>
__device__ __forceinline__ uint32_t q_elem(const void* q, int64_t idx) {
  if constexpr (QT == PKV_F32) {
    return fbits(static_cast<const float*>(q)[idx]);
  } else {
    return static_cast<const uint16_t*>(q)[idx];
  }
}

template <int QT>
__device__ __forceinline__ void store_out4(void* out, int64_t idx, float a, float b, float c,
                                           float d) {
  if constexpr (QT == PKV_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx) = f32x4{a, b, c, d};
  } else if constexpr (QT == PKV_F16) {
    u32x2 w = {(uint32_t)f32_to_f16(a) | ((uint32_t)f32_to_f16(b) << 16),
               (uint32_t)f32_to_f16(c) | ((uint32_t)f32_to_f16(d) << 16)};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + idx) = w;
  } else {
    u32x2 w = {(uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16),
               (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16)};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + idx) = w;
  }
}

// Two f32 values -> a packed f16 or bf16 pair, round to nearest even (one
// v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32 on gfx950).
template <int MT>
__device__ __forceinline__ uint32_t pack_p(float a, float b) {
  const f32x2 v = {a, b};
  if constexpr (MT == MT_F16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
}

// IEEE maximum: no operand canonicalisation (which fmaxf costs on MFMA
// results).  The softmax takes it over scores that are finite or -inf.
__device__ __forceinline__ float fmax_ieee(float x, float y) {
  return __builtin_elementwise_maximum(x, y);
}

// Max of a value over the four 16-lane rows of a wave (lanes L, L ^ 16,
// L ^ 32, L ^ 48): gfx950's row swaps, no LDS round trip.
__device__ __forceinline__ float rows_max(float v) {
  const auto x16 = __builtin_amdgcn_permlane16_swap(fbits(v), fbits(v), false, false);
  v = fmax_ieee(bitsf(x16[0]), bitsf(x16[1]));
  const auto x32 = __builtin_amdgcn_permlane32_swap(fbits(v), fbits(v), false, false);
  return fmax_ieee(bitsf(x32[0]), bitsf(x32[1]));
}

// ---------------------------------------------------------------------------
// Work plan (computed identically by every wave of both kernels).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int64_t wave_incl_scan_i64(int64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int64_t t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// A wave-uniform value held in VGPRs, moved to SGPRs.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// A wave-uniform pointer, moved to SGPRs (so that address arithmetic on it
// stays scalar and memory instructions take it as their scalar base).
template <typename T>
__device__ __forceinline__ T* sptr(T* p) {
  return reinterpret_cast<T*>(uni64(reinterpret_cast<int64_t>(p)));
}

__device__ __forceinline__ int64_t readlane_i64(int64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), lane);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Context length of sequence b, clamped to what the table can address.
__device__ __forceinline__ int seq_ctx(const DecodeArgs& a, int b) {
  int c = a.context_lens[b];
  return c < 0 ? 0 : (c > a.ctx_cap ? a.ctx_cap : c);
}

struct Plan {
  int64_t items;   // total work items
  int tpi;         // tiles per item (a unit of n tiles makes ceil(n / tpi) items)
};

// Clamped context lengths of sequences 64*c + lane (0 past the batch).  The
// first 256 sequences' come from registers filled once (the only read of
// context_lens for batches up to 256); later ones are read again.
struct SeqCtx {
  int cached[4];
  __device__ __forceinline__ void fill(const DecodeArgs& a, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 64 * i + lane;
      cached[i] = b < a.batch ? seq_ctx(a, b) : 0;
    }
  }
  __device__ __forceinline__ int ctx(const DecodeArgs& a, int c, int lane) const {
    if (c < 4) {   // uniform selects: the array stays in registers
      int v = cached[0];
      v = c == 1 ? cached[1] : v;
      v = c == 2 ? cached[2] : v;
      v = c == 3 ? cached[3] : v;
      return v;
    }
    const int b = 64 * c + lane;
    return b < a.batch ? seq_ctx(a, b) : 0;
  }
  __device__ __forceinline__ int tiles(const DecodeArgs& a, int c, int lane) const {
    return (ctx(a, c, lane) + kTileTokens - 1) / kTileTokens;
  }
};

// Chunks (items per unit) of a decode sequence of n tiles: ceil(n / tpi), and
// one for an empty sequence, whose item writes its zeros (so that a call whose
// units are never split needs no second kernel).
__device__ __forceinline__ int seq_chunks(int n, int tpi) {
  return n > 0 ? (n + tpi - 1) / tpi : 1;
}

__device__ __forceinline__ int64_t count_items(const DecodeArgs& a, const SeqCtx& st, int tpi,
                                               int lane) {
  int64_t items = 0;
  for (int c = 0; 64 * c < a.batch; ++c)
    if (64 * c + lane < a.batch) items += seq_chunks(st.tiles(a, c, lane), tpi);
  return uni64(wave_sum_i64(items) * ((int64_t)a.plan_heads * a.head_tiles));
}

// Tiles per item: about (total tiles) / (slots - units), so that one round of
// items fits the slots even after each unit's count is rounded up; several
// rounds when an item would pass the kernel's item limit `cap`.  (Filling the
// slots exactly, with more and smaller items, measured slower.)  tiles and
// live count (unit, tile) pairs and units with any tile.
__device__ __forceinline__ int plan_tpi(int64_t tiles, int64_t live, int64_t slots, int cap) {
  slots = slots > 0 ? slots : 1;
  int64_t se = slots - live;
  if (se < slots / 2) se = slots / 2;
  if (se < 1) se = 1;
  int64_t k = (tiles + se * cap - 1) / (se * cap);
  if (k < 1) k = 1;
  int64_t t = (tiles + k * se - 1) / (k * se);
  t = t < kItemTilesMin ? kItemTilesMin : (t > cap ? cap : t);
  return (int)t;
}

// The decode plan (every wave computes it the same way); st keeps the
// contexts it read, for seq_of_item.
__device__ inline Plan make_plan(const DecodeArgs& a, int lane, SeqCtx& st) {
  st.fill(a, lane);
  int64_t tiles = 0, live = 0;
  for (int c = 0; 64 * c < a.batch; ++c) {
    const int n = st.tiles(a, c, lane);
    tiles += n;
    live += n > 0;
  }
  const int64_t ups = (int64_t)a.plan_heads * a.head_tiles;
  tiles = uni64(wave_sum_i64(tiles) * ups);
  live = uni64(wave_sum_i64(live) * ups);
  Plan p;
  p.tpi = plan_tpi(tiles, live, a.slots, a.item_cap);
  p.items = count_items(a, st, p.tpi, lane);
  return p;
}

// Items of a sequence are numbered chunk-major, then by KV head, then by head
// tile: item = first + (c * plan_heads + g) * head_tiles + ht, with
// m = seq_chunks(n, tpi) chunks of the sequence's n tiles per unit; chunk c
// covers tiles [c*n/m, (c+1)*n/m).  (g runs over plan_heads KV heads: all of
// them for decode, one for a multi-token virtual sequence, which carries its
// own.)  Consecutive items thus read the same blocks, one (block, KV head)
// tile each.
struct SeqItems {
  int64_t first;   // number of the sequence's first item
  int ctx;         // clamped context length
  int n;           // tiles
  int m;           // chunks per unit
};

// The decode sequence holding item q (false if q is past the last item).
__device__ inline bool seq_of_item(const DecodeArgs& a, const Plan& p, const SeqCtx& st,
                                   int64_t q, int lane, int& b_out, SeqItems& s) {
  const int64_t units_per_seq = (int64_t)a.plan_heads * a.head_tiles;
  int64_t base = 0;
  for (int b0 = 0; b0 < a.batch; b0 += kWave) {
    const int b = b0 + lane;
    const int ctx = st.ctx(a, b0 / kWave, lane);
    const int n = (ctx + kTileTokens - 1) / kTileTokens;
    const int m = b < a.batch ? seq_chunks(n, p.tpi) : 0;
    const int64_t cnt = (int64_t)m * units_per_seq;
    const int64_t incl = wave_incl_scan_i64(cnt, lane) + base;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(q >= incl - cnt && q < incl);
    if (hit) {
      const int L = __builtin_ctzll(hit);
      b_out = b0 + L;
      s.first = readlane_i64(incl - cnt, L);
      s.ctx = __builtin_amdgcn_readlane(ctx, L);
      s.n = __builtin_amdgcn_readlane(n, L);
      s.m = __builtin_amdgcn_readlane(m, L);
      return true;
    }
    base = readlane_i64(incl, kWave - 1);
  }
  return false;
}

// Query rows of real sequence b of a multi-token call: first row q0 and count
// L.  query_start is a precondition (0, nondecreasing, ending at q_rows); for
// memory safety only, both ends are clamped into [0, q_rows], so every row
// q0 .. q0 + L - 1 lies inside q and out.
__device__ __forceinline__ void query_span(const DecodeArgs& a, int b, int& q0, int& L) {
  int s = a.query_start[b], e = a.query_start[b + 1];
  s = s < 0 ? 0 : (s > a.q_rows ? a.q_rows : s);
  e = e < s ? s : (e > a.q_rows ? a.q_rows : e);
  q0 = s;
  L = e - s;
}

// Multi-token calls: the plan is made once per call by multi_prep_kernel,
// which also numbers the items of each virtual sequence and maps every item
// to its virtual sequence (so a workgroup finds its work in a few loads).
__device__ __forceinline__ int64_t planned_items(const DecodeArgs& a) { return a.plan_info[0]; }
__device__ __forceinline__ void planned_seq(const DecodeArgs& a, int64_t item, int& b,
                                            SeqItems& s) {
  b = a.item_vseq[item];
  s.first = a.vseq_first[b];
  s.m = a.vseq_m[b];
  s.ctx = seq_ctx(a, b);
  s.n = (s.ctx + kTileTokens - 1) / kTileTokens;
}

}  // namespace pkv
