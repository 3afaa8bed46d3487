// pkv_prefill.hip — causal attention of many new query tokens per sequence
// over a paged KV cache (prompt chunks), hand-written for gfx950.
//
// What is computed is the multi-token form of the paged attention in
// [P3] «大模型推理加速实战：KV Cache内存优化与PagedAttention分页管理方案»
// (PagedAttention section: the cache is gathered through the block table and
// standard attention runs over it), with the causal rule that query token j
// of a sequence whose cache holds c tokens after the call sees positions
// 0 .. c - L + j.  Query head h reads KV head h / G ([P1] §3).
//
// When a sequence brings hundreds of (query token, head) rows per KV head,
// the work is a dense contraction: about 64 flop per K/V byte per 64 rows.
// The design for CDNA4:
//
//  * A workgroup of W waves takes W consecutive items of the work plan: the
//    row tiles of one (virtual sequence, chunk of its context), which read the
//    same K/V tiles.  Each 32-token step of those tiles is loaded from the
//    cache once per workgroup (16 bytes per thread and instruction, in the
//    storage order, which is already the MFMA operand order) into LDS, and
//    every wave reads it from there: no copy per wave through the caches.
//    LDS holds several steps, filled by direct global-to-LDS loads, so the
//    next steps' loads are in flight while the current ones are multiplied,
//    with no registers held for them; one barrier per set of steps.
//  * A wave holds RT tiles of 16 rows: Q in registers for the whole item,
//    S^T = K Q^T with v_mfma_f32_16x16x32_{f16,bf16} per 16 tokens, online
//    softmax in the exp2 domain, and O^T += V^T P^T with the same 32-deep MFMA
//    over the step's two 16-token groups (the K index of the PV product runs
//    over the lane's four tokens of each group, in the order the QK output
//    leaves P in the registers).
//  * Steps that every row of the wave sees whole take an unmasked path; the
//    rest mask tokens past the context or past a row's causal position, and
//    zero the V values of slots past the context.
//  * Items, virtual sequences, the plan (made once per call by the prep
//    kernel) and the split-K merge are those of the multi-token decode kernel
//    (pkv_decode.hip): a virtual sequence here is a group of W * RT * 16 rows.
//
// Caches: 16-bit of the query's type (f16/f16, bf16/bf16), FP8 E4M3FN (codes
// converted exactly after the LDS read, the per-tensor scales folded into the
// logits and the output) or INT8 with row scales (f16 queries: offset f16
// subnormal codes, as in the decode kernel; bf16: exact conversion), with f16
// or bf16 queries.
#include <atomic>

#include "pkv_common.h"
#include "pkv_internal.h"
#include "pkv_kernel.h"

// Compile-time tuning knobs (defaults are the shipped configuration):
//   PKV_PREFILL_WAVES_PER_EU   occupancy target of the prefill kernel
//   PKV_PREFILL_DEPTH_2B       LDS buffers of one step each, 16-bit caches
//   PKV_PREFILL_SYNC_2B        steps multiplied between two barriers, 16-bit
//                              caches (the buffers go round in sets of it; the
//                              loads of NB - SPS steps are in flight)
//   PKV_PREFILL_DEPTH_FP8, PKV_PREFILL_SYNC_FP8   the same for FP8 caches
//   PKV_PREFILL_DEPTH_Q, PKV_PREFILL_SYNC_Q   the same for INT8, INT4
//   PKV_PREFILL_K_AHEAD        with 2 or more steps per barrier, each later
//                              step's K bytes read during the step before it
// (16-bit caches: 2 steps per barrier in 4 buffers, 64 KB of LDS, took the
// f16 prompt chunk from 352 to 331 us.  For FP8, 2 steps in 4 buffers took
// 262 -> 251 us once the step's scalar work was trimmed.  INT8 and INT4 gained
// nothing from 2 steps in 4 buffers until the second step's K was read ahead:
// then 293.7 -> 286.9 us (INT8) and 273.1 -> 266.4 (INT4), and 3 steps in 6
// buffers another 285.5 -> 283.2 and 266.6 -> 263.6 (FP8 that way: 0.5 %
// slower); the read-ahead took f16 252.1 -> 248.9 and FP8 243.1 -> 240.1.)
#ifndef PKV_PREFILL_WAVES_PER_EU
#define PKV_PREFILL_WAVES_PER_EU 2
#endif
#ifndef PKV_PREFILL_DEPTH_2B
#define PKV_PREFILL_DEPTH_2B 4
#endif
#ifndef PKV_PREFILL_SYNC_2B
#define PKV_PREFILL_SYNC_2B 2
#endif
#ifndef PKV_PREFILL_DEPTH_FP8
#define PKV_PREFILL_DEPTH_FP8 4
#endif
#ifndef PKV_PREFILL_SYNC_FP8
#define PKV_PREFILL_SYNC_FP8 2
#endif
#ifndef PKV_PREFILL_DEPTH_Q
#define PKV_PREFILL_DEPTH_Q 6
#endif
#ifndef PKV_PREFILL_K_AHEAD
#define PKV_PREFILL_K_AHEAD 1
#endif
#ifndef PKV_PREFILL_SYNC_Q
#define PKV_PREFILL_SYNC_Q 3
#endif

namespace pkv {

// Sizes of one instance.
template <int KV, int D>
struct PrefillShape {
  static constexpr int W = kPrefillWaves;
  static constexpr int R = (int)row_bytes_of(KV, D);   // bytes per stored row
  static constexpr int GB = 16 * R;               // bytes of one 16-token group of one cache
  static constexpr int STEP = 4 * GB;             // K and V of two groups
  static constexpr bool two_byte = KV == PKV_F16 || KV == PKV_BF16;
  static constexpr int NB = two_byte ? PKV_PREFILL_DEPTH_2B
                            : KV == PKV_FP8_E4M3FN ? PKV_PREFILL_DEPTH_FP8
                                                   : PKV_PREFILL_DEPTH_Q;   // LDS buffers
  static constexpr int SPS = two_byte ? PKV_PREFILL_SYNC_2B
                             : KV == PKV_FP8_E4M3FN ? PKV_PREFILL_SYNC_FP8
                                                    : PKV_PREFILL_SYNC_Q;   // steps per barrier
  // INT8: each wave's copy of a step's 64 row scales (K g0, K g1, V g0, V g1)
  static constexpr int SCW = row_scaled(KV) ? kPrefillWaves : 1;
};

// One group of the plan: the W items (row tiles of one virtual sequence,
// chunk of its context) starting at item0, one per wave.
// KV: the cache's storage type, QT (f16 or bf16, the MFMA type), FP8 E4M3FN
// (converted exactly after the LDS read) or INT8 with row scales (f16 queries:
// offset f16 subnormal codes, the offsets taken back out; bf16: converted
// exactly through f32).
template <int QT, int KV, int D, int BS>
__device__ __forceinline__ void prefill_group(
    const DecodeArgs& a, int64_t item0, uint8_t (*lds)[PrefillShape<KV, D>::STEP],
    float (*lds_sc)[PrefillShape<KV, D>::SCW][64]) {
  constexpr int MT = MfmaOf<QT>::value;
  static_assert(MT == MT_F16 || MT == MT_BF16, "f16 or bf16 queries");
  static_assert(KV == QT || KV == PKV_FP8_E4M3FN || KV == PKV_I8 || (KV == PKV_I4 && D == 128),
                "a 16-bit cache of the query's type, FP8, INT8 or INT4 (d 128)");
  constexpr bool fp8 = KV == PKV_FP8_E4M3FN;
  constexpr bool i4 = KV == PKV_I4;
  constexpr bool i8 = row_scaled(KV);      // INT8 or INT4: row scales (names below say i8)
  constexpr bool bytewide = fp8 || KV == PKV_I8;   // one byte per element: 16 d per K chunk
  constexpr bool offset = i8 && MT == MT_F16;      // codes as offset f16 subnormals
  constexpr float code_offset = i4 ? 8.0f : 128.0f;
  using C = Cvt<KV, MT>;
  constexpr int W = kPrefillWaves;
  constexpr int RT = kPrefillRowTiles;
  constexpr int R = PrefillShape<KV, D>::R;
  constexpr int GB = PrefillShape<KV, D>::GB;
  constexpr int NL = R / 64;               // 16-byte reads per lane per group
  constexpr int KQ = D / 32;               // MFMA operand quads per lane per K group
  constexpr int NC = D / 16;               // 16-wide d chunks of the output
  constexpr int STEP = PrefillShape<KV, D>::STEP;
  constexpr int NLD = STEP / (16 * 64 * W);   // 16-byte global loads per thread per step
  static_assert(NLD >= 1 && STEP % (16 * 64 * W) == 0, "step must split evenly over the threads");
  static_assert(GB % 1024 == 0, "a wave's loads stay inside one group");
  constexpr int NB = PrefillShape<KV, D>::NB;
  constexpr int NLW = NLD + (i8 ? 1 : 0);   // loads per thread per step (INT8: + row scales)
  constexpr int SPS = PrefillShape<KV, D>::SPS;
  static_assert(SPS >= 1 && NB % SPS == 0 && NB >= 2 * SPS, "buffers in whole sets of SPS");
  static_assert((NB - 2 * SPS) * NLW <= 63, "vmcnt threshold");
  static_assert(BS >= 16 && (BS & (BS - 1)) == 0, "block sizes are powers of two, >= 16");

  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6);         // (uniform: keeps the load addresses scalar)
  const int lane = tid & (kWave - 1);
  const int r16 = lane & 15;
  const int c16 = lane >> 4;

  int b;
  SeqItems sq;
  planned_seq(a, item0, b, sq);
  b = uni(b);
  const int64_t item = item0 + wave;
  const int local0 = uni((int)(item0 - sq.first));
  const int chunk = local0 / W;                                 // (head_tiles == W)
  const int ctx = uni(sq.ctx);
  const int t_begin = uni((int)((int64_t)chunk * sq.n / sq.m) * kTileTokens);
  int t_end = (int)((int64_t)(chunk + 1) * sq.n / sq.m) * kTileTokens;
  t_end = uni(t_end < ctx ? t_end : ctx);
  const int ntiles = (t_end - t_begin + 15) >> 4;
  const int nsteps = (ntiles + 1) >> 1;
  const bool whole_unit = sq.m == 1;
  const int bq = uni(a.vseq_b[b]);
  if (bq < 0) return;                      // padding (never planned: no context)
  const int g = uni(a.vseq_g[b]);
  const int rt = uni(a.vseq_rt[b]);

  // ---- this wave's rows: row = query token * G + head of the group ----
  const int G = a.num_q_heads / a.num_kv_heads;
  int q0, L;
  query_span(a, bq, q0, L);
  q0 = uni(q0);
  L = uni(L);
  int cr = a.real_ctx[bq];
  cr = uni(cr < 0 ? 0 : (cr > a.ctx_cap ? a.ctx_cap : cr));
  const int row0 = (W * rt + wave) * 16 * RT;
  bool head_ok[RT];
  int64_t hq[RT];
  int prow[RT];                            // last position each of this lane's rows sees
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    const int rho = row0 + 16 * k + r16;
    const int j = rho / G;
    head_ok[k] = rho < L * G && q0 + j < a.q_rows;
    hq[k] = (int64_t)(q0 + j) * a.num_q_heads + g * G + rho % G;
    prow[k] = cr - L + j;
  }
  // A wave whose rows all lie past the sequence's rows still loads its share
  // of every step and meets every barrier; it skips the products.
  const bool wave_live = __builtin_amdgcn_ballot_w64(head_ok[0]) != 0;
  const int p_min = cr - L + row0 / G;     // smallest causal limit of the wave's rows
  const int full_end = p_min < t_end ? p_min + 1 : t_end;
  const int nfull = full_end > t_begin ? (full_end - t_begin) >> 4 : 0;   // whole tiles

  // Physical block of a tile (-1: outside the pool; its tokens are skipped),
  // read by a scalar load from the sequence's block table: one instruction
  // on the step's scalar path, where the wave's registers of entries took
  // four lane reads and a choice among them.  (The table is read-only here.)
  using ConstI32 = const __attribute__((address_space(4))) int32_t;
  ConstI32* bt_row = (ConstI32*)(uintptr_t)(a.block_tables + (int64_t)bq * a.max_blocks_per_seq);
  // (raw entry of a tile, clamped to the item's last tile so that the read
  // stays in the table; phys_of checks it where it is used.  A tile past the
  // item thus reads a block of the item: its tokens lie past the context and
  // are masked like any other such token.)
  auto tile_entry = [&](int tile) -> int {
    const uint32_t tc = (uint32_t)(tile < ntiles ? tile : ntiles - 1);
    return bt_row[((uint32_t)t_begin + tc * 16u) / (uint32_t)BS];
  };
  auto phys_of = [&](int v) { return (uint32_t)v < (uint32_t)a.num_blocks ? v : -1; };
  auto tile_phys = [&](int tile) -> int { return phys_of(tile_entry(tile)); };

  // ---- query operands (lane: row r16 of each row tile, the d positions of
  // its K chunks) ----
  // Query operands, in the d order of the K operands: 16-bit K chunks carry
  // d = 32 j + 8 c16 .. + 7 (quad j); FP8 and INT8 K chunks carry
  // d = 64 j + 16 c16 .. + 15 (quads 2 j and 2 j + 1 after conversion); an
  // INT4 chunk carries d = 32 c16 .. + 31, word j as quad j.
  u32x4 qop[RT][KQ];                       // (quads: the MFMA's B operands as they are)
#pragma unroll
  for (int k = 0; k < RT; ++k) {
#pragma unroll
    for (int j = 0; j < KQ; ++j) qop[k][j] = u32x4{0u, 0u, 0u, 0u};
    if (head_ok[k]) {
      const uint8_t* qrow = static_cast<const uint8_t*>(a.q) + hq[k] * D * 2;
      if constexpr (i4) {
        // INT4: the lane's K chunk holds d = 32 c16 .. 32 c16 + 31, and input
        // word j converts to elements 8 j + (0 4 1 5 2 6 3 7): q pairs are
        // taken in that order.
#pragma unroll
        for (int j = 0; j < KQ; ++j) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + (32 * c16 + 8 * j) * 2);
          qop[k][j] = u32x4{__builtin_amdgcn_perm(w[2], w[0], 0x05040100u),
                            __builtin_amdgcn_perm(w[2], w[0], 0x07060302u),
                            __builtin_amdgcn_perm(w[3], w[1], 0x05040100u),
                            __builtin_amdgcn_perm(w[3], w[1], 0x07060302u)};
        }
      } else {
#pragma unroll
        for (int j = 0; j < KQ; ++j) {
          const int d0 = bytewide ? 64 * (j / 2) + 16 * c16 + 8 * (j % 2) : 32 * j + 8 * c16;
          qop[k][j] = *reinterpret_cast<const u32x4*>(qrow + d0 * 2);
        }
      }
    }
  }
  // logits in the exp2 domain; FP8: the per-tensor scales (K into the logits,
  // V into the output); INT8: per token, 1/s (s = 127 / absmax of the row)
  // into the logit and into P.
  float kfac = a.scale * 1.4426950408889634f;
  float vfac = 1.0f;
  if constexpr (fp8) {
    kfac *= a.k_scale[0];
    vfac = a.v_scale[0];
  }
  // Offset codes: K enters the MFMA as (q + o) 2^-24 (o = 128 for INT8, 8
  // for INT4), so the logit is (2^24 S_mfma - o sum(q)) kfac / s, with sum(q)
  // over the row's query (INT4: at full weight): the QK accumulation starts
  // at -o sum(q) 2^-24, and each token's factor 2^24 kfac / s is formed once
  // per step with its reciprocal.  V comes out as 2^-24 (sum p' q + o sum p')
  // (2^-20 for INT4's odd column blocks), with sum p' (the P values fed,
  // p / s) from one more MFMA against ones.
  const float kmul = offset ? kfac * 16777216.0f : kfac;   // times 1 / s per token
  float s_init[RT];
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    float qs = 0.f;
    if constexpr (offset) {
#pragma unroll
      for (int j = 0; j < KQ; ++j) {
        f16x8 h = __builtin_bit_cast(f16x8, qop[k][j]);
        if constexpr (i4) {
          // INT4 high nibbles (odd words) enter as (q + 8) 2^-20: the query
          // words that meet them are taken at 1/16, a power of two.
          const f16x8 w16 = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)0.0625f, (_Float16)0.0625f,
                             (_Float16)1.0f, (_Float16)1.0f, (_Float16)0.0625f, (_Float16)0.0625f};
          h = h * w16;
          qop[k][j] = __builtin_bit_cast(u32x4, h);
        }
        // (sum of the words as fed, the scaled ones at 16 times their value)
#pragma unroll
        for (int e = 0; e < 8; ++e) qs += (i4 && (e & 2)) ? 16.0f * (float)h[e] : (float)h[e];
      }
      qs += __shfl_xor(qs, 16, kWave);
      qs += __shfl_xor(qs, 32, kWave);
    }
    s_init[k] = offset ? -code_offset * qs * 5.9604644775390625e-8f : 0.0f;   // (2^-24)
  }

  // Per row: m_run, the reference the row's P values are taken against (exp2
  // domain), acc = unnormalised O^T and lsum = the sum of those P, from one
  // more MFMA against ones (so it adds exactly the rounded P of the PV
  // product).  The reference moves only when a row's max passes it by more
  // than kLazy (log2 units), so P <= 2^kLazy and most steps rescale nothing;
  // the normalised result is the same whichever reference is used.  The test
  // is made on each lane's own scores against thr = (m_run + kLazy) / kf, a
  // raw-score bound (kf > 0), so the row's max over lanes is taken only on the
  // steps that move the reference.  mref: m_run kept finite for the
  // exponentials.  INT8, INT4: the step's scores become exponents x = logit -
  // mref at once, one fma per score with its token's factor (which a raw-score
  // bound cannot take: the factor varies by token), and the test is x > kLazy
  // (thr = kLazy; -inf while the row has no reference, mref 0 until then); a
  // step that moves the reference shifts its exponents by the change.
  constexpr float kLazy = 8.0f;
  f32x4 acc[RT][NC];
  f32x4 lsum[RT];
  f32x4 accp[RT];                          // offset codes: sum of the P fed to PV
  float m_run[RT], thr[RT], mref[RT];
#pragma unroll
  for (int k = 0; k < RT; ++k) {
#pragma unroll
    for (int nc = 0; nc < NC; ++nc) acc[k][nc] = f32x4{0.f, 0.f, 0.f, 0.f};
    lsum[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    accp[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[k] = -__builtin_inff();
    thr[k] = -__builtin_inff();
    mref[k] = i8 ? 0.0f : -3.402823466e38f;
  }

  // ---- global -> registers -> LDS.  Thread tid's load j of a step is the
  // 16-byte chunk c = j * 64 W + tid of the step's [K g0][K g1][V g0][V g1]
  // bytes, stored at LDS byte 16 c; a wave's chunks lie in one group of one
  // cache.  Tiles past the item or outside the pool load zeros. ----
  const uint8_t* __restrict__ kbase = static_cast<const uint8_t*>(a.k_cache);
  const uint8_t* __restrict__ vbase = static_cast<const uint8_t*>(a.v_cache);
  // Physical blocks of a step's two tiles (uniform; -1: past the item or
  // outside the pool).
  auto step_phys = [&](int step, int& p0, int& p1) {
    const int t0 = 2 * step;
    p0 = tile_phys(t0);
    p1 = tile_phys(t0 + 1);
  };
  // The loads go straight to LDS (gfx950's 16-byte global_load_lds: lane l
  // writes at the wave's LDS base + 16 l), so no registers hold the steps in
  // flight.  Every step issues the same NLD loads per thread (a tile past the
  // item or outside the pool loads the first group of block 0 instead, which
  // the products mask like any token past the context), so a fixed vmcnt
  // threshold waits for exactly the oldest step.
  // (Scalar work here is on the step's critical path: each part's row is
  // formed once per step, and when a load instruction covers exactly one
  // part, the part is a constant.)
  constexpr bool part_per_load = 64 * W == GB / 16;
  auto issue = [&](int step, int p0, int p1, int buf) {
    // rows of the step's two tiles (their first token); 0 for a tile past the
    // item or outside the pool
    // ((block, head) pairs number under 2^32: each holds at least 1 KB)
    const int s0 = (t_begin + 32 * step) & (BS - 1);   // slot of the step's first token
    // (a block outside the pool, -1, loads block 0's rows instead: masked)
    const uint32_t b0 = (uint32_t)(p0 > 0 ? p0 : 0), b1 = (uint32_t)(p1 > 0 ? p1 : 0);
    const uint64_t row0 = (uint64_t)(b0 * (uint32_t)a.num_kv_heads + (uint32_t)g) * BS + s0;
    const uint64_t row1 = (uint64_t)(b1 * (uint32_t)a.num_kv_heads + (uint32_t)g) * BS + ((s0 + 16) & (BS - 1));
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int c0 = j * 64 * W + wave * 64;           // the wave's first chunk
      const int part = part_per_load ? j : c0 / (GB / 16);   // 0 K g0, 1 K g1, 2 V g0, 3 V g1
      const uint64_t row = (part & 1) ? row1 : row0;
      const int cw = part_per_load ? wave * 64 : c0 % (GB / 16);   // chunk within the part
      const uint8_t* src = (part < 2 ? kbase : vbase) + row * R + (cw + lane) * 16;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                       (__attribute__((address_space(3))) void*)(&lds[buf][c0 * 16]),
                                       16, 0, 0);
    }
    if constexpr (i8) {
      // The step's row scales, 4 bytes per lane into this wave's copy: lane
      // l is token l % 16 of group (l / 16) % 2 of K (l < 32) or V.
      const uint64_t row = ((lane >> 4) & 1) ? row1 : row0;
      const float* src = (lane < 32 ? a.k_scale : a.v_scale) + row + (lane & 15);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                       (__attribute__((address_space(3))) void*)(&lds_sc[buf][wave][0]),
                                       4, 0, 0);
    }
  };
  // End of a set of steps: this wave's LDS reads are done (lgkmcnt 0, so the
  // buffers can be refilled after the barrier) and its loads of the next set
  // have landed: all its loads, or all but the newest NB - 2 SPS steps'
  // (vmcnt n).
  // The barrier carries no memory fence, which would wait for every load in
  // flight; the empty asm statements keep the compiler from moving LDS
  // accesses across it.
  auto step_barrier = [](bool steady) {
    constexpr int n = (NB - 2 * SPS) * NLW;
    if (steady)
      __builtin_amdgcn_s_waitcnt(0x0070 | (n & 15) | ((n >> 4) << 14));   // vmcnt(n) lgkmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0x0070);                                 // vmcnt(0) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // (scores here are finite or -inf, never NaN: IEEE maximum and the row
  // swaps of pkv_kernel.h)
  auto fmax2 = [](float x, float y) { return fmax_ieee(x, y); };
  auto fmax4 = [&](float x, float y, float z, float w) { return fmax2(fmax2(x, y), fmax2(z, w)); };
  auto pack2 = [](float x, float y) -> uint32_t { return pack_p<MT>(x, y); };
  const uint32_t one2 = MT == MT_F16 ? 0x3C003C00u : 0x3F803F80u;   // (1, 1) as f16 / bf16
  const u32x4 ones = {one2, one2, one2, one2};
  auto mfma32 = [](const u32x4& x, const u32x4& y, const f32x4& c) -> f32x4 {
    if constexpr (MT == MT_F16)
      return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x),
                                                    __builtin_bit_cast(f16x8, y), c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                     __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
  };

  // ---- one step (two 16-token groups) from LDS buffer `buf`.  `checked`
  // (uniform): the step may hold tokens past the context, past a row's causal
  // position or outside the pool, which are masked; only the masking is
  // conditional, so the accumulators never cross a branch. ----
  // S^T = K Q^T for both groups of the step in LDS buffer `buf`.
  auto qk = [&](int buf, f32x4 (&s)[RT][2]) {
    const uint8_t* base = lds[buf];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      u32x4 kq[KQ];
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(base + gi * GB + lane * 16 + 1024 * j);
        if constexpr (i4) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            uint32_t w[4];
            C::word(raw[c], w);
            kq[c] = u32x4{w[0], w[1], w[2], w[3]};
          }
        } else if constexpr (bytewide) {
          uint32_t w[8];
          C::run(raw, w);
          kq[2 * j] = u32x4{w[0], w[1], w[2], w[3]};
          kq[2 * j + 1] = u32x4{w[4], w[5], w[6], w[7]};
        } else {
          kq[j] = raw;
        }
      }
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        s[k][gi] = f32x4{s_init[k], s_init[k], s_init[k], s_init[k]};
#pragma unroll
        for (int c = 0; c < KQ; ++c) s[k][gi] = mfma32(kq[c], qop[k][c], s[k][gi]);
      }
    }
  };
  // Two or more steps per barrier (16-bit and FP8 caches): a step's K bytes
  // read during the previous step of its set (its buffer landed with the set),
  // then converted and multiplied from those registers.
  constexpr bool kAhead = PKV_PREFILL_K_AHEAD != 0 && PrefillShape<KV, D>::SPS >= 2;
  auto read_k = [&](int buf, u32x4 (&kk)[2][NL]) {
    const uint8_t* base = lds[buf];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int j = 0; j < NL; ++j)
        kk[gi][j] = *reinterpret_cast<const u32x4*>(base + gi * GB + lane * 16 + 1024 * j);
  };
  auto qk_pre = [&](const u32x4 (&kk)[2][NL], f32x4 (&s)[RT][2]) {
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      u32x4 kq[KQ];
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        if constexpr (i4) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            uint32_t w[4];
            C::word(kk[gi][j][c], w);
            kq[c] = u32x4{w[0], w[1], w[2], w[3]};
          }
        } else if constexpr (bytewide) {
          uint32_t w[8];
          C::run(kk[gi][j], w);
          kq[2 * j] = u32x4{w[0], w[1], w[2], w[3]};
          kq[2 * j + 1] = u32x4{w[4], w[5], w[6], w[7]};
        } else {
          kq[j] = kk[gi][j];
        }
      }
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        s[k][gi] = f32x4{s_init[k], s_init[k], s_init[k], s_init[k]};
#pragma unroll
        for (int c = 0; c < KQ; ++c) s[k][gi] = mfma32(kq[c], qop[k][c], s[k][gi]);
      }
    }
  };
  // The rest of a step: softmax of its scores s, then PV.
  // INT8, INT4: the step's 64 row scales (this wave's own copy) become their
  // reciprocals in place, one per lane (K's times kmul); each lane then reads
  // the 16 it uses (its four tokens of each group, K in ks[gi], V in vs[gi]).
  // (A wave's LDS accesses complete in order: the reads see the writes.)  Done
  // before the step's QK products are issued, so this chain of LDS round trips
  // runs beside them (INT4 311.6 -> 304.8 us; INT8 equal).
  auto scales = [&](int buf, f32x4 (&ks)[2], f32x4 (&vs)[2]) {
    if constexpr (i8) {
      float* sc = &lds_sc[buf][wave][0];
      const float r = __builtin_amdgcn_rcpf(sc[lane]);
      // (V's kept finite: a stored scale is positive, and a slot past the
      // context may hold anything, whose P of 0 must then give 0)
      sc[lane] = lane < 32 ? r * kmul : fminf(fabsf(r), 3.402823466e38f);
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        ks[gi] = *reinterpret_cast<const f32x4*>(&sc[16 * gi + 4 * c16]);
        vs[gi] = *reinterpret_cast<const f32x4*>(&sc[32 + 16 * gi + 4 * c16]);
      }
    }
  };
  auto finish = [&](bool checked, int step, int buf, int p0, int p1, f32x4 (&s)[RT][2],
                    const f32x4 (&ksp)[2], const f32x4 (&vsp)[2], int kbuf,
                    u32x4 (&knext)[2][NL]) {
    const uint8_t* base = lds[buf];
    int n_valid[2] = {16, 16};
    if (checked) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        int n = t_end - (t_begin + (2 * step + gi) * 16);
        n = n > 16 ? 16 : (n < 0 ? 0 : n);
        n_valid[gi] = (gi ? p1 : p0) < 0 ? 0 : n;
      }
    }
    // V operands, read now so their latency hides behind the softmax.  Lane
    // 16 c16 + r16 of a V group holds, for d = 16 nc + r16, tokens
    // 4 c16 .. 4 c16 + 3 (8 bytes per chunk nc); the operand of chunk nc is
    // group 0's 8 bytes then group 1's, read straight into its registers (one
    // two-address LDS read: the groups lie 8 x 512 bytes apart).  The empty
    // asm statement after each operand keeps the compiler from pairing reads
    // of different operands instead, which leaves every operand to be copied
    // together register by register.
    // (FP8, INT8: a lane's 16 bytes hold four chunks of 4 bytes, each
    // converted to two words; the operand is group 0's pair then group 1's.)
    u32x4 va[NC];
    if constexpr (i4) {
      // INT4: word w of a lane's 16 bytes converts to column blocks 2 w
      // (words 0, 2 of the result) and 2 w + 1 (words 1, 3), each as tokens
      // (0, 2), (1, 3) of the lane's four (P is packed in that order).
      const u32x4 r0 = *reinterpret_cast<const u32x4*>(base + 2 * GB + lane * 16);
      const u32x4 r1 = *reinterpret_cast<const u32x4*>(base + 3 * GB + lane * 16);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t w0[4], w1[4];
        C::word(r0[w], w0);
        C::word(r1[w], w1);
        va[2 * w] = u32x4{w0[0], w0[2], w1[0], w1[2]};
        va[2 * w + 1] = u32x4{w0[1], w0[3], w1[1], w1[3]};
      }
      if constexpr (kAhead) {
        if (kbuf >= 0) {
          read_k(kbuf, knext);
          asm volatile("" ::: "memory");
        }
      }
    } else if constexpr (bytewide) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const u32x4 r0 = *reinterpret_cast<const u32x4*>(base + 2 * GB + lane * 16 + 1024 * j);
        const u32x4 r1 = *reinterpret_cast<const u32x4*>(base + 3 * GB + lane * 16 + 1024 * j);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t w0[2], w1[2];
          C::word(r0[q], w0);
          C::word(r1[q], w1);
          va[4 * j + q] = u32x4{w0[0], w0[1], w1[0], w1[1]};
        }
      }
      if constexpr (kAhead) {
        if (kbuf >= 0) {
          read_k(kbuf, knext);
          asm volatile("" ::: "memory");
        }
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int off = lane * 16 + 1024 * j + 8 * h;
          const u32x2 v0 = *reinterpret_cast<const u32x2*>(base + 2 * GB + off);
          const u32x2 v1 = *reinterpret_cast<const u32x2*>(base + 3 * GB + off);
          va[2 * j + h] = u32x4{v0[0], v0[1], v1[0], v1[1]};
          asm volatile("" ::: "memory");
        }
      }
      if constexpr (kAhead) {
        if (kbuf >= 0) {
          read_k(kbuf, knext);
          asm volatile("" ::: "memory");
        }
      }
    }

    // Online softmax over the step's 32 tokens (lane: tokens 4 c16 + i of each
    // group, row r16 of each row tile).  kfac > 0, so the max of the raw
    // scores gives the max logit.  Masked scores become -inf (a select: stale
    // slots may hold NaN), so their P is exp2(-inf) = 0.
    const int tok0 = t_begin + 2 * step * 16 + 4 * c16;
    // INT8, INT4: exponents against mref (per-token factors), so kf = 1 below.
    float kf = kfac;
    f32x4 vr[2] = {f32x4{1.f, 1.f, 1.f, 1.f}, f32x4{1.f, 1.f, 1.f, 1.f}};   // INT8: 1 / s_v
    if constexpr (i8) {
      kf = 1.0f;
      // (per token: K's 2^24 kfac / s_k and V's 1 / s_v, read by `scales`)
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const f32x4 ks = ksp[gi];
        const f32x4 vs = vsp[gi];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float kr = ks[i];
          vr[gi][i] = vs[i];
#pragma unroll
          for (int k = 0; k < RT; ++k) s[k][gi][i] = __builtin_fmaf(s[k][gi][i], kr, -mref[k]);
        }
      }
    }
    if (checked) {
#pragma unroll
      for (int k = 0; k < RT; ++k)
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = 4 * c16 + i < n_valid[gi] && tok0 + 16 * gi + i <= prow[k];
            s[k][gi][i] = ok ? s[k][gi][i] : -__builtin_inff();
          }
    }
    float mx[RT];
    bool need = false;
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      mx[k] = fmax2(fmax4(s[k][0][0], s[k][0][1], s[k][0][2], s[k][0][3]),
                    fmax4(s[k][1][0], s[k][1][1], s[k][1][2], s[k][1][3]));
      need = need || mx[k] > thr[k];
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float rkf = 1.0f / kf;
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        // (INT8, INT4: the scores are exponents against mref)
        const float m_new = fmax2(m_run[k], i8 ? rows_max(mx[k]) + mref[k] : rows_max(mx[k]) * kf);
        // (a row that has seen no token keeps -inf and zeros)
        const float alpha = m_new == -__builtin_inff() ? 1.0f : __builtin_amdgcn_exp2f(m_run[k] - m_new);
#pragma unroll
        for (int nc = 0; nc < NC; ++nc) acc[k][nc] *= alpha;
        lsum[k] *= alpha;
        if constexpr (offset) accp[k] *= alpha;
        m_run[k] = m_new;
        if constexpr (i8) {
          const float ref = m_new == -__builtin_inff() ? 0.0f : m_new;
          const float delta = ref - mref[k];
#pragma unroll
          for (int gi = 0; gi < 2; ++gi)
#pragma unroll
            for (int i = 0; i < 4; ++i) s[k][gi][i] -= delta;
          mref[k] = ref;
          thr[k] = m_new == -__builtin_inff() ? -__builtin_inff() : kLazy;
        } else {
          thr[k] = (m_new + kLazy) * rkf;
          // (a row that has seen no token: every score is -inf, and the finite
          // reference keeps exp2 at 0 rather than NaN)
          mref[k] = fmax2(m_new, -3.402823466e38f);
        }
      }
    }
    u32x4 pb[RT];
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      float p[8];
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          p[4 * gi + i] = i8 ? __builtin_amdgcn_exp2f(s[k][gi][i])
                             : __builtin_amdgcn_exp2f(__builtin_fmaf(s[k][gi][i], kf, -mref[k]));
      pb[k] = u32x4{pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7])};
      lsum[k] = mfma32(ones, pb[k], lsum[k]);
      if constexpr (i8) {
        // P fed to PV: p / s_v (a masked token's p is 0 and its 1 / s_v finite)
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[4 * gi + i] *= vr[gi][i];
        if constexpr (i4)   // (token order of the INT4 V operand)
          pb[k] = u32x4{pack2(p[0], p[2]), pack2(p[1], p[3]), pack2(p[4], p[6]), pack2(p[5], p[7])};
        else
          pb[k] = u32x4{pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7])};
        if constexpr (offset) accp[k] = mfma32(ones, pb[k], accp[k]);
      }
    }

    // O^T += V^T P^T, 32 tokens deep.  Slots past the context may hold
    // anything: their V values are zeroed (INT8/INT4 codes are finite and P
    // is 0 there, and INT4's token order differs: no mask).
    if (!i8 && checked) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int cnt = n_valid[gi] - 4 * c16;
        const uint32_t m0 = (cnt > 0 ? 0xFFFFu : 0u) | (cnt > 1 ? 0xFFFF0000u : 0u);
        const uint32_t m1 = (cnt > 2 ? 0xFFFFu : 0u) | (cnt > 3 ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int nc = 0; nc < NC; ++nc) {
          va[nc][2 * gi] &= m0;
          va[nc][2 * gi + 1] &= m1;
        }
      }
    }
#pragma unroll
    for (int nc = 0; nc < NC; ++nc)
#pragma unroll
      for (int k = 0; k < RT; ++k) acc[k][nc] = mfma32(va[nc], pb[k], acc[k][nc]);
  };

  // ---- the step loop: SPS steps multiplied per barrier, the loads of the
  // next NB - SPS steps in flight meanwhile ----
  // Physical blocks of the tiles of the steps in LDS or in flight, by buffer.
  int phq0[NB], phq1[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) phq0[i] = phq1[i] = -1;
#pragma unroll
  for (int i = 0; i < NB - SPS; ++i) {
    if (i < nsteps) {
      step_phys(i, phq0[i], phq1[i]);
      issue(i, phq0[i], phq1[i], i);
    }
  }
  // Block-table entries of the set loaded next, read (scalar loads) one set
  // ahead and checked where they are used, so that the loads' latency never
  // stands between a step and its global loads.
  int nxt0[SPS], nxt1[SPS];
#pragma unroll
  for (int e = 0; e < SPS; ++e) {
    nxt0[e] = tile_entry(2 * (NB - SPS + e));
    nxt1[e] = tile_entry(2 * (NB - SPS + e) + 1);
  }
  step_barrier(false);
  u32x4 knext[2][NL];                      // (kAhead: the next step's K bytes)
  for (int step0 = 0; step0 < nsteps; step0 += NB) {
    // (unrolled by NB so the buffer numbers are constants)
#pragma unroll
    for (int u = 0; u < NB; u += SPS) {
      if (step0 + u < nsteps) {
        // The set loaded now goes into the buffers read before the last
        // barrier.
#pragma unroll
        for (int e = 0; e < SPS; ++e) {
          const int nx = step0 + u + NB - SPS + e;
          const int nb = (u + NB - SPS + e) % NB;
          if (nx < nsteps) {
            phq0[nb] = phys_of(nxt0[e]);
            phq1[nb] = phys_of(nxt1[e]);
            issue(nx, phq0[nb], phq1[nb], nb);
          }
        }
#pragma unroll
        for (int e = 0; e < SPS; ++e) {
          const int nn = step0 + u + NB + e;   // (loaded at the next set)
          nxt0[e] = tile_entry(2 * nn);
          nxt1[e] = tile_entry(2 * nn + 1);
        }
#pragma unroll
        for (int e = 0; e < SPS; ++e) {
          const int step = step0 + u + e;
          if (wave_live && step < nsteps) {
            f32x4 sc[RT][2];
            f32x4 ksp[2], vsp[2];
            scales(u + e, ksp, vsp);
            if (kAhead && e > 0)
              qk_pre(knext, sc);
            else
              qk(u + e, sc);
            // (the next step of the set: its K read at the end of this one's V reads)
            const int kbuf = kAhead && e + 1 < SPS && step + 1 < nsteps ? u + e + 1 : -1;
            finish(2 * step + 2 > nfull || (phq0[u + e] | phq1[u + e]) < 0, step, u + e,
                   phq0[u + e], phq1[u + e], sc, ksp, vsp, kbuf, knext);
          }
        }
        // (the next set has landed everywhere: all but the newest NB - 2 SPS
        // steps' loads, when every one of them was issued, else all loads)
        step_barrier(step0 + u + NB - 1 < nsteps);
      }
    }
  }
  if (!wave_live) return;

  // ---- epilogue (as in the multi-token decode kernel) ----
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    const float l_tot = lsum[k][0];        // (every entry holds the row's sum)
    if (!head_ok[k]) continue;
    if constexpr (offset) {
#pragma unroll
      for (int nc = 0; nc < NC; ++nc)
        acc[k][nc] = acc[k][nc] * ((i4 && (nc & 1)) ? 1048576.0f : 16777216.0f) -
                     code_offset * accp[k][0];
    }
    if (whole_unit) {
      const float inv = l_tot > 0.f ? vfac / l_tot : 0.f;
#pragma unroll
      for (int nc = 0; nc < NC; ++nc)
        store_out4<QT>(a.out, hq[k] * D + nc * 16 + c16 * 4, acc[k][nc][0] * inv,
                       acc[k][nc][1] * inv, acc[k][nc][2] * inv, acc[k][nc][3] * inv);
    } else if (item < a.max_items) {
      const int64_t slot = item * (16 * RT) + 16 * k + r16;
      if (c16 == 0) {
        a.ws_ml[2 * slot] = m_run[k];
        a.ws_ml[2 * slot + 1] = l_tot;
      }
#pragma unroll
      for (int nc = 0; nc < NC; ++nc)
        *reinterpret_cast<f32x4*>(a.ws_acc + slot * D + nc * 16 + c16 * 4) = acc[k][nc] * vfac;
    }
  }
}

// Slots (resident waves) the plan is made for: whole workgroups per CU.
// Workgroup k takes the k-th group of multi_prep_kernel's order, longest
// first: the hardware deals workgroups round-robin over the 8 XCDs and starts
// each XCD's next one as another finishes, so every XCD runs a longest-first
// schedule over an even share of the sizes.  (The grid is the host's bound on
// the groups; workgroups past the plan's count return at once.)
template <int QT, int KV, int D, int BS>
__global__ __launch_bounds__(64 * kPrefillWaves)
__attribute__((amdgpu_waves_per_eu(PKV_PREFILL_WAVES_PER_EU)))
void prefill_kernel(DecodeArgs a) {
  using Sh = PrefillShape<KV, D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[Sh::NB][Sh::STEP];   // [K g0][K g1][V g0][V g1]
  __shared__ __attribute__((aligned(16))) float lds_sc[Sh::NB][Sh::SCW][64];   // INT8 row scales
  const int64_t groups = a.plan_info[10];
  const int64_t items = planned_items(a);   // (the item map's entries)
  for (int64_t k = blockIdx.x; k < groups; k += gridDim.x) {
    const int64_t item0 = (int64_t)a.group_order[k] * kPrefillWaves;
    if (item0 + kPrefillWaves <= items) prefill_group<QT, KV, D, BS>(a, item0, lds, lds_sc);
  }
}

template <int QT, int KV, int D, int BS>
static hipError_t prefill_slots3(DecodeArgs& a, int num_cus) {
  static std::atomic<int> occupancy{0};    // resident workgroups per CU (compiled property)
  int per_cu = occupancy.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void*>(prefill_kernel<QT, KV, D, BS>), 64 * kPrefillWaves, 0);
    if (e != hipSuccess) return e;
    occupancy.store(per_cu, std::memory_order_relaxed);
  }
  int waves = (per_cu < 1 ? 1 : per_cu) * kPrefillWaves;
  if (waves > kWavesPerCuCap) waves = kWavesPerCuCap / kPrefillWaves * kPrefillWaves;
  a.slots = num_cus * waves;
  if (a.slots > kMaxSlots) a.slots = kMaxSlots;
  return hipSuccess;
}

template <int QT, int KV, int D, int BS>
static hipError_t launch_prefill3(DecodeArgs& a, int num_cus, bool slots_only, hipStream_t st) {
  if (slots_only) return prefill_slots3<QT, KV, D, BS>(a, num_cus);
  const int64_t need = max_items_bound(a.batch, a.head_tiles, a.ctx_cap, a.slots);
  const int64_t grid = ((need + kPrefillWaves - 1) / kPrefillWaves + 7) / 8 * 8;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<QT, KV, D, BS>), dim3((unsigned)grid), dim3(64 * kPrefillWaves),
                     0, st, a);
  return hipGetLastError();
}

template <int QT, int KV, int D>
static hipError_t launch_prefill2(DecodeArgs& a, int bs, int num_cus, bool slots_only,
                                  hipStream_t st) {
  return bs == 16 ? launch_prefill3<QT, KV, D, 16>(a, num_cus, slots_only, st)
                  : launch_prefill3<QT, KV, D, 256>(a, num_cus, slots_only, st);
}

template <int QT, int KV>
static hipError_t launch_prefill1(DecodeArgs& a, int head_dim, int bs, int num_cus,
                                  bool slots_only, hipStream_t st) {
  return head_dim == 64 ? launch_prefill2<QT, KV, 64>(a, bs, num_cus, slots_only, st)
                        : launch_prefill2<QT, KV, 128>(a, bs, num_cus, slots_only, st);
}

hipError_t launch_prefill(DecodeArgs& a, int q_dtype, int kv_dtype, int head_dim, int block_size,
                          int num_cus, bool slots_only, hipStream_t st) {
  if (a.head_tiles != kPrefillWaves || a.wave_rows != 16 * kPrefillRowTiles ||
      (head_dim != 64 && head_dim != 128))
    return hipErrorInvalidValue;
  const int hd = head_dim, bs = block_size;
  if (q_dtype == PKV_F16) {
    switch (kv_dtype) {
      case PKV_F16: return launch_prefill1<PKV_F16, PKV_F16>(a, hd, bs, num_cus, slots_only, st);
      case PKV_FP8_E4M3FN:
        return launch_prefill1<PKV_F16, PKV_FP8_E4M3FN>(a, hd, bs, num_cus, slots_only, st);
      case PKV_I8: return launch_prefill1<PKV_F16, PKV_I8>(a, hd, bs, num_cus, slots_only, st);
      case PKV_I4:
        return hd == 128 ? launch_prefill2<PKV_F16, PKV_I4, 128>(a, bs, num_cus, slots_only, st)
                         : hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
  }
  if (q_dtype == PKV_BF16) {
    switch (kv_dtype) {
      case PKV_BF16: return launch_prefill1<PKV_BF16, PKV_BF16>(a, hd, bs, num_cus, slots_only, st);
      case PKV_FP8_E4M3FN:
        return launch_prefill1<PKV_BF16, PKV_FP8_E4M3FN>(a, hd, bs, num_cus, slots_only, st);
      case PKV_I8: return launch_prefill1<PKV_BF16, PKV_I8>(a, hd, bs, num_cus, slots_only, st);
      case PKV_I4:
        return hd == 128 ? launch_prefill2<PKV_BF16, PKV_I4, 128>(a, bs, num_cus, slots_only, st)
                         : hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
