// pkv_decode.hip — decode attention over a paged KV cache, hand-written for gfx950.
//
// What is computed ([P1] «LLM推理显存优化：KV Cache管理3大策略实测，节省60%显存开销»
// §2–§4; [P3] «大模型推理加速实战：KV Cache内存优化与PagedAttention分页管理方案»,
// PagedAttention section): for each sequence b and query head h, softmax attention
// of q[b][h] over the cached rows of KV head h / G, each row found through the
// sequence's block table.  The pages run this on NVIDIA parts with vLLM's kernel;
// the design here is for CDNA4:
//
//  * One 64-lane wave per work item: a run of 16-token tiles of one (sequence,
//    KV head, tile of up to 16 query heads of that KV head's group) unit.  The
//    KV rows are read from HBM once per KV head and shared by the whole query
//    group.  Every wave plans the cut itself from the device-resident context
//    lengths, so that one round of near-equal items fills the waves the GPU
//    runs at once (ragged batches otherwise leave a tail of stragglers).
//    Items are dealt to the 8 XCDs in contiguous ranges, and the KV heads of
//    one (sequence, chunk) go to the waves of one workgroup, so that adjacent
//    (block, head) tiles are read together.
//  * The cache stores each 16-token group of a (block, KV head) tile in MFMA
//    operand order (pkv_common.h: k_group_offset, v_group_offset), so K and V
//    are both read with 16 B per lane and 1 KB contiguous per instruction
//    straight into operand registers: no LDS, no transposes.
//  * Tokens go 16 at a time.  QK^T is one MFMA chain per 16 tokens:
//    S^T[16 tok][16 heads] = K[16 tok][d] * Q^T[d][16 heads]
//    (v_mfma_f32_16x16x32_{f16,bf16}, or 16x16x4 for f32); Q sits in registers
//    for the whole item.
//  * Online softmax in the exp2 domain on the MFMA output registers.  A lane
//    holds 4 tokens of one head, so a head's max needs two cross-lane steps.
//  * PV as O^T[d][heads] += V^T[d][16 tok] * P^T[16 tok][heads]
//    (v_mfma_f32_16x16x16, or 16x16x4 for f32).  P^T is exactly the QK output
//    layout, so P never leaves its registers.
//  * A unit cut into several items gets (max, sum, unnormalised output) per
//    item, merged by a second kernel with the log-sum-exp rule.  A unit that is
//    one item is finished in place.
//  * Tokens past the context are selected out of the softmax (never
//    multiplied), and their V values are masked to zero, so stale or NaN bytes
//    in unused slots never reach the sums.
//  * Several query tokens per sequence (prompt chunks, draft verification) use
//    the same kernel with MULTI set: a wave takes 32 rows of (query token, head
//    of the group), each lane masking tokens past its row's causal position;
//    up to four such waves of one (sequence, KV head, chunk) form a
//    workgroup, or, when a virtual sequence is one wave, eight waves take the
//    KV heads of one (sequence, chunk) as in decode.  multi_prep_kernel turns
//    each sequence's rows into "virtual sequences" whose contexts end at their
//    last row's position, so the planner and the merge above work unchanged.
#include <stdlib.h>

#include <atomic>
#include <type_traits>

#include "pkv_common.h"
#include "pkv_internal.h"
#include "pkv_kernel.h"

// Compile-time tuning knobs (defaults are the shipped configuration):
//   PKV_NT_LOADS            KV loads carry the non-temporal hint
//   PKV_NT_SCALE_LOADS      row-scale loads (INT8, INT4) carry it too
//   PKV_WAVES_PER_EU        occupancy target, KV other than INT8
//   PKV_STAGES_2B           pipeline depth (tiles in flight), 16-bit and f32 KV
//   PKV_STAGES_I8           pipeline depth (tiles in flight), INT8 KV
//   PKV_STAGES_FP8          pipeline depth (tiles in flight), FP8 KV
//   PKV_STAGES_I4           pipeline depth (tiles in flight), INT4 KV
//   PKV_STAGES_MULTI        pipeline depth (tiles in flight), multi-token calls
//   PKV_MULTI_WAVES_PER_EU  occupancy target, multi-token calls
//   PKV_WAVES_PER_EU_I4     occupancy target, INT4 KV
//   PKV_WAVES_PER_EU_FP8    occupancy target, FP8 KV
//   PKV_SLOTS_PER_CU_FP8      items planned per compute unit and round, FP8 KV
//   PKV_SLOTS_PER_CU_DEFAULT  items planned per compute unit and round
//   PKV_SLOTS_PER_CU_I8       the same for INT8 KV
//   PKV_SLOTS_PER_CU_I4       the same for INT4 KV
//   PKV_TILES_PER_UPDATE_I4   16-token tiles per online-softmax step, INT4 KV
//   PKV_TILES_PER_UPDATE_I8   the same for INT8 KV
//   PKV_TILES_PER_UPDATE_FP8  the same for FP8 KV
//   PKV_I4_DEEP_UNITS         INT4 decode: most units for the DEEP instance
//   PKV_*_I4_DEEP             stages, occupancy, items per CU and tiles per
//                             step of that instance
#ifndef PKV_NT_LOADS
#define PKV_NT_LOADS 1
#endif
#ifndef PKV_NT_SCALE_LOADS
#define PKV_NT_SCALE_LOADS 1
#endif
#ifndef PKV_WAVES_PER_EU
#define PKV_WAVES_PER_EU 3
#endif
#ifndef PKV_STAGES_2B
#define PKV_STAGES_2B 1
#endif
#ifndef PKV_STAGES_I8
#define PKV_STAGES_I8 1
#endif
#ifndef PKV_STAGES_FP8
#define PKV_STAGES_FP8 2
#endif
#ifndef PKV_SLOTS_PER_CU_DEFAULT
#define PKV_SLOTS_PER_CU_DEFAULT 8
#endif
#ifndef PKV_SLOTS_PER_CU_I8
#define PKV_SLOTS_PER_CU_I8 16
#endif
#ifndef PKV_STAGES_I4
#define PKV_STAGES_I4 2
#endif
#ifndef PKV_STAGES_MULTI
#define PKV_STAGES_MULTI 1
#endif
#ifndef PKV_MULTI_WAVES_PER_EU
#define PKV_MULTI_WAVES_PER_EU 2
#endif
#ifndef PKV_WAVES_PER_EU_I4
#define PKV_WAVES_PER_EU_I4 4
#endif
#ifndef PKV_SLOTS_PER_CU_I4
#define PKV_SLOTS_PER_CU_I4 16
#endif
#ifndef PKV_WAVES_PER_EU_FP8
#define PKV_WAVES_PER_EU_FP8 PKV_WAVES_PER_EU
#endif
#ifndef PKV_SLOTS_PER_CU_FP8
#define PKV_SLOTS_PER_CU_FP8 PKV_SLOTS_PER_CU_DEFAULT
#endif
#ifndef PKV_ITEM_TILES_I8
#define PKV_ITEM_TILES_I8 512
#endif
#ifndef PKV_ITEM_TILES_I4
#define PKV_ITEM_TILES_I4 256
#endif
#ifndef PKV_TILES_PER_UPDATE_I4
#define PKV_TILES_PER_UPDATE_I4 1
#endif
#ifndef PKV_TILES_PER_UPDATE_I8
#define PKV_TILES_PER_UPDATE_I8 1
#endif
#ifndef PKV_TILES_PER_UPDATE_FP8
#define PKV_TILES_PER_UPDATE_FP8 1
#endif
#ifndef PKV_I4_DEEP_UNITS
#define PKV_I4_DEEP_UNITS 512
#endif
#ifndef PKV_STAGES_I4_DEEP
#define PKV_STAGES_I4_DEEP 2
#endif
#ifndef PKV_WAVES_PER_EU_I4_DEEP
#define PKV_WAVES_PER_EU_I4_DEEP 2
#endif
#ifndef PKV_SLOTS_PER_CU_I4_DEEP
#define PKV_SLOTS_PER_CU_I4_DEEP 8
#endif
#ifndef PKV_TILES_PER_UPDATE_I4_DEEP
#define PKV_TILES_PER_UPDATE_I4_DEEP 2
#endif

namespace pkv {

// ---------------------------------------------------------------------------
// Partition kernel.
//
// The tile loop is software-pipelined: while tile i is converted and
// multiplied, the K/V loads of the next tiles are already in flight (register
// sets used in rotation, the loop unrolled so no register copy waits on a
// load).  The waves of a workgroup are independent and need no LDS.
// ---------------------------------------------------------------------------
// Lane L of each 16-lane row, broadcast to the whole row (DPP row_newbcast).
// Every lane is written, so the destination's old value is not needed (no
// initialising move).
template <int L>
__device__ __forceinline__ float row_bcast(float v) {
  return bitsf((uint32_t)__builtin_amdgcn_mov_dpp((int)fbits(v), 0x150 + L, 0xF, 0xF, false));
}

// A 16-byte load from a wave-uniform base plus the lane's byte offset.  The
// base has passed through readfirstlane, which hides its address space, so it
// is cast to a global pointer first and the offset added after: the load then
// takes the scalar base and a 32-bit vector offset.  (The empty asm makes the
// offset a value of the load's own block, so instruction selection sees a
// zero-extended 32-bit value rather than a 64-bit copy made before the loop.)
__device__ __forceinline__ u32x4 ld16(const uint8_t* base, uint32_t off) {
  asm("" : "+v"(off));
  const __attribute__((address_space(1))) uint8_t* g = (const __attribute__((address_space(1))) uint8_t*)base;
  const __attribute__((address_space(1))) u32x4* p = (const __attribute__((address_space(1))) u32x4*)(g + off);
#if PKV_NT_LOADS
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

__device__ __forceinline__ float ld_f32(const float* base, int idx) {
  const __attribute__((address_space(1))) float* p = (const __attribute__((address_space(1))) float*)base + idx;
#if PKV_NT_SCALE_LOADS
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}


// Per KV type: pipeline depth (tiles in flight per wave), occupancy target and
// items planned per CU and round.  Measured on MI355X, HBM streams best with
// roughly 14-16 MB outstanding over the chip: 16-bit and f32 KV (8 KB tiles)
// run without prefetch at 8 waves per CU; FP8 (4 KB tiles) keeps two tiles in
// flight at 8 waves per CU; INT8, whose tiles carry more vector work (row
// scales), runs without prefetch at 16 waves per CU; INT4 (1 KB tiles per
// cache) keeps two tiles in flight at 16 waves per CU.  Multi-token calls
// (32 rows per wave, ~170 VGPRs) run at 2 waves per SIMD without prefetch.
// DEEP (INT4 only, chosen by the host when the batch has few units, so that
// half the items still split every unit): 8 items per CU at 2 waves per
// SIMD, two tiles per softmax step and the next two in flight.
template <int KV, bool DEEP = false>
struct Tuning {
  static constexpr bool deep = DEEP && KV == PKV_I4;
  static constexpr int stages =
      deep ? PKV_STAGES_I4_DEEP
           : KV == PKV_I8 ? PKV_STAGES_I8
                          : KV == PKV_I4 ? PKV_STAGES_I4
                                         : (KV == PKV_FP8_E4M3FN ? PKV_STAGES_FP8 : PKV_STAGES_2B);
  static constexpr int waves_per_eu =
      deep ? PKV_WAVES_PER_EU_I4_DEEP
           : KV == PKV_I8 ? 4
                          : (KV == PKV_I4 ? PKV_WAVES_PER_EU_I4
                                          : (KV == PKV_FP8_E4M3FN ? PKV_WAVES_PER_EU_FP8
                                                                  : PKV_WAVES_PER_EU));
  static constexpr int slots_per_cu =
      deep ? PKV_SLOTS_PER_CU_I4_DEEP
           : KV == PKV_I8 ? PKV_SLOTS_PER_CU_I8
                          : (KV == PKV_I4 ? PKV_SLOTS_PER_CU_I4
                                          : (KV == PKV_FP8_E4M3FN ? PKV_SLOTS_PER_CU_FP8
                                                                  : PKV_SLOTS_PER_CU_DEFAULT));
  // Most tiles per item (block-table registers per lane at 16-token blocks:
  // one per 64 tiles).  Longer items keep long contexts to one round of items;
  // INT4 (four times the tiles per byte, each reading its entry) measured
  // slower with 8 registers.
  static constexpr int item_tiles =
      KV == PKV_I4 ? PKV_ITEM_TILES_I4 : (KV == PKV_I8 ? PKV_ITEM_TILES_I8 : kItemTilesMax);
  static_assert(item_tiles >= kItemTilesMin && item_tiles <= kItemTilesMax, "item limit");
  // The host bounds the items of every plan (grid and workspace rows) with the
  // smallest limit of any kernel, kPrefillItemTilesMax: no decode instance may
  // plan shorter items than that.
  static_assert(item_tiles >= kPrefillItemTilesMax, "max_items_bound assumes this limit");
  // Tiles per online-softmax step (their loads are issued together; INT4's PV
  // products then run 32 tokens deep).
  static constexpr int tiles_per_update =
      deep ? PKV_TILES_PER_UPDATE_I4_DEEP
           : KV == PKV_I4 ? PKV_TILES_PER_UPDATE_I4
                          : (KV == PKV_I8 ? PKV_TILES_PER_UPDATE_I8
                                          : (KV == PKV_FP8_E4M3FN ? PKV_TILES_PER_UPDATE_FP8 : 1));
};

// Waves per workgroup: decode takes kDecodeWaves consecutive items (the KV
// heads of one (sequence, chunk)); a multi-token call takes the row tiles of
// one virtual sequence, or kDecodeWaves items when a virtual sequence is one
// wave (then the prep kernel may number a sequence's KV heads chunk by chunk).
__host__ __device__ __forceinline__ int multi_wpg(const DecodeArgs& a, bool multi) {
  return multi && a.head_tiles > 1 ? a.head_tiles : kDecodeWaves;
}

// MULTI: several query tokens per sequence (causal).  The planner then works
// on virtual sequences, one per (sequence, KV head, group of head_tiles 32-row
// tiles of (query token, head of the group) rows), whose context ends at the
// group's last causal limit; a.context_lens holds those lengths and a.vseq_b /
// a.vseq_g / a.vseq_rt say which sequence, KV head and row group each is
// (written by multi_prep_kernel).  A wave takes one 32-row tile; the
// head_tiles waves of a group form one workgroup (multi_wpg).
template <int KV, int QT, int D, int BS, bool MULTI, bool DEEP = false>
__global__ __launch_bounds__(64 * (MULTI && kMultiGroupMax > kDecodeWaves ? kMultiGroupMax
                                                                           : kDecodeWaves))
__attribute__((amdgpu_waves_per_eu(MULTI ? PKV_MULTI_WAVES_PER_EU : Tuning<KV, DEEP>::waves_per_eu)))
void decode_partition_kernel(DecodeArgs a) {
  constexpr int MT = MfmaOf<QT>::value;
  constexpr int eb = dtype_bytes(KV);  // (INT4: handled apart wherever it matters)
  constexpr int R = (int)row_bytes_of(KV, D);   // bytes per stored row
  constexpr int NL = R / 64;           // 16-byte loads per lane per 16-row tile
  using C = Cvt<KV, MT>;
  constexpr int WPC = C::out_words;    // MFMA words per chunk
  constexpr int KW = NL * WPC;         // MFMA words per lane for a K tile (= D/8 or D/4)
  constexpr int NC = D / 16;           // 16-wide d chunks of the output
  constexpr int VG = 4 / eb;           // 16-wide d chunks per 16 bytes of a V lane
  // Query rows per wave, in tiles of 16 (the MFMA's N): 16 for decode, 32 for
  // multi-token calls, whose query tokens x heads of a KV head run to dozens of
  // rows (each loaded K/V tile then serves twice the rows).
  constexpr int RT = MULTI ? kMultiRowTiles : 1;
  constexpr int NT = MULTI ? 1 : Tuning<KV, DEEP>::tiles_per_update;   // tiles per softmax step

  const int lane = threadIdx.x & (kWave - 1);
  const int r16 = lane & 15;   // MFMA row/column index of this lane
  const int c16 = lane >> 4;   // MFMA k-group of this lane

  // ---- which item: contiguous item ranges per XCD (workgroups go round-robin
  // over the 8 XCDs, so blockIdx % 8 is the XCD).  A workgroup's waves take
  // aligned consecutive items.  Multi-token: head_tiles waves, the row tiles of
  // one (virtual sequence, KV head, chunk), which read the same K/V tiles in
  // step, so the copies after the first come from the CU's caches.  Decode:
  // kDecodeWaves waves, the KV heads of one (sequence, chunk), which read
  // adjacent tiles of the same blocks.  The waves share nothing (no LDS, no
  // barrier), so any of them may stop early. ----
  const int wpg = multi_wpg(a, MULTI);               // waves per workgroup
  Plan plan;
  SeqCtx seqs;                                        // (decode: the contexts read once)
  if constexpr (MULTI) {
    plan.items = planned_items(a);                    // made by multi_prep_kernel
    plan.tpi = 0;
  } else {
    plan = make_plan(a, lane, seqs);
  }
  const int64_t groups = (plan.items + wpg - 1) / wpg;
  const int64_t per_xcd = (groups + 7) / 8;
  const int64_t slot_in_xcd = blockIdx.x / 8;
  const int64_t item =
      ((int64_t)(blockIdx.x % 8) * per_xcd + slot_in_xcd) * wpg + (threadIdx.x >> 6);
  if (slot_in_xcd >= per_xcd || item >= plan.items) return;
  int b;
  SeqItems sq;
  if constexpr (MULTI) {
    planned_seq(a, item, b, sq);
  } else {
    if (!seq_of_item(a, plan, seqs, item, lane, b, sq)) return;
  }
  b = uni(b);
  const int local = uni((int)(item - sq.first));   // < m * units per sequence
  // items per chunk: a multi-token call whose virtual sequences are single
  // row groups numbers the KV heads of a sequence chunk by chunk (plan_info[11])
  const int upc = MULTI ? (a.plan_info[11] ? a.num_kv_heads * a.head_tiles : a.head_tiles)
                        : a.plan_heads * a.head_tiles;
  const int g = MULTI ? uni(a.vseq_g[b]) : uni((local % upc) / a.head_tiles);
  const int chunk = uni(local / upc);
  const int ht = uni(local % a.head_tiles);
  const int ctx = uni(sq.ctx);
  const int t_begin = uni((int)((int64_t)chunk * sq.n / sq.m) * kTileTokens);
  int t_end = (int)((int64_t)(chunk + 1) * sq.n / sq.m) * kTileTokens;
  t_end = uni(t_end < ctx ? t_end : ctx);
  const int ntiles = (t_end - t_begin + 15) >> 4;
  const bool whole_unit = sq.m == 1;
  // The first item of each sequence records where its items start and how
  // many each unit has, for the merge kernel (multi-token calls: done by the
  // prep kernel).
  if (!MULTI && a.ws_seq && local == 0 && lane == 0) {
    a.ws_seq[2 * b] = sq.first;
    a.ws_seq[2 * b + 1] = sq.m;
  }

  const int G = a.num_q_heads / a.num_kv_heads;
  bool head_ok[RT];
  int64_t hq[RT];             // this lane's rows of q and out
  int prow[RT];               // last cache position each of this lane's rows may see
  int p_min = 0x7FFFFFFF;     // the smallest such position over the wave's rows
  int bq = b;                 // the real sequence (block table row)
  if constexpr (MULTI) {
    bq = uni(a.vseq_b[b]);
    if (bq < 0) return;                                // padding (never planned: no context)
    const int rt = uni(a.vseq_rt[b]);
    int q0, L;
    query_span(a, bq, q0, L);
    q0 = uni(q0);
    L = uni(L);
    int cr = a.real_ctx[bq];
    cr = uni(cr < 0 ? 0 : (cr > a.ctx_cap ? a.ctx_cap : cr));
    const int row0 = (a.head_tiles * rt + ht) * 16 * RT;   // first row of this wave
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      const int rho = row0 + 16 * k + r16;             // row = query token * G + head
      const int j = rho / G;
      head_ok[k] = rho < L * G && q0 + j < a.q_rows;
      hq[k] = (int64_t)(q0 + j) * a.num_q_heads + g * G + rho % G;
      prow[k] = cr - L + j;
    }
    p_min = cr - L + row0 / G;
    if (__builtin_amdgcn_ballot_w64(head_ok[0]) == 0) return;   // a row tile past the rows
  } else {
    const int h_first = g * G + ht * 16;             // first query head of this tile
    int nh = G - ht * 16;
    nh = nh > 16 ? 16 : nh;
    head_ok[0] = r16 < nh;
    hq[0] = (int64_t)b * a.num_q_heads + h_first + r16;
    prow[0] = 0x7FFFFFFF;
  }
  // Leading tiles of the item that every row sees whole (uniform).
  const int full_end = p_min < t_end ? p_min + 1 : t_end;   // (no overflow at INT_MAX)
  const int nfull = full_end > t_begin ? (full_end - t_begin) >> 4 : 0;

  // Block-table entries of the item, one per lane per register.
  constexpr int NREG =
      (Tuning<KV, DEEP>::item_tiles * kTileTokens / BS + (BS > kTileTokens ? 1 : 0) + 63) / 64;
  const int first_blk = t_begin / BS;
  const int nblk = ntiles > 0 ? (t_end - 1) / BS - first_blk + 1 : 0;   // (empty: an item of zeros)
  int blk[NREG];
#pragma unroll
  for (int r = 0; r < NREG; ++r) {
    const int idx = r * 64 + lane;
    int v = -1;
    if (idx < nblk) v = a.block_tables[(int64_t)bq * a.max_blocks_per_seq + first_blk + idx];
    blk[r] = (v >= a.num_blocks) ? -1 : v;
  }

  // Query operand: lane holds head r16 at the d positions its K chunks carry
  // (the same bytes of q in memory order: 16-byte loads).
  uint32_t qop[RT][KW];
#pragma unroll
  for (int k = 0; k < RT; ++k)
#pragma unroll
    for (int i = 0; i < KW; ++i) qop[k][i] = 0u;
#pragma unroll
  for (int k = 0; k < RT; ++k) {
  if constexpr (KV == PKV_I4 && MT == MT_F32) {
   if (head_ok[k]) {
    // INT4, f32 queries: the lane's K chunk holds d = 32 c16 .. 32 c16 + 31,
    // converted one element per word in that order.
    const uint8_t* src = static_cast<const uint8_t*>(a.q) + (hq[k] * D + 32 * c16) * 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(src + 16 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) qop[k][4 * i + e] = w[e];
    }
   }
  } else if constexpr (KV == PKV_I4) {
   if (head_ok[k]) {
    // INT4: the lane's K chunk holds d = 32 c16 .. 32 c16 + 31; word i of it
    // converts to elements 8 i + (0 4 1 5 2 6 3 7), so q pairs are taken in
    // that order.
    const uint8_t* src = static_cast<const uint8_t*>(a.q) + (hq[k] * D + 32 * c16) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(src + 16 * i);
      qop[k][4 * i + 0] = __builtin_amdgcn_perm(w[2], w[0], 0x05040100u);   // (8i, 8i+4)
      qop[k][4 * i + 1] = __builtin_amdgcn_perm(w[2], w[0], 0x07060302u);   // (8i+1, 8i+5)
      qop[k][4 * i + 2] = __builtin_amdgcn_perm(w[3], w[1], 0x05040100u);   // (8i+2, 8i+6)
      qop[k][4 * i + 3] = __builtin_amdgcn_perm(w[3], w[1], 0x07060302u);   // (8i+3, 8i+7)
    }
   }
  } else if (head_ok[k]) {
    constexpr int qsize = QT == PKV_F32 ? 4 : 2;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int d0 = (64 * j + 16 * c16) / eb;
      const uint8_t* src = static_cast<const uint8_t*>(a.q) + (hq[k] * D + d0) * qsize;
#pragma unroll
      for (int o = 0; o < WPC; o += 4) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(src + 4 * o);
        qop[k][j * WPC + o] = w[0];
        qop[k][j * WPC + o + 1] = w[1];
        qop[k][j * WPC + o + 2] = w[2];
        qop[k][j * WPC + o + 3] = w[3];
      }
    }
  }
  }

  // OffsetCodes — INT8 and INT4 with f16 queries: codes enter the MFMAs as
  // f16 subnormals (q + o) 2^-24 (o = 128 for INT8, 8 for INT4; INT4 high
  // nibbles as (q + 8) 2^-20), which costs one bit operation per word.  Query
  // words that meet INT4 high nibbles are taken at 1/16 (a power of two), so
  // S = 2^24 S_mfma - o sum(q); V comes out as 2^-24 (sum p q + o sum p) (2^-20
  // for INT4's odd column blocks), with sum p (the P values the MFMA saw)
  // from one more MFMA against ones.  The offsets are small next to the sums
  // they are taken from (fp32 keeps about 1e-5 of the result).
  constexpr bool offset_codes = (KV == PKV_I4 || KV == PKV_I8) && MT == MT_F16;
  constexpr float code_offset = KV == PKV_I4 ? 8.0f : 128.0f;
  float qsum[RT];
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    qsum[k] = 0.f;
    if constexpr (offset_codes) {
      const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
#pragma unroll
      for (int i = 0; i < KW; ++i) {
        f16x2 h = __builtin_bit_cast(f16x2, qop[k][i]);
        const bool hi = KV == PKV_I4 && (i & 1);
        if (hi) {
          h = h * sixteenth;
          qop[k][i] = __builtin_bit_cast(uint32_t, h);
        }
        const float t = (float)h[0] + (float)h[1];
        qsum[k] += hi ? 16.f * t : t;
      }
      qsum[k] += __shfl_xor(qsum[k], 16, kWave);
      qsum[k] += __shfl_xor(qsum[k], 32, kWave);
    }
  }

  // Constant factors: logits are taken in the exp2 domain.
  float kfac = a.scale * 1.4426950408889634f;
  float vfac = 1.0f;
  // Offset codes: z = (s - o qsum 2^-24) * (kfac 2^24 / row scale), the first
  // term by starting the QK accumulation at -o qsum 2^-24, the second one
  // factor per token (row-scaled caches: kfac enters the reciprocal once).
  f32x4 s_init[RT];
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    const float b0 = offset_codes ? -code_offset * qsum[k] * 5.9604644775390625e-8f : 0.f;
    s_init[k] = f32x4{b0, b0, b0, b0};
  }
  const float kf_row = offset_codes ? kfac * 16777216.0f : kfac;   // times 1 / row scale
  // Lazy-rescaling slack (log2 units): P <= 2^kSlack.  Row-scaled caches feed
  // P / s to the 16-bit PV operand (1/s = amax/127 for INT8, amax/7 for INT4),
  // so their slack is smaller: with it, P / s stays finite in f16 for every row
  // whose values are finite in f16 (amax <= 65504; INT4: 4 * 65504 / 7).
  constexpr float kSlack = KV == PKV_I4 ? 2.0f : (row_scaled(KV) ? 4.0f : 8.0f);
  if constexpr (KV == PKV_FP8_E4M3FN) {
    kfac *= a.k_scale[0] * cvt_gain<KV, MT>();
    vfac = a.v_scale[0] * cvt_gain<KV, MT>();
  }

  const uint8_t* __restrict__ kbase = static_cast<const uint8_t*>(a.k_cache);
  const uint8_t* __restrict__ vbase = static_cast<const uint8_t*>(a.v_cache);

  f32x4 acc[RT][NC];
  f32x4 acc_p[RT];                      // offset codes: sum of P per head (every row)
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int k = 0; k < RT; ++k) {
#pragma unroll
    for (int nc = 0; nc < NC; ++nc) acc[k][nc] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc_p[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[k] = -__builtin_inff();
    l_run[k] = 0.f;
  }

  // Physical block of a tile (-1: outside the pool, the tile is skipped).
  auto tile_phys = [&](int tile) -> int {
    const int rel = (t_begin + tile * 16) / BS - first_blk;   // uniform
    // Every register read at a constant index (scalar selects), so the array
    // stays in registers.
    int v = __builtin_amdgcn_readlane(blk[0], rel & 63);
#pragma unroll
    for (int r = 1; r < NREG; ++r) {
      const int w = __builtin_amdgcn_readlane(blk[r], rel & 63);
      v = (rel >> 6) == r ? w : v;
    }
    return v;
  };
  // First cache row of a tile in the [NB][Hkv][BS] row space.
  auto tile_row0 = [&](int tile, int phys) -> int64_t {
    phys = phys < 0 ? 0 : phys;
    return ((int64_t)phys * a.num_kv_heads + g) * BS + ((t_begin + tile * 16) % BS);
  };

  // Per-lane byte offset inside a 16-token group (32-bit, so the loads take a
  // scalar group base plus one vector offset).  Both caches are stored in the
  // MFMA operand order, so every load is 1 KB contiguous per instruction.
  const uint32_t loff = (uint32_t)(lane * 16);

  // Issue the loads of one tile into a register set.
  // Row scales (INT8, INT4): lane 16*c + i holds the scale of token 4*c + i (i < 4) of
  // the tile (one register per tile and cache); the lanes that need tokens
  // 4*c16 .. 4*c16+3 fetch them from their row's first four lanes.
  const int scale_tok = 4 * c16 + (r16 & 3);
  auto issue = [&](int tile, u32x4* kr, u32x4* vr, float& ks, float& vs, int& phys) {
    phys = tile_phys(tile);
    const int64_t row0 = tile_row0(tile, phys);
    // Uniform: keep it scalar.  (uni64 moves the two halves as unsigned words;
    // readfirstlane returns a signed int, and widening the low half directly
    // would copy its bit 31 into the high word, past 2^31 bytes into a pool.)
    // The tile bases pass through readfirstlane, so each load takes them as
    // its scalar base with the lane's 32-bit offset (no 64-bit vector add).
    const uint64_t tb = (uint64_t)uni64((int64_t)row0 * R);
    const uint8_t* ktile = sptr(kbase + tb);
    const uint8_t* vtile = sptr(vbase + tb);
#pragma unroll
    for (int j = 0; j < NL; ++j) kr[j] = ld16(ktile, loff + 1024 * j);
#pragma unroll
    for (int j = 0; j < NL; ++j) vr[j] = ld16(vtile, loff + 1024 * j);
    if constexpr (row_scaled(KV)) {
      const uint64_t sb = (uint64_t)uni64(row0);
      ks = ld_f32(sptr(a.k_scale + sb), scale_tok);
      vs = ld_f32(sptr(a.v_scale + sb), scale_tok);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the compute they overlap
  };

  // Softmax update and both contractions for NT loaded tiles: one online-
  // softmax step over their 16 NT tokens (the running max, its cross-lane
  // reduction and the rescale decision are taken once per NT tiles).
  // `checked` (a std::bool_constant): a tile may be partial, outside the pool
  // or past the item, so tokens are masked one by one; otherwise all are live.
  auto compute = [&](auto checked_c, int tile, const u32x4 (*kraw)[NL], const u32x4 (*vraw)[NL],
                     const float* ks1, const float* vs1, const int* phys) {
    constexpr bool checked = decltype(checked_c)::value;
    // INT8 / INT4: 1/s of this lane's scale (v_rcp_f32, ~1 ulp), then each lane
    // takes its four tokens' values from its row's first four lanes (DPP row
    // broadcast of lane i of each 16-lane row).
    auto bcast4 = [&](float x) {
      return f32x4{row_bcast<0>(x), row_bcast<1>(x), row_bcast<2>(x), row_bcast<3>(x)};
    };
    // Live tokens of each tile (<= 0: a tile outside the pool or past the item).
    int n_valid[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      n_valid[t] = 16;
      if constexpr (checked) {
        const int n = t_end - (t_begin + (tile + t) * 16);
        n_valid[t] = phys[t] < 0 ? 0 : (n > 16 ? 16 : n);
      }
    }

    // Tokens 4*c16 + i of this lane past the context get zero V (masks on the
    // converted operands; all ones for a full tile).
    uint32_t vmask[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int vcnt = n_valid[t] - 4 * c16;
#pragma unroll
      for (int i = 0; i < 4; ++i) vmask[t][i] = i < vcnt ? 0xFFFFFFFFu : 0u;
    }

    // S^T = K Q^T
    f32x4 s[NT][RT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint32_t kop[KW];
#pragma unroll
      for (int j = 0; j < NL; ++j) C::run(kraw[t][j], kop + j * WPC);
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        s[t][k] = s_init[k];
        if constexpr (MT == MT_F16) {
#pragma unroll
          for (int c = 0; c < KW / 4; ++c) {
            const u32x4 ka = {kop[4 * c], kop[4 * c + 1], kop[4 * c + 2], kop[4 * c + 3]};
            const u32x4 qb = {qop[k][4 * c], qop[k][4 * c + 1], qop[k][4 * c + 2], qop[k][4 * c + 3]};
            s[t][k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, ka),
                                                             __builtin_bit_cast(f16x8, qb), s[t][k], 0, 0, 0);
          }
        } else if constexpr (MT == MT_BF16) {
#pragma unroll
          for (int c = 0; c < KW / 4; ++c) {
            const u32x4 ka = {kop[4 * c], kop[4 * c + 1], kop[4 * c + 2], kop[4 * c + 3]};
            const u32x4 qb = {qop[k][4 * c], qop[k][4 * c + 1], qop[k][4 * c + 2], qop[k][4 * c + 3]};
            s[t][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka),
                                                              __builtin_bit_cast(bf16x8, qb), s[t][k], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int c = 0; c < KW; ++c)
            s[t][k] = __builtin_amdgcn_mfma_f32_16x16x4f32(bitsf(kop[c]), bitsf(qop[k][c]), s[t][k], 0, 0, 0);
        }
      }
      // (several tiles: one tile's converted K at a time)
      if constexpr (NT > 1) __builtin_amdgcn_sched_barrier(0);
    }
    f32x4 krcp[NT], vrcp[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      krcp[t] = vrcp[t] = f32x4{1.f, 1.f, 1.f, 1.f};
      if constexpr (row_scaled(KV)) {
        krcp[t] = bcast4(__builtin_amdgcn_rcpf(ks1[t]) * kf_row);
        vrcp[t] = bcast4(__builtin_amdgcn_rcpf(vs1[t]));
      }
    }

    // Online softmax (lane: tokens 4*c16 + i of row r16 of each row tile).
    float p[RT][NT][4];
    float m_new[RT], p_sum[RT];
    bool up[RT];
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      float z[NT][4];
      float mx = -__builtin_inff();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (row_scaled(KV))
            z[t][i] = s[t][k][i] * krcp[t][i];   // (kfac, and 2^24 for offset codes, inside)
          else
            z[t][i] = s[t][k][i] * kfac;
          if constexpr (checked) {
            const bool ok =
                4 * c16 + i < n_valid[t] && t_begin + (tile + t) * 16 + 4 * c16 + i <= prow[k];
            z[t][i] = ok ? z[t][i] : -__builtin_inff();
          }
          mx = fmax_ieee(mx, z[t][i]);
        }
      }
      mx = rows_max(mx);
      // Lazy rescaling: the reference max m_run moves only when a tile's max
      // passes it by more than kSlack (log2 units), so most tiles neither
      // rescale nor take an exponential for it.  P is then at most 2^kSlack:
      // the result is the same up to rounding, and the partial (m, l, acc)
      // a split unit leaves stays consistent (l and acc share the reference).
      // -inf + kSlack is -inf, so a row's first live tile always moves it; a
      // row that has seen no live token keeps m_run = -inf and P = 0.
      up[k] = mx > m_run[k] + kSlack;
      m_new[k] = up[k] ? mx : m_run[k];
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // v_exp_f32 directly: results below 2^-126 may flush to zero, which
          // only drops weights under 1e-38 of the largest.
          float e;
          if constexpr (checked)   // (z finite implies m_new finite)
            e = z[t][i] != -__builtin_inff() ? __builtin_amdgcn_exp2f(z[t][i] - m_new[k]) : 0.f;
          else
            e = __builtin_amdgcn_exp2f(z[t][i] - m_new[k]);
          p[k][t][i] = e;
          psum = (t == 0 && i == 0) ? e : psum + e;
        }
      }
      p_sum[k] = psum;
      if constexpr (row_scaled(KV)) {
        // (the guard keeps a masked token's P at 0 even if its slot's scale is NaN)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            p[k][t][i] = (!checked || p[k][t][i] > 0.f) ? p[k][t][i] * vrcp[t][i] : 0.f;
      }
    }
    // Rescale only when some row's reference max moved.
    bool moved = false;
#pragma unroll
    for (int k = 0; k < RT; ++k) moved = moved || up[k];
    if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        const float alpha = up[k] ? __builtin_amdgcn_exp2f(m_run[k] - m_new[k]) : 1.0f;
#pragma unroll
        for (int nc = 0; nc < NC; ++nc) acc[k][nc] *= alpha;
        if constexpr (offset_codes) acc_p[k][0] *= alpha;   // only row 0 is read
        l_run[k] *= alpha;
      }
    }
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      l_run[k] += p_sum[k];
      m_run[k] = m_new[k];
    }

    // O^T += V^T P^T.  Lane 16*c16 + r16 holds, for d = 16*nc + r16, the V values
    // of tokens 4*c16 .. 4*c16+3 (storage order), i.e. the A operand.
    const f16x4 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
    if constexpr (KV == PKV_I4 && NT == 2 && MT != MT_F32) {
      // Two tiles in one 32-deep product per column block: the lane's four
      // tokens of each tile, in the order of the 16-deep form below.
      u32x4 pb[RT];
#pragma unroll
      for (int k = 0; k < RT; ++k)
        pb[k] = u32x4{pack_p<MT>(p[k][0][0], p[k][0][2]), pack_p<MT>(p[k][0][1], p[k][0][3]),
                      pack_p<MT>(p[k][1][0], p[k][1][2]), pack_p<MT>(p[k][1][1], p[k][1][3])};
      // Codes are finite and P is exactly 0 past the context, so no mask.
#pragma unroll
      for (int wd = 0; wd < NC / 2; ++wd) {
        uint32_t w0[4], w1[4];
        C::word(vraw[0][0][wd], w0);
        C::word(vraw[1][0][wd], w1);
        const u32x4 va = {w0[0], w0[2], w1[0], w1[2]}, vb = {w0[1], w0[3], w1[1], w1[3]};
#pragma unroll
        for (int k = 0; k < RT; ++k) {
          if constexpr (MT == MT_F16) {
            acc[k][2 * wd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(f16x8, va), __builtin_bit_cast(f16x8, pb[k]), acc[k][2 * wd], 0, 0, 0);
            acc[k][2 * wd + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(f16x8, vb), __builtin_bit_cast(f16x8, pb[k]), acc[k][2 * wd + 1], 0,
                0, 0);
          } else {
            acc[k][2 * wd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, va), __builtin_bit_cast(bf16x8, pb[k]), acc[k][2 * wd], 0, 0,
                0);
            acc[k][2 * wd + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, vb), __builtin_bit_cast(bf16x8, pb[k]), acc[k][2 * wd + 1], 0,
                0, 0);
          }
        }
      }
      if constexpr (offset_codes) {
        const f16x8 ones8 = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                             (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int k = 0; k < RT; ++k)
          acc_p[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones8, __builtin_bit_cast(f16x8, pb[k]),
                                                            acc_p[k], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if constexpr (KV == PKV_I4 && MT == MT_F32) {
          // Byte b of word wd of the lane's 16 bytes holds token 4 c16 + b of
          // column blocks 2 wd (low nibble) and 2 wd + 1 (high): converted,
          // word 2 b and 2 b + 1.  Codes are finite and P is exactly 0 past the
          // context, so no mask.
#pragma unroll
          for (int wd = 0; wd < NC / 2; ++wd) {
            uint32_t w[8];
            C::word(vraw[t][0][wd], w);
#pragma unroll
            for (int k = 0; k < RT; ++k)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                acc[k][2 * wd] = __builtin_amdgcn_mfma_f32_16x16x4f32(bitsf(w[2 * i]), p[k][t][i],
                                                                      acc[k][2 * wd], 0, 0, 0);
                acc[k][2 * wd + 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                    bitsf(w[2 * i + 1]), p[k][t][i], acc[k][2 * wd + 1], 0, 0, 0);
              }
          }
        } else if constexpr (KV == PKV_I4) {
          // Word wd of the lane's 16 bytes converts to column blocks 2 wd (words
          // 0, 2) and 2 wd + 1 (words 1, 3), each as tokens (0, 2), (1, 3) of the
          // lane's four: P is packed in the same token order.
          u32x2 pb[RT];
#pragma unroll
          for (int k = 0; k < RT; ++k)
            pb[k] = u32x2{pack_p<MT>(p[k][t][0], p[k][t][2]), pack_p<MT>(p[k][t][1], p[k][t][3])};
          // Codes are finite and P is exactly 0 past the context, so no mask.
#pragma unroll
          for (int wd = 0; wd < NC / 2; ++wd) {
            uint32_t w[4];
            C::word(vraw[t][0][wd], w);
            const u32x2 va = {w[0], w[2]}, vb = {w[1], w[3]};
#pragma unroll
            for (int k = 0; k < RT; ++k) {
              if constexpr (MT == MT_F16) {
                acc[k][2 * wd] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                    __builtin_bit_cast(f16x4, va), __builtin_bit_cast(f16x4, pb[k]), acc[k][2 * wd], 0, 0,
                    0);
                acc[k][2 * wd + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                    __builtin_bit_cast(f16x4, vb), __builtin_bit_cast(f16x4, pb[k]), acc[k][2 * wd + 1], 0,
                    0, 0);
              } else {
                acc[k][2 * wd] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                    __builtin_bit_cast(i16x4, va), __builtin_bit_cast(i16x4, pb[k]), acc[k][2 * wd], 0, 0,
                    0);
                acc[k][2 * wd + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                    __builtin_bit_cast(i16x4, vb), __builtin_bit_cast(i16x4, pb[k]), acc[k][2 * wd + 1], 0,
                    0, 0);
              }
            }
          }
          if constexpr (offset_codes) {
#pragma unroll
            for (int k = 0; k < RT; ++k)
              acc_p[k] = __builtin_amdgcn_mfma_f32_16x16x16f16(ones, __builtin_bit_cast(f16x4, pb[k]),
                                                               acc_p[k], 0, 0, 0);
          }
        } else if constexpr (MT == MT_F32) {
#pragma unroll
          for (int nc = 0; nc < NC; ++nc) {
            uint32_t w[4];
            if constexpr (eb == 4) {
#pragma unroll
              for (int i = 0; i < 4; ++i) w[i] = vraw[t][nc][i];
            } else if constexpr (eb == 1) {
              C::word(vraw[t][nc / VG][nc % VG], w);
            } else {
              C::word(vraw[t][nc / VG][2 * (nc % VG)], w);
              C::word(vraw[t][nc / VG][2 * (nc % VG) + 1], w + 2);
            }
#pragma unroll
            for (int k = 0; k < RT; ++k)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc[k][nc] = __builtin_amdgcn_mfma_f32_16x16x4f32(bitsf(w[i] & vmask[t][i]), p[k][t][i],
                                                                  acc[k][nc], 0, 0, 0);
          }
        } else {
          u32x2 pb[RT];
#pragma unroll
          for (int k = 0; k < RT; ++k)
            pb[k] = u32x2{pack_p<MT>(p[k][t][0], p[k][t][1]), pack_p<MT>(p[k][t][2], p[k][t][3])};
          const uint32_t m01 = (vmask[t][0] & 0xFFFFu) | (vmask[t][1] & 0xFFFF0000u);
          const uint32_t m23 = (vmask[t][2] & 0xFFFFu) | (vmask[t][3] & 0xFFFF0000u);
          // uniform: only a sequence's last tile is partial.  INT8 codes are finite
          // and P is exactly 0 past the context: no mask needed.
          const bool full = !checked || n_valid[t] == 16 || KV == PKV_I8;
#pragma unroll
          for (int nc = 0; nc < NC; ++nc) {
            uint32_t w[2];
            if constexpr (eb == 1) {
              C::word(vraw[t][nc / VG][nc % VG], w);
            } else {
              w[0] = vraw[t][nc / VG][2 * (nc % VG)];
              w[1] = vraw[t][nc / VG][2 * (nc % VG) + 1];
            }
            u32x2 va = {w[0], w[1]};
            if (!full) va = u32x2{w[0] & m01, w[1] & m23};
#pragma unroll
            for (int k = 0; k < RT; ++k) {
              if constexpr (MT == MT_F16) {
                acc[k][nc] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, va),
                                                                   __builtin_bit_cast(f16x4, pb[k]),
                                                                   acc[k][nc], 0, 0, 0);
              } else {
                acc[k][nc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, va),
                                                                       __builtin_bit_cast(i16x4, pb[k]),
                                                                       acc[k][nc], 0, 0, 0);
              }
            }
          }
          if constexpr (offset_codes) {
#pragma unroll
            for (int k = 0; k < RT; ++k)
              acc_p[k] = __builtin_amdgcn_mfma_f32_16x16x16f16(ones, __builtin_bit_cast(f16x4, pb[k]),
                                                               acc_p[k], 0, 0, 0);
          }
        }
      }
    }
  };

  // S-deep pipeline over groups of NT tiles: group i lives in register set
  // i % S; while it is multiplied, groups i+1 .. i+S-1 are in flight.  1-byte
  // KV tiles carry half the bytes of 16-bit ones, so they keep more in flight.
  // The steady state has no branch around the loads (a load issued on one
  // path only would make the wait counts conservative); a short tail follows.
  constexpr int S = MULTI ? PKV_STAGES_MULTI : Tuning<KV, DEEP>::stages;
  u32x4 kr[S][NT][NL], vr[S][NT][NL];
  float ks[S][NT], vs[S][NT];
  int ph[S][NT];   // physical block of each tile in each register set (-1: skipped)
#pragma unroll
  for (int i = 0; i < S; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      ks[i][t] = vs[i][t] = 1.f;
      ph[i][t] = -1;
    }
  // Loads of group gr into register set st; `guarded`: tiles past the item
  // (only in an item's last group) are not loaded.
  auto issue_group = [&](int gr, int st, bool guarded) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tl = gr * NT + t;
      if (!guarded || tl < ntiles)
        issue(tl, kr[st][t], vr[st][t], ks[st][t], vs[st][t], ph[st][t]);
      else
        ph[st][t] = -1;
    }
  };
  // The steady loop takes only groups that every row sees whole and never an
  // item's last group (the only one that can be partial), so its tiles take
  // the unchecked path.  An item whose table has an entry outside the pool
  // (whose tiles are skipped) and the tail take the checked path.
  bool bad_entry = false;
#pragma unroll
  for (int r = 0; r < NREG; ++r) bad_entry = bad_entry || (r * 64 + lane < nblk && blk[r] < 0);
  const bool table_ok = __builtin_amdgcn_ballot_w64(bad_entry) == 0;
  const int ngroups = (ntiles + NT - 1) / NT;
  int gr = 0;
  if (ngroups > 2 * S - 1) {
#pragma unroll
    for (int i = 0; i < S - 1; ++i) issue_group(i, i, false);
    if (table_ok) {
      for (; gr + 2 * S - 1 < ngroups && (gr + S) * NT <= nfull; gr += S) {
#pragma unroll
        for (int i = 0; i < S; ++i) {
          const int nx = (i + S - 1) % S;
          issue_group(gr + i + S - 1, nx, false);
          compute(std::false_type{}, (gr + i) * NT, kr[i], vr[i], ks[i], vs[i], ph[i]);
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < S - 1; ++i)
      if (i < ngroups) issue_group(i, i, true);
  }
  for (; gr < ngroups; gr += S) {
#pragma unroll
    for (int i = 0; i < S; ++i) {
      if (gr + i < ngroups) {
        const int nx = (i + S - 1) % S;
        if (gr + i + S - 1 < ngroups) issue_group(gr + i + S - 1, nx, true);
        compute(std::true_type{}, (gr + i) * NT, kr[i], vr[i], ks[i], vs[i], ph[i]);
      }
    }
  }

  // ---- epilogue ----
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    float l_tot = l_run[k] + __shfl_xor(l_run[k], 16, kWave);
    l_tot += __shfl_xor(l_tot, 32, kWave);
    if (!head_ok[k]) continue;
    if constexpr (offset_codes) {
#pragma unroll
      for (int nc = 0; nc < NC; ++nc)
        acc[k][nc] = acc[k][nc] * ((KV == PKV_I4 && (nc & 1)) ? 1048576.0f : 16777216.0f) -
                     code_offset * acc_p[k][0];
    }
    if (whole_unit) {
      // (l_tot = 0 only for a row that sees no token: its output is zeros)
      const float inv = l_tot > 0.f ? vfac / l_tot : 0.f;
#pragma unroll
      for (int nc = 0; nc < NC; ++nc)
        store_out4<QT>(a.out, hq[k] * D + nc * 16 + c16 * 4, acc[k][nc][0] * inv,
                       acc[k][nc][1] * inv, acc[k][nc][2] * inv, acc[k][nc][3] * inv);
    } else if (item < a.max_items) {
      const int64_t slot = item * (16 * RT) + 16 * k + r16;   // partial row of this item and row
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

// ---------------------------------------------------------------------------
// Merge of a unit's items: out = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c.
// The item kernel recorded each (virtual) sequence's first item and items per
// unit.  D/4 lanes cover one partial row with 16-byte loads, so one load
// instruction takes 64/(D/4) items at once; the lane groups are added in a
// fixed order at the end (results do not depend on timing).  A unit that was
// one item was finished by the item kernel.
// ---------------------------------------------------------------------------
// One output row from its m partial rows row0 + c * row_step (a row that saw
// no token in any item, M = -inf, gets zeros).
// Fast path of merge_row: up to NV * (64 / (D / 4)) partials are held in NV
// registers of 4 floats after one round of loads.  The decode merge (one wave
// per (head, sequence)) takes 16; the multi-token merge (a wave per row, many
// more waves) takes 4, which keeps it at 8 resident waves per SIMD.
template <int QT, int D, int NV>
__device__ __forceinline__ void merge_row(const DecodeArgs& a, int64_t row0, int64_t row_step,
                                          int m, int64_t hq, int lane) {
  constexpr int LPP = D / 4;          // lanes per partial row
  constexpr int PPI = kWave / LPP;    // partials per load instruction
  const int grp = lane / LPP;         // which partial of an instruction
  const int dq = lane % LPP;          // which 4 output elements
  if (m <= NV * PPI) {
    // Up to NV * PPI partials: every (max, sum) and every output row is
    // loaded in one round, before any of them is used (the general path
    // below needs the maxima before it reads the rows).  Same sums in the
    // same order, so the same result.
    float mc = -__builtin_inff(), lc = 0.f;
    if (lane < m) {
      const int64_t row = row0 + lane * row_step;
      mc = a.ws_ml[2 * row];
      lc = a.ws_ml[2 * row + 1];
    }
    f32x4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = i * PPI + grp;
      v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (c < m) v[i] = *reinterpret_cast<const f32x4*>(a.ws_acc + (row0 + c * row_step) * D + 4 * dq);
    }
    const float M = wave_max(mc);
    if (M == -__builtin_inff()) {
      if (grp == 0) store_out4<QT>(a.out, hq * D + 4 * dq, 0.f, 0.f, 0.f, 0.f);
      return;
    }
    const float L = wave_sum(lane < m ? __builtin_amdgcn_exp2f(mc - M) * lc : 0.f);
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = i * PPI + grp;
      const float mi = __shfl(mc, c < m ? c : 0, kWave);
      if (c < m) o += __builtin_amdgcn_exp2f(mi - M) * v[i];
    }
#pragma unroll
    for (int off = LPP; off < kWave; off <<= 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] += __shfl_xor(o[i], off, kWave);
    }
    if (grp != 0) return;
    const float inv = 1.0f / L;
    store_out4<QT>(a.out, hq * D + 4 * dq, o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    return;
  }
  float M = -__builtin_inff();
  for (int c = lane; c < m; c += kWave) M = fmaxf(M, a.ws_ml[2 * (row0 + c * row_step)]);
  M = wave_max(M);
  if (M == -__builtin_inff()) {
    if (grp == 0) store_out4<QT>(a.out, hq * D + 4 * dq, 0.f, 0.f, 0.f, 0.f);
    return;
  }
  float L = 0.f;
  for (int c = lane; c < m; c += kWave) {
    const int64_t row = row0 + c * row_step;
    L += __builtin_amdgcn_exp2f(a.ws_ml[2 * row] - M) * a.ws_ml[2 * row + 1];
  }
  L = wave_sum(L);

  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int c0 = 0; c0 < m; c0 += PPI) {
    const int c = c0 + grp;
    if (c < m) {
      const int64_t row = row0 + c * row_step;
      const float w = __builtin_amdgcn_exp2f(a.ws_ml[2 * row] - M);
      const f32x4 v = *reinterpret_cast<const f32x4*>(a.ws_acc + row * D + 4 * dq);
      o += w * v;
    }
  }
#pragma unroll
  for (int off = LPP; off < kWave; off <<= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] += __shfl_xor(o[i], off, kWave);
  }
  if (grp != 0) return;
  const float inv = 1.0f / L;
  store_out4<QT>(a.out, hq * D + 4 * dq, o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
}

// Decode: one wave per (query head, sequence).  Launched only when a unit may
// be split (a workspace); units that were one item, empty sequences
// included, were finished by the partition kernel.
template <int QT, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int64_t hq = (int64_t)b * a.num_q_heads + h;
  const int64_t first = a.ws_seq[2 * b];
  const int m = (int)a.ws_seq[2 * b + 1];
  if (m <= 1) return;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int g = h / G;
  const int ht = (h % G) / 16;
  const int r = (h % G) % 16;
  // Partial row of chunk c: item (first + (c*plan_heads + g)*head_tiles + ht), head r.
  const int64_t upc = (int64_t)a.plan_heads * a.head_tiles;
  if (first + ((int64_t)(m - 1) * a.plan_heads + g) * a.head_tiles + ht >= a.max_items) return;
  merge_row<QT, D, 16>(a, (first + (int64_t)g * a.head_tiles + ht) * 16 + r, upc * 16, m, hq,
                       lane);
}

// Several query tokens per sequence: one workgroup of 8 waves per virtual
// sequence (sequence, KV head, group of 32-row tiles of (query token, head)
// rows), each wave merging every 8th row; rows of a virtual sequence with no context (rows
// before the cache) get zeros.  Only the virtual sequences of the prep kernel's
// merge list are visited by prompt-chunk calls (units cut into several
// items, or no context): a call whose units were all whole items launches
// this kernel and ends it at once.  The decode-shaped kernel's calls keep one
// workgroup column per virtual sequence.
constexpr int kMergeWaves = 8;
constexpr int kMergeGroups = 512;   // workgroups along x; each takes every 512th list entry
template <int QT, int D>
__device__ __forceinline__ void merge_vseq(const DecodeArgs& a, int v) {
  const int TR = a.wave_rows;                 // rows of a wave's tile
  const int ROWS = TR * a.head_tiles;         // rows of a virtual sequence
  const int g = a.vseq_g[v];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int bq = a.vseq_b[v];
  if (bq < 0) return;                 // a padding entry
  const int64_t row0 = (int64_t)ROWS * a.vseq_rt[v];   // first row of this virtual sequence
  int q0, L;
  query_span(a, bq, q0, L);
  int64_t rows = (int64_t)L * G - row0;
  rows = rows > ROWS ? ROWS : rows;
  // rows past the query tensor (inconsistent query_start) are never written
  const int64_t rows_q = (int64_t)(a.q_rows - q0) * G - row0;
  rows = rows < rows_q ? rows : rows_q;
  if (rows <= 0) return;
  auto out_row = [&](int r) -> int64_t {
    const int64_t rho = row0 + r;
    return (q0 + rho / G) * a.num_q_heads + g * G + rho % G;
  };
  // Rows r = blockIdx.y * kMergeWaves + wave + k * kMergeWaves * gridDim.y: a
  // second grid dimension gives every wave one row when rows per virtual
  // sequence are few and split many times (each row's merge is a chain of
  // dependent loads).
  const int r_first = blockIdx.y * kMergeWaves + wave;
  const int r_step = kMergeWaves * gridDim.y;
  if (seq_ctx(a, v) == 0) {
    for (int r = r_first; r < rows; r += r_step)
      if (lane < D / 4) store_out4<QT>(a.out, out_row(r) * D + 4 * lane, 0.f, 0.f, 0.f, 0.f);
    return;
  }
  if (!a.ws_seq) return;
  const int64_t first = a.ws_seq[2 * v];
  const int m = (int)a.ws_seq[2 * v + 1];
  if (m <= 1) return;
  // (one KV head per virtual sequence) chunk c, row tile ht: item
  // first + c*S + ht with S items per chunk (head_tiles, or the KV heads of the
  // sequence when they are numbered chunk by chunk), rows item*TR ..
  const int64_t S = a.plan_info[11] ? (int64_t)a.num_kv_heads * a.head_tiles : a.head_tiles;
  if (first + (int64_t)(m - 1) * S + a.head_tiles - 1 >= a.max_items) return;
  for (int r = r_first; r < rows; r += r_step)
    merge_row<QT, D, 4>(a, (first + r / TR) * TR + r % TR, S * TR, m, out_row(r), lane);
}
// (the decode-shaped kernel's calls: few virtual sequences, most of them
// split; one workgroup column per virtual sequence, no list to read first)
template <int QT, int D>
__global__ __launch_bounds__(64 * kMergeWaves) void multi_merge_kernel(DecodeArgs a) {
  merge_vseq<QT, D>(a, blockIdx.x);
}
// (prompt chunks: the virtual sequences of the merge list)
template <int QT, int D>
__global__ __launch_bounds__(64 * kMergeWaves) void prefill_merge_kernel(DecodeArgs a) {
  const int64_t n = a.plan_info[12];          // entries of the merge list
  for (int64_t i = blockIdx.x; i < n; i += gridDim.x) merge_vseq<QT, D>(a, a.merge_list[i]);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS
// round trips): Hillis-Steele within each row of 16 lanes (row_shr 1, 2, 4,
// 8; a source before the row's first lane reads 0), then lane 15 of rows 0
// and 2 added to rows 1 and 3 (row_bcast 15), then lane 31 to rows 2 and 3
// (row_bcast 31).  Rows left out by the row mask keep their value.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}

// Largest value over the 64 lanes of a wave, the same DPP pattern as the scan.
__device__ __forceinline__ int wave_max(int x) {
  auto mx = [](int p, int q) { return p > q ? p : q; };
  x = mx(x, __builtin_amdgcn_update_dpp(x, x, 0x111, 0xf, 0xf, false));   // row_shr:1
  x = mx(x, __builtin_amdgcn_update_dpp(x, x, 0x112, 0xf, 0xf, false));   // row_shr:2
  x = mx(x, __builtin_amdgcn_update_dpp(x, x, 0x114, 0xf, 0xf, false));   // row_shr:4
  x = mx(x, __builtin_amdgcn_update_dpp(x, x, 0x118, 0xf, 0xf, false));   // row_shr:8
  x = mx(x, __builtin_amdgcn_update_dpp(x, x, 0x142, 0xa, 0xf, false));   // row_bcast:15
  x = mx(x, __builtin_amdgcn_update_dpp(x, x, 0x143, 0xc, 0xf, false));   // row_bcast:31
  return __builtin_amdgcn_readlane(x, kWave - 1);
}

// Inclusive prefix sums of two ints per thread over a 1024-thread block:
// scans within each wave, then the 16 wave totals (two barriers in all);
// tot_x, tot_y get the block totals.  wtot: LDS, [16][2].
__device__ __forceinline__ void block_scan2(int& x, int& y, int (*wtot)[2], int& tot_x, int& tot_y) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  x = wave_incl_scan(x);
  y = wave_incl_scan(y);
  if (lane == kWave - 1) {
    wtot[w][0] = x;
    wtot[w][1] = y;
  }
  __syncthreads();
  int ox = 0, oy = 0;
  tot_x = tot_y = 0;
#pragma unroll
  for (int i = 0; i < 1024 / kWave; ++i) {
    const int a = wtot[i][0], b = wtot[i][1];
    if (i < w) {
      ox += a;
      oy += b;
    }
    tot_x += a;
    tot_y += b;
  }
  x += ox;
  y += oy;
  __syncthreads();   // (wtot is reused by the next call)
}

// x / d for x >= 0 and a uniform d > 0, by a shift when d is a power of two
// (sh = log2 d, else -1).  The prep kernel runs on one compute unit with four
// waves per SIMD, so every vector instruction costs; integer division is tens.
__device__ __forceinline__ int div_by(int x, int d, int sh) { return sh >= 0 ? x >> sh : x / d; }
__device__ __forceinline__ int log2_if_pow2(int d) { return (d & (d - 1)) == 0 ? __builtin_ctz(d) : -1; }

// Virtual sequences of a multi-token call (one workgroup): for sequence b, each
// KV head times each group of row tiles, with the context the group's last row
// may see; entries past the last are padding with no context.  Decode-shaped
// calls number them KV head major (the workgroups running together on an XCD,
// which take items in numbering order, share one head's K/V in its L2).  Prompt
// chunks number them row group major, so the KV heads of one row group, which
// share its context and hence its tiles, chunks and place in the order of
// groups, are adjacent: the plan below then takes one row group at a time
// instead of each of its KV heads (the one-workgroup kernel's work drops by
// the KV head count).  Sequences go 1024 at a time: a block scan gives each
// its first entry, then every thread fills entries, finding its sequence by
// binary search over the scan.
__global__ __launch_bounds__(1024) void multi_prep_kernel(DecodeArgs a, int batch_real,
                                                          int32_t* vctx) {
  __shared__ int scan[1024];   // inclusive: entries of sequences b0 .. b0 + t
  __shared__ int seq_len[1024], seq_cx[1024];   // new tokens and context of sequence b0 + t
  constexpr int kCtxCache = 4096;               // contexts of the first virtual sequences
  __shared__ int vctx_s[kCtxCache];
  __shared__ int carry;
  __shared__ int several_groups;               // some sequence has more than one row group
  __shared__ int wtot[1024 / kWave][2];
  const int t = threadIdx.x;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int ROWS = a.wave_rows * a.head_tiles;   // rows of a virtual sequence
  const int g_sh = log2_if_pow2(G), rows_sh = log2_if_pow2(ROWS);
  const int H = a.num_kv_heads, h_sh = log2_if_pow2(H);
  const bool by_row_group = a.prefill;   // numbering (row group, KV head)
  if (t == 0) carry = several_groups = 0;
  __syncthreads();
  for (int b0 = 0; b0 < batch_real; b0 += 1024) {
    const int b = b0 + t;
    int L = 0, cx = 0;
    if (b < batch_real) {
      // (query_start is a precondition; clamped so that a bad entry cannot
      // make a count overflow or an index leave its array: 0 <= L <= q_rows)
      int q0;
      query_span(a, b, q0, L);
      cx = a.real_ctx[b];
      cx = cx < 0 ? 0 : (cx > a.ctx_cap ? a.ctx_cap : cx);
    }
    seq_len[t] = L;
    seq_cx[t] = cx;
    // (L * G < 2^31: the host limits q_rows * G)
    const int ng = div_by(L * G + ROWS - 1, ROWS, rows_sh);   // row groups of the sequence
    // (one atomic per wave: an atomic on one LDS address from many lanes is
    // turned into a loop over the lanes)
    if (__builtin_amdgcn_ballot_w64(ng > 1) != 0 && (t & (kWave - 1)) == 0) atomicOr(&several_groups, 1);
    const int64_t n64 = (int64_t)a.num_kv_heads * ng;
    // (KV head, row group) entries; past a.batch (the host's bound) nothing is
    // written, so the count is capped there
    int n = (int)(n64 < a.batch ? n64 : a.batch);
    int unused = 0, total = 0, unused_tot = 0;
    block_scan2(n, unused, wtot, total, unused_tot);
    scan[t] = n;                             // inclusive
    __syncthreads();
    const int base = carry;
    for (int e = t; e < total; e += 1024) {
      const int64_t v64 = (int64_t)base + e;
      if (v64 < 0 || v64 >= a.batch) break;
      const int v = (int)v64;
      // first sequence whose scan passes e (among this block's sequences)
      int lo = 0, hi = batch_real - b0 - 1 < 1023 ? batch_real - b0 - 1 : 1023;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (scan[mid] > e) hi = mid; else lo = mid + 1;
      }
      const int bb = b0 + lo;
      const int Lb = seq_len[lo];
      const int ng = div_by(Lb * G + ROWS - 1, ROWS, rows_sh);   // row groups of the sequence
      const int local = e - (lo > 0 ? scan[lo - 1] : 0);
      int gg, rt;
      if (by_row_group) {
        rt = div_by(local, H, h_sh);
        gg = local - rt * H;
      } else {
        gg = ng == 1 ? local : local / ng;
        rt = local - gg * ng;
      }
      const int ctx = seq_cx[lo];
      int last = ROWS * rt + ROWS - 1;
      last = last < Lb * G - 1 ? last : Lb * G - 1;
      int c = ctx - Lb + div_by(last, G, g_sh) + 1;
      c = c < 0 ? 0 : c;
      vctx[v] = c;
      // (LDS copy: per row group when numbered by row groups, else per entry)
      if (by_row_group) {
        const int r = div_by(v, H, h_sh);
        if (gg == 0 && r < kCtxCache) vctx_s[r] = c;
      } else if (v < kCtxCache) {
        vctx_s[v] = c;
      }
      a.vseq_b[v] = bb;
      a.vseq_rt[v] = rt;
      a.vseq_g[v] = gg;
    }
    __syncthreads();
    if (t == 0) {
      int64_t c = (int64_t)base + total;
      carry = (int)(c < 0 ? 0 : (c > a.batch ? a.batch : c));
    }
    __syncthreads();
  }
  for (int v = carry + t; v < a.batch; v += 1024) {
    vctx[v] = 0;
    a.vseq_b[v] = -1;            // padding: no sequence, no rows
    a.vseq_rt[v] = 0;
    a.vseq_g[v] = 0;
  }

  // ---- the plan, once for every kernel of the call: make_plan's rule over
  // all virtual sequences (one KV head each, head_tiles units), then each
  // one's items numbered and mapped back to it.  It runs over planning units:
  // row groups, each standing for its wt = H adjacent virtual sequences, when
  // numbered by row groups; else single virtual sequences (wt = 1).  (Only
  // this workgroup reads what was written above: the barrier's workgroup-scope
  // fence makes it visible.)  Padding entries (from carry on) have no context,
  // hence no tiles and no items, and nothing reads their plan: the loops
  // below stop at carry. ----
  __syncthreads();
  const int nv = carry;
  // (every sequence's entry count is a multiple of H, and so is a.batch (the
  // host's bound), hence carry: the row groups are whole)
  const int wt = by_row_group ? H : 1;
  const int nu = by_row_group ? div_by(nv, H, h_sh) : nv;   // planning units
  __shared__ int64_t red[2][1024 / kWave];
  __shared__ int64_t carry_items;
  __shared__ int carry_mrg;                    // entries of the merge list so far
  // Prompt-chunk groups by size: key 256 - tiles, at least 0 (a group holds
  // 1 .. kItemTilesMax tiles); per key, the first free position of the order,
  // and each wave's count of the current round.
  constexpr int kKeys = 256;
  __shared__ int key_next[kKeys];
  __shared__ int key_wave[1024 / kWave][kKeys];
  __shared__ int wave_rounds[1024 / kWave];    // most groups of one unit, per wave
  __shared__ int pos_s[1024], grp_s[1024];     // a round's place and group of unit u0 + t
  const int units = a.head_tiles;
  // (contexts of the first kCtxCache units from LDS, the rest from the
  // workspace: a row group's is its first virtual sequence's)
  auto ctx_of = [&](int u) { return u < kCtxCache ? vctx_s[u] : seq_ctx(a, u * wt); };
  int64_t tiles = 0, live = 0;
  for (int u = t; u < nu; u += 1024) {
    const int n = (ctx_of(u) + kTileTokens - 1) / kTileTokens;
    tiles += n;
    live += n > 0;
  }
  // Wave sums by DPP scans in 32-bit pieces: live counts fit; tiles as 24-bit
  // low and high parts (a thread's tiles stay under 2^48, so each part's sum
  // over 64 lanes stays under 2^30).
  {
    const int lo = __builtin_amdgcn_readlane(wave_incl_scan((int)(tiles & 0xFFFFFF)), kWave - 1);
    const int hi = __builtin_amdgcn_readlane(wave_incl_scan((int)(tiles >> 24)), kWave - 1);
    tiles = ((int64_t)hi << 24) + lo;
    live = __builtin_amdgcn_readlane(wave_incl_scan((int)live), kWave - 1);
  }
  if ((t & (kWave - 1)) == 0) {
    red[0][t / kWave] = tiles;
    red[1][t / kWave] = live;
  }
  if (t == 0) carry_items = 0, carry_mrg = 0;
  if (t < kKeys) key_next[t] = 0;
  for (int i = t; i < (1024 / kWave) * kKeys; i += 1024) (&key_wave[0][0])[i] = 0;
  __syncthreads();
  tiles = live = 0;
  for (int w = 0; w < 1024 / kWave; ++w) {
    tiles += red[0][w];
    live += red[1][w];
  }
  tiles *= wt;
  live *= wt;
  // The prompt-chunk kernel is bound by its products, not by HBM: once the
  // units fill a round of slots, items take whole contexts up to the item
  // limit (fewer partial rows to write and merge); otherwise make_plan's rule.
  // (the prompt-chunk kernel reads its block-table entries with scalar loads,
  // so its items are not limited by registers of entries: up to kItemTilesMax;
  // groups of more than kKeys - 1 tiles all sort first, in numbering order)
  const int cap = a.prefill ? kItemTilesMax : a.item_cap;
  const int tpi = a.prefill && live * units >= a.slots
                      ? cap
                      : plan_tpi(tiles * units, live * units, a.slots, cap);
  // When every virtual sequence is one wave and one row group, the KV heads of
  // a sequence are consecutive virtual sequences with one context, hence one
  // chunk count m: their items are numbered chunk by chunk (item = F + c*Hkv +
  // g), so a workgroup's waves read the same blocks' adjacent (block, head)
  // tiles, as in decode.  Otherwise each virtual sequence's items are
  // consecutive, and a row group's H virtual sequences' items follow one
  // another.
  const bool by_chunk = !a.prefill && a.head_tiles == 1 && several_groups == 0;
  // The prompt-chunk kernel takes its groups (the units of one chunk of one
  // virtual sequence, one workgroup each) in decreasing order of their tiles:
  // the hardware starts workgroups in grid order as others finish and deals
  // them round-robin over the 8 XCDs, so this is longest-first list scheduling
  // on every XCD, with the sizes spread evenly over the XCDs.  (Left in
  // numbering order, the longest sequences' groups filled whole XCDs and
  // finished one round after the rest.)  Groups of one size keep numbering
  // order, so the KV heads of one row group sit side by side and, with as many
  // KV heads as XCDs, each XCD reads one head's K/V.  A stable counting sort
  // over planning units (a row group's H groups of a chunk take H adjacent
  // places): the sizes first, then the groups placed round by round below.
  const bool order_groups = a.prefill && a.group_order != nullptr;
  const int tpi_sh = log2_if_pow2(tpi);   // (the prompt-chunk kernel's tpi is 256)
  // Tiles of chunk c of a unit's n tiles cut into m chunks: floor((c+1)n/m) -
  // floor(cn/m), = q + floor((c+1)r/m) - floor(cr/m) with n = qm + r, in 32-bit
  // arithmetic while (c+1)r < 2^32 (m <= 65535), else in 64-bit.
  auto group_tiles = [](int n, int m, int c) {
    if (m == 1) return n;
    if (m <= 65535) {
      const uint32_t um = (uint32_t)m, q = (uint32_t)n / um, r = (uint32_t)n - q * um;
      return (int)(q + ((uint32_t)(c + 1) * r) / um - ((uint32_t)c * r) / um);
    }
    return (int)((int64_t)(c + 1) * n / m - (int64_t)c * n / m);
  };
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  const uint64_t below = (1ull << lane) - 1;
  // Lanes of this wave whose key equals this lane's, among the lanes in
  // `peers` (8 ballots over the bits of the key).
  auto same_key = [](uint64_t peers, int key) {
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t on = __builtin_amdgcn_ballot_w64(((key >> bit) & 1) != 0);
      peers &= ((key >> bit) & 1) ? on : ~on;
    }
    return peers;
  };
  int rounds = 0;   // most groups of one unit (order_groups only)
  if (order_groups) {
    // Groups per size, in planning units: one LDS atomic per (wave, size), by
    // the size's first lane (the sizes of many groups are equal: per-lane
    // atomics on one address serialise).
    int my_rounds = 0;
    for (int u0 = 0; u0 < nu; u0 += 1024) {
      const int u = u0 + t;
      int n = 0, m = 0;
      if (u < nu) {
        n = (ctx_of(u) + kTileTokens - 1) / kTileTokens;
        m = div_by(n + tpi - 1, tpi, tpi_sh);
      }
      my_rounds = m > my_rounds ? m : my_rounds;
      for (int c = 0; __builtin_amdgcn_ballot_w64(c < m) != 0; ++c) {
        const bool has = c < m;
        int key = has ? kKeys - group_tiles(n, m, c) : 0;
        key = key < 0 ? 0 : (key > kKeys - 1 ? kKeys - 1 : key);
        const uint64_t peers = same_key(__builtin_amdgcn_ballot_w64(has), key);
        if (has && (peers & below) == 0) atomicAdd(&key_next[key], __builtin_popcountll(peers));
      }
    }
    my_rounds = wave_max(my_rounds);
    if (lane == 0) wave_rounds[wave] = my_rounds;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 1024 / kWave; ++w) rounds = wave_rounds[w] > rounds ? wave_rounds[w] : rounds;
    const int cnt0 = t < kKeys ? key_next[t] : 0;
    int x = cnt0, y = 0, tx, ty;
    block_scan2(x, y, wtot, tx, ty);           // (ends with a barrier)
    // (groups of larger sizes come first; a unit's groups are wt groups.  The
    // count stays under 2^31: groups are counted in int32 on the host)
    if (t < kKeys) key_next[t] = (x - cnt0) * wt;
    __syncthreads();
  }
  for (int u0 = 0; u0 < nu; u0 += 1024) {
    const int u = u0 + t;
    int m = 0, n = 0;
    if (u < nu) {
      n = (ctx_of(u) + kTileTokens - 1) / kTileTokens;
      m = div_by(n + tpi - 1, tpi, tpi_sh);
    }
    const int cnt = m * units;                 // items of each of the unit's virtual sequences
    // (merge: a unit cut into several items, or no context: rows of zeros)
    const int mrg = u < nu && (m > 1 || n == 0) ? 1 : 0;
    int inc_items = cnt, inc_mrg = mrg, tot_items = 0, tot_mrg = 0;
    block_scan2(inc_items, inc_mrg, wtot, tot_items, tot_mrg);
    // first item of the unit's first virtual sequence; its k-th follows at
    // first + k * cnt.  The unit's first item, chunks and merge-list place go
    // through LDS (the sequence arrays of the first phase, no longer used) to
    // one thread per virtual sequence, whose stores are then adjacent.
    int64_t first = 0;
    if (u < nu) {
      first = carry_items + (int64_t)wt * (inc_items - cnt);
      scan[t] = (int)first;                    // (< 2^31: items are counted in int32 on the host)
      seq_len[t] = m;
      seq_cx[t] = mrg ? carry_mrg + wt * (inc_mrg - 1) : -1;
    }
    __syncthreads();
    const int nb = nu - u0 < 1024 ? nu - u0 : 1024;   // units of this block
    for (int j = t; j < wt * nb; j += 1024) {
      const int uj = by_row_group ? div_by(j, H, h_sh) : j;
      const int k = j - uj * wt;                 // the unit's k-th virtual sequence
      const int v = u0 * wt + j;
      const int mj = seq_len[uj];
      const int cj = mj * units;
      if (seq_cx[uj] >= 0) a.merge_list[seq_cx[uj] + k] = v;
      int64_t f = scan[uj] + (int64_t)k * cj;
      int64_t step = 1;
      if (by_chunk) {
        // (the scan gave F + g*m; the sequence's group starts at F)
        const int g = a.vseq_g[v];
        f -= (int64_t)g * (mj - 1);
        step = a.num_kv_heads;
      }
      a.vseq_first[v] = (int32_t)f;
      a.vseq_m[v] = mj;
      if (a.ws_seq) *reinterpret_cast<i64x2*>(a.ws_seq + 2 * v) = i64x2{f, mj};   // (16-byte aligned)
      // The item map.  The prompt-chunk kernel reads only each group's first
      // item (a group is the units items of one chunk), so prompt chunks write
      // those alone: the map's stores are most of this one compute unit's
      // memory traffic.
      if (a.prefill) {
        for (int c = 0; c < mj && f + c * units < a.map_cap; ++c) a.item_vseq[f + c * units] = v;
      } else {
        for (int i = 0; i < cj && f + i * step < a.map_cap; ++i) a.item_vseq[f + i * step] = v;
      }
    }
    if (order_groups) {
      // Round c places chunk c of every unit of this block: the unit's rank
      // among the round's units of its size comes from ballots (lanes of equal
      // key, in lane order) and the counts of the waves before; its wt groups
      // take wt adjacent places, written by wt adjacent threads (the place and
      // group number go through LDS).
      for (int c = 0; c < rounds; ++c) {
        const bool has = u < nu && c < m;
        int key = has ? kKeys - group_tiles(n, m, c) : 0;
        key = key < 0 ? 0 : (key > kKeys - 1 ? kKeys - 1 : key);   // (256 tiles or more: key 0)
        const uint64_t peers = same_key(__builtin_amdgcn_ballot_w64(has), key);
        if (has && (peers & below) == 0) key_wave[wave][key] = __builtin_popcountll(peers);
        __syncthreads();
        if (u < nu) {
          int pos = -1;
          if (has) {
            // (the 16 reads are independent: unrolled, they are in flight together)
            int rank = __builtin_popcountll(peers & below);
#pragma unroll
            for (int w = 0; w < 1024 / kWave; ++w) rank += w < wave ? key_wave[w][key] : 0;
            pos = key_next[key] + rank * wt;
          }
          pos_s[t] = pos;
          // (first < 2^31: items are counted in int32 on the host; the group
          // of virtual sequence k of the unit is (first + k*cnt) / units + c)
          grp_s[t] = (int32_t)first / units + c;
        }
        __syncthreads();
        for (int j = t; j < wt * nb; j += 1024) {
          const int uj = by_row_group ? div_by(j, H, h_sh) : j;
          const int k = j - uj * wt;
          const int pos = pos_s[uj];
          if (pos >= 0 && pos + k < a.group_cap) a.group_order[pos + k] = grp_s[uj] + k * seq_len[uj];
        }
        if (t < kKeys) {
          int sum = 0;
#pragma unroll
          for (int w = 0; w < 1024 / kWave; ++w) sum += key_wave[w][t];
#pragma unroll
          for (int w = 0; w < 1024 / kWave; ++w) key_wave[w][t] = 0;
          key_next[t] += sum * wt;
        }
        __syncthreads();
      }
    }
    __syncthreads();
    if (t == 0) {
      carry_items += (int64_t)wt * tot_items;
      carry_mrg += wt * tot_mrg;
    }
    __syncthreads();
  }
  if (t == 0) {
    // (the host sizes the map for the most items any plan makes)
    a.plan_info[0] = carry_items < a.map_cap ? carry_items : a.map_cap;
    a.plan_info[1] = tpi;
    // (groups of the prompt-chunk kernel: whole workgroups of items)
    const int64_t groups = carry_items / units;
    a.plan_info[10] = groups < a.group_cap ? groups : a.group_cap;
    a.plan_info[11] = by_chunk ? 1 : 0;
    a.plan_info[12] = carry_mrg;
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch over the compiled instances.
// ---------------------------------------------------------------------------
// Items planned per compute unit and round.  Fewer concurrent waves than the
// kernel's occupancy allows read HBM more efficiently (fewer streams fighting
// over DRAM rows), as long as enough bytes stay in flight.  PKV_SLOTS_PER_CU
// overrides the per-type default (tuning); 0 when unset.
static int slots_per_cu_override() {
  static const int v = [] {
    const char* e = getenv("PKV_SLOTS_PER_CU");
    const int x = e ? atoi(e) : 0;
    return x > 0 ? x : 0;
  }();
  return v;
}

// Extra arguments of a multi-query call; bound_only: compute the items bound
// of the instance into *bound_only and launch nothing.
struct MultiLaunch {
  int batch_real;
  int32_t* vctx;
  int64_t* bound_only = nullptr;
};

template <int KV, int QT, int D, int BS, bool MULTI, bool DEEP>
static hipError_t launch5(DecodeArgs& a, int num_cus, const MultiLaunch& ml, hipStream_t st) {
  using T = Tuning<KV, DEEP>;
  auto* kern = decode_partition_kernel<KV, QT, D, BS, MULTI, DEEP>;
  a.item_cap = T::item_tiles;   // the plan's item limit is this instance's
  // Resident waves per CU of this instance: a property of the compiled code,
  // queried once (every device the library runs on is gfx950).
  static std::atomic<int> occupancy{0};
  int per_cu = occupancy.load(std::memory_order_relaxed);
  hipError_t e = hipSuccess;
  if (per_cu == 0) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                      64, 0);
    if (e != hipSuccess) return e;
    occupancy.store(per_cu, std::memory_order_relaxed);
  }
  per_cu = per_cu < 1 ? 1 : (per_cu > kWavesPerCuCap ? kWavesPerCuCap : per_cu);
  const int target = slots_per_cu_override() > 0 ? slots_per_cu_override() : T::slots_per_cu;
  if (target < per_cu) per_cu = target;
  const int wpg = multi_wpg(a, MULTI);
  if (MULTI && per_cu > wpg) per_cu = per_cu / wpg * wpg;   // whole workgroups
  a.slots = num_cus * per_cu;
  if (a.slots > kMaxSlots) a.slots = kMaxSlots;
  const int64_t units = (int64_t)a.plan_heads * a.head_tiles;
  if (ml.bound_only) {   // this instance's own limit and slots
    *ml.bound_only = max_items_bound(a.batch, units, a.ctx_cap, a.slots, a.item_cap);
    return hipSuccess;
  }
  // The workspace was sized for kMaxSlots; fewer slots never need more items.
  // Every item has at least kItemTilesMin tiles, so a unit makes at most
  // ceil(tiles / kItemTilesMin) items: small batches launch few workgroups.
  int64_t need = max_items_bound(a.batch, units, a.ctx_cap, a.slots);
  // (an empty decode sequence still makes one item per unit, its zeros)
  const int64_t unit_tiles = ((int64_t)a.ctx_cap + kTileTokens - 1) / kTileTokens;
  int64_t unit_items = (unit_tiles + kItemTilesMin - 1) / kItemTilesMin;
  unit_items = unit_items < 1 ? 1 : unit_items;
  const int64_t short_bound = (int64_t)a.batch * units * unit_items;
  if (short_bound < need) need = short_bound > 0 ? short_bound : 1;
  const int64_t grid = ((need + wpg - 1) / wpg + 7) / 8 * 8;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if constexpr (MULTI) {
    hipLaunchKernelGGL(multi_prep_kernel, dim3(1), dim3(1024), 0, st, a, ml.batch_real, ml.vctx);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * wpg), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (MULTI) {
    const int rows = a.wave_rows * a.head_tiles;   // rows of a virtual sequence: one per wave
    hipLaunchKernelGGL((multi_merge_kernel<QT, D>), dim3(a.batch, (rows + kMergeWaves - 1) / kMergeWaves),
                       dim3(64 * kMergeWaves), 0, st, a);
  }
  else if (a.ws_seq)   // (no workspace: no unit can be split, every item finished in place)
    hipLaunchKernelGGL((decode_merge_kernel<QT, D>), dim3(a.num_q_heads, a.batch), dim3(64), 0,
                       st, a);
  return hipGetLastError();
}

// INT4 decode takes the DEEP instance when the batch has at most
// PKV_I4_DEEP_UNITS (sequence, KV head, head tile) units: its 8 items per CU
// then still split the units (measured on the 70B GQA-8 layer, 256 units:
// 112.7 against 119.6 us; on 13B MHA-40, 1,280 units, the 16-items-per-CU
// instance stays ahead, 69.1 against 76.2 us).  The choice depends only on
// the call's sizes, so the workspace bound and the launch agree.
template <int KV, int QT, int D, int BS, bool MULTI>
static hipError_t launch4(DecodeArgs& a, int num_cus, const MultiLaunch& ml, hipStream_t st) {
  if constexpr (KV == PKV_I4 && !MULTI) {
    const int64_t units = (int64_t)a.batch * a.plan_heads * a.head_tiles;
    if (units <= PKV_I4_DEEP_UNITS) return launch5<KV, QT, D, BS, MULTI, true>(a, num_cus, ml, st);
  }
  return launch5<KV, QT, D, BS, MULTI, false>(a, num_cus, ml, st);
}

template <int KV, int QT, int D, bool MULTI>
static hipError_t launch3(DecodeArgs& a, int bs, int cus, const MultiLaunch& ml, hipStream_t st) {
  return bs == 16 ? launch4<KV, QT, D, 16, MULTI>(a, cus, ml, st)
                  : launch4<KV, QT, D, 256, MULTI>(a, cus, ml, st);
}

template <int KV, int QT, bool MULTI>
static hipError_t launch2(DecodeArgs& a, int d, int bs, int cus, const MultiLaunch& ml,
                          hipStream_t st) {
  return d == 64 ? launch3<KV, QT, 64, MULTI>(a, bs, cus, ml, st)
                 : launch3<KV, QT, 128, MULTI>(a, bs, cus, ml, st);
}

template <int QT, bool MULTI>
static hipError_t launch1(DecodeArgs& a, int kv, int d, int bs, int cus, const MultiLaunch& ml,
                          hipStream_t st) {
  switch (kv) {
    case PKV_I8: return launch2<PKV_I8, QT, MULTI>(a, d, bs, cus, ml, st);
    case PKV_FP8_E4M3FN: return launch2<PKV_FP8_E4M3FN, QT, MULTI>(a, d, bs, cus, ml, st);
    case PKV_I4:
      if (d != 128) return hipErrorInvalidValue;   // (rejected by the entry points)
      return launch3<PKV_I4, QT, 128, MULTI>(a, bs, cus, ml, st);
    default: return launch2<QT, QT, MULTI>(a, d, bs, cus, ml, st);
  }
}

template <bool MULTI>
static hipError_t launch0(DecodeArgs& a, int q_dtype, int kv_dtype, int head_dim, int block_size,
                          int num_cus, const MultiLaunch& ml, hipStream_t st) {
  switch (q_dtype) {
    case PKV_F32: return launch1<PKV_F32, MULTI>(a, kv_dtype, head_dim, block_size, num_cus, ml, st);
    case PKV_F16: return launch1<PKV_F16, MULTI>(a, kv_dtype, head_dim, block_size, num_cus, ml, st);
    default: return launch1<PKV_BF16, MULTI>(a, kv_dtype, head_dim, block_size, num_cus, ml, st);
  }
}

hipError_t launch_decode(DecodeArgs& a, int q_dtype, int kv_dtype, int head_dim, int block_size,
                         int num_cus, hipStream_t st) {
  return launch0<false>(a, q_dtype, kv_dtype, head_dim, block_size, num_cus, MultiLaunch{0, nullptr},
                        st);
}

hipError_t decode_items_needed(DecodeArgs& a, int q_dtype, int kv_dtype, int head_dim,
                               int block_size, int num_cus, int64_t* items) {
  return launch0<false>(a, q_dtype, kv_dtype, head_dim, block_size, num_cus,
                        MultiLaunch{0, nullptr, items}, nullptr);
}

template <int QT, int D>
static hipError_t launch_prefill_call(DecodeArgs& a, int batch_real, int32_t* vctx, int kv_dtype,
                                      int block_size, int num_cus, hipStream_t st) {
  a.item_cap = kPrefillItemTilesMax;
  hipError_t e = launch_prefill(a, QT, kv_dtype, D, block_size, num_cus, true, st);   // a.slots
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(multi_prep_kernel, dim3(1), dim3(1024), 0, st, a, batch_real, vctx);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_prefill(a, QT, kv_dtype, D, block_size, num_cus, false, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_merge_kernel<QT, D>), dim3(a.batch < kMergeGroups ? a.batch : kMergeGroups),
                     dim3(64 * kMergeWaves), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_multi(DecodeArgs& a, int batch_real, int32_t* vctx, int q_dtype, int kv_dtype,
                        int head_dim, int block_size, int num_cus, bool prefill, hipStream_t st) {
  if (prefill) {
    // (the cache types the prompt-chunk kernel takes are checked by launch_prefill)
    if ((q_dtype != PKV_F16 && q_dtype != PKV_BF16) || (head_dim != 64 && head_dim != 128))
      return hipErrorInvalidValue;
    if (q_dtype == PKV_F16)
      return head_dim == 64
                 ? launch_prefill_call<PKV_F16, 64>(a, batch_real, vctx, kv_dtype, block_size, num_cus, st)
                 : launch_prefill_call<PKV_F16, 128>(a, batch_real, vctx, kv_dtype, block_size, num_cus, st);
    return head_dim == 64
               ? launch_prefill_call<PKV_BF16, 64>(a, batch_real, vctx, kv_dtype, block_size, num_cus, st)
               : launch_prefill_call<PKV_BF16, 128>(a, batch_real, vctx, kv_dtype, block_size, num_cus, st);
  }
  if (a.wave_rows != 16 * kMultiRowTiles) return hipErrorInvalidValue;
  return launch0<true>(a, q_dtype, kv_dtype, head_dim, block_size, num_cus,
                       MultiLaunch{batch_real, vctx}, st);
}

}  // namespace pkv
