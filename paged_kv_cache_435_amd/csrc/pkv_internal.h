// pkv_internal.h — argument blocks, the decode work plan, and launchers shared
// by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Decode work is cut into items: an item is a run of 16-token tiles of one
// (sequence, KV head, tile of <= 16 query heads) unit, processed by one wave.
// The kernels plan the cut themselves from context_lens (device-resident), so
// that the item count matches the number of waves the GPU runs at once: one
// round of near-equal items, no tail of stragglers.
constexpr int kTileTokens = 16;
// Fewest tiles per item (128 tokens).  Small batches are latency-bound: a wave
// walks its tiles one load after another, so shorter items finish sooner
// (one 512-token sequence: 21.2 us at 16 tiles, 16.9 at 8); large batches plan
// far longer items and do not see it.  Tuning knob.
#ifndef PKV_ITEM_TILES_MIN
#define PKV_ITEM_TILES_MIN 8
#endif
constexpr int kItemTilesMin = PKV_ITEM_TILES_MIN;
// Most tiles per item: a lane holds one block-table entry per 64 tiles (at 16-token
// blocks).  The decode kernels take up to kItemTilesMax (8 registers; INT4,
// measured slower with 8, keeps 4); the prompt-chunk kernel, short of
// registers, kPrefillItemTilesMax.
constexpr int kItemTilesMax = 512;          // 8192 tokens
constexpr int kPrefillItemTilesMax = 256;   // 4096 tokens
constexpr int kWavesPerCuCap = 16;   // at most 4 waves per SIMD are planned for
constexpr int kMaxCus = 256;         // MI355X; plans never use more slots than this many CUs give
constexpr int kMaxSlots = kMaxCus * kWavesPerCuCap;
// Multi-token calls: 16-row tiles of (query token, head) rows per wave, and
// at most this many waves (32-row tiles) per workgroup.
#ifndef PKV_MULTI_ROW_TILES
#define PKV_MULTI_ROW_TILES 2
#endif
#ifndef PKV_MULTI_GROUP_MAX
#define PKV_MULTI_GROUP_MAX 4
#endif
// One-token decode: waves per workgroup.  A workgroup takes consecutive items,
// which are the KV heads of one (sequence, chunk): its waves then read the
// same blocks' adjacent (block, head) tiles at about the same time, which
// HBM serves faster than the same bytes spread over unrelated blocks.
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 8
#endif
constexpr int kDecodeWaves = PKV_DECODE_WAVES;
constexpr int kMultiRowTiles = PKV_MULTI_ROW_TILES;
constexpr int kMultiGroupMax = PKV_MULTI_GROUP_MAX;
// Prompt chunks (many rows per sequence, 16-bit caches): waves per workgroup
// of the LDS-sharing kernel and 16-row tiles per wave.  It is used when the
// mean rows per sequence fill at least one workgroup.
#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 4
#endif
#ifndef PKV_PREFILL_ROW_TILES
#define PKV_PREFILL_ROW_TILES 2
#endif
constexpr int kPrefillWaves = PKV_PREFILL_WAVES;
constexpr int kPrefillRowTiles = PKV_PREFILL_ROW_TILES;

// Everything the decode kernels read, passed by value.
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int64_t* ws_seq;  // [batch][2]: first item and items per unit of each sequence
  float* ws_ml;     // [max_items][16][2]: running max (log2 domain), sum
  float* ws_acc;    // [max_items][16][head_dim]: unnormalised output
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_tiles;          // ceil(G / 16): query heads of a group are taken 16 at a time
                               // (multi: row tiles per virtual sequence)
  int32_t plan_heads;          // KV heads per planned sequence: num_kv_heads (multi: 1)
  int32_t item_cap;            // most tiles per item the launched kernel holds table entries for
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t ctx_cap;             // context lengths are clamped to [0, ctx_cap]
  int32_t slots;               // items planned per round (waves resident at once)
  int32_t max_items;           // capacity of the workspace, in items
  float scale;
  // Several query tokens per sequence (multi-query calls only; batch is then
  // the number of virtual sequences and context_lens their lengths).
  int32_t* vseq_b;             // real sequence of each virtual sequence
  int32_t* vseq_rt;            // its group of row tiles of (query token, head) rows
  int32_t* vseq_g;             // its KV head
  const int32_t* query_start;  // [real batch + 1]: first query row of each sequence
  const int32_t* real_ctx;     // context_lens of the real sequences
  int32_t q_rows;              // query rows (tokens) in q and out
  int32_t wave_rows;           // (query token, head) rows per wave: 16 x row tiles
  // The plan of a multi-query call, made by its prep kernel.
  int64_t* plan_info;          // [0] items, [1] tiles per item, [10] prompt-chunk groups,
                               // [11] by-chunk numbering
  int32_t* group_order;        // prompt-chunk groups, longest first (multi_prep_kernel)
  int64_t group_cap;           // entries of group_order
  int32_t* merge_list;         // virtual sequences the merge kernel visits (multi_prep_kernel):
                               // units cut into several items, or no context (rows of zeros)
  int32_t* vseq_first;         // first item of each virtual sequence
  int32_t* vseq_m;             // items (chunks of its context) per row tile
  int32_t* item_vseq;          // virtual sequence of each item
  int64_t map_cap;             // entries of item_vseq
  int32_t prefill;             // the call takes the prompt-chunk kernel
};

// Host-side bound on the items a plan can make (grid size and workspace rows).
// With N tiles in U units and S slots, the plan uses S' = max(S - U, S/2) and
// t >= N / (k S') tiles per item over k rounds with an item limit L, so it
// makes at most sum ceil(n_u / t) <= k S' + U items, with k S' < N / L + S'.
// Hence at most N / L + S + U; the smaller limit (the prompt-chunk kernel's)
// bounds the plans of every kernel.
inline int64_t max_items_bound(int64_t batch, int64_t units_per_seq, int64_t max_context_len,
                               int64_t slots, int64_t item_cap = kPrefillItemTilesMax) {
  const int64_t units = batch * units_per_seq;
  const int64_t tiles = units * ((max_context_len + kTileTokens - 1) / kTileTokens);
  return (tiles + item_cap - 1) / item_cap + slots + units;
}

hipError_t launch_decode(DecodeArgs& a, int q_dtype, int kv_dtype, int head_dim, int block_size,
                         int num_cus, hipStream_t st);

// The most items the decode instance for these types and sizes can plan on
// this device (its own slots and item limit; no launch): a tighter bound than
// the dtype-blind one the workspace size uses.
hipError_t decode_items_needed(DecodeArgs& a, int q_dtype, int kv_dtype, int head_dim,
                               int block_size, int num_cus, int64_t* items);

// Multi-query: a.batch = virtual sequences (upper bound), a.context_lens =
// vctx (written by the prep kernel first), batch_real real sequences.
// prefill: the LDS-sharing kernel (a.head_tiles = kPrefillWaves, a.wave_rows =
// 16 kPrefillRowTiles; 16-bit caches of the query's type, FP8, INT8 or INT4), else the
// multi-token decode kernel (a.wave_rows = 16 kMultiRowTiles).
hipError_t launch_multi(DecodeArgs& a, int batch_real, int32_t* vctx, int q_dtype, int kv_dtype,
                        int head_dim, int block_size, int num_cus, bool prefill, hipStream_t st);

// The prefill kernel alone (pkv_prefill.hip); launch_multi runs the plan
// before it and the merge after it.  slots_only: set a.slots (the resident
// waves the plan is made for) and launch nothing.
hipError_t launch_prefill(DecodeArgs& a, int q_dtype, int kv_dtype, int head_dim, int block_size,
                          int num_cus, bool slots_only, hipStream_t st);

hipError_t launch_quantize(const void* x, int x_dtype, int64_t n_rows, int row_len, int out_dtype,
                           void* out, float* scale, int scale_given, hipStream_t st);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* pairs, int32_t n_pairs, int64_t block_bytes,
                              int64_t block_rows, int32_t num_blocks, hipStream_t st);

// Swap copies: pools K, V, K scales, V scales (source and destination), and
// the pairs of one launch passed by value.
struct SwapArrays {
  const void* src[4];
  void* dst[4];
};
constexpr int kSwapChunk = 256;
struct SwapChunk {
  int32_t n;
  int32_t src[kSwapChunk];
  int32_t dst[kSwapChunk];
};
hipError_t launch_swap_blocks(const SwapArrays& arr, int arrays, const int32_t* pairs,
                              int32_t n_pairs, int64_t block_bytes, int64_t scale_bytes,
                              hipStream_t st);

hipError_t launch_append(const void* k, const void* v, int src_dtype, int num_tokens,
                         const int64_t* slots, void* k_cache, void* v_cache, float* k_scale,
                         float* v_scale, int num_blocks, int block_size, int num_kv_heads,
                         int head_dim, int cache_dtype, hipStream_t st);

}  // namespace pkv
