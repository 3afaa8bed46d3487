// pkv_api.hip — the C ABI: argument checks, workspace sizing for the decode
// work plan, dispatch, and the per-thread error text.  Declarations and the meaning of every
// argument are in include/pagedkv.h.
#include <stdlib.h>

#include <map>
#include <mutex>
#include <string>

#include "pkv_common.h"
#include "pkv_internal.h"

namespace {

thread_local std::string g_last_error;

pkv_status fail(pkv_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

pkv_status ok() {
  g_last_error.clear();
  return PKV_OK;
}

pkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool is_float_dtype(int32_t d) { return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device (cached per device; host query only).
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  cache[dev] = cus;
  return cus;
}

// Workspace: per sequence (first item, items per unit), 16 B, padded to 256 B;
// then rows of one (max, sum) pair and one head_dim-long output per (item, head
// of its 16-head tile).
int64_t row_bytes(int64_t head_dim) { return 16 * (2 + head_dim) * 4; }
int64_t seq_bytes(int64_t batch) { return (batch * 16 + 255) / 256 * 256; }

// Items the plan can make for these sizes when it plans for the largest slot
// count (kMaxSlots; a device with fewer resident waves makes fewer items).
// 0 when every unit fits one item (contexts of at most kItemTilesMin tiles):
// no workspace is needed then.
int64_t workspace_items(int64_t batch, int64_t num_q_heads, int64_t num_kv_heads,
                        int64_t max_context_len) {
  if (max_context_len <= (int64_t)pkv::kItemTilesMin * pkv::kTileTokens) return 0;
  const int64_t units = num_kv_heads * ceil_div(num_q_heads / num_kv_heads, 16);
  return pkv::max_items_bound(batch, units, max_context_len, pkv::kMaxSlots);
}

// kv_swap_blocks: at most this many runs of consecutive blocks go as DMA
// transfers; more take the copy kernel.
constexpr int32_t kSwapDmaRuns = 32;

// Several query tokens per sequence.  The rows of a KV head, (query token,
// head of its group), are cut into virtual sequences, the planner's unit of
// work, each run as one workgroup whose waves read every K/V tile together.
// Two shapes: prompt chunks (a mean of at least one workgroup's rows per
// sequence, f16/bf16 queries over a cache of their type, FP8, INT8 or INT4) take the
// LDS-sharing kernel, kPrefillWaves waves of kPrefillRowTiles 16-row tiles;
// everything else takes the multi-token decode kernel, whose waves hold
// kMultiRowTiles tiles and whose group size follows the mean rows per
// sequence (so a few draft tokens do not leave waves idle).
struct MultiShape {
  int64_t row_tiles;   // 16-row tiles per wave
  int64_t waves;       // waves (row groups) per virtual sequence
  bool prefill;
};
#ifndef PKV_PREFILL_MIN_ROWS
#define PKV_PREFILL_MIN_ROWS (16 * PKV_PREFILL_ROW_TILES * PKV_PREFILL_WAVES)
#endif
MultiShape multi_shape(int64_t batch, int64_t num_query_tokens, int64_t group, bool prefill_ok) {
  const int64_t rows = num_query_tokens * group;
  // (PKV_PREFILL_MIN_ROWS, a tuning knob: mean rows per sequence from which the
  // prompt-chunk kernel is used; one workgroup's rows by default.  One token
  // per sequence always takes the decode-shaped kernel, whose result is then
  // exactly paged_attention_decode's.)
  if (prefill_ok && num_query_tokens > batch && rows >= batch * PKV_PREFILL_MIN_ROWS)
    return MultiShape{pkv::kPrefillRowTiles, pkv::kPrefillWaves, true};
  const int64_t tr = 16 * pkv::kMultiRowTiles;
  int64_t g = (rows + batch * tr - 1) / (batch * tr);
  g = g < 1 ? 1 : (g > pkv::kMultiGroupMax ? pkv::kMultiGroupMax : g);
  return MultiShape{pkv::kMultiRowTiles, g, false};
}
bool prefill_types(int32_t q_dtype, int32_t kv_dtype, int32_t head_dim) {
  return (q_dtype == PKV_F16 || q_dtype == PKV_BF16) &&
         (((kv_dtype == q_dtype || kv_dtype == PKV_FP8_E4M3FN || kv_dtype == PKV_I8) &&
           (head_dim == 64 || head_dim == 128)) ||
          (kv_dtype == PKV_I4 && head_dim == 128));
}
int64_t multi_vseqs(int64_t batch, int64_t num_query_tokens, int64_t group, int64_t kv_heads,
                    const MultiShape& sh) {
  const int64_t rows = 16 * sh.row_tiles * sh.waves;
  return kv_heads * ((num_query_tokens * group + rows - 1) / rows + batch);
}
int64_t multi_items(int64_t vseqs, int64_t units_per_vseq, int64_t max_context_len) {
  if (max_context_len <= (int64_t)pkv::kItemTilesMin * pkv::kTileTokens) return 0;
  return pkv::max_items_bound(vseqs, units_per_vseq, max_context_len, pkv::kMaxSlots);
}
// Entries of the item -> virtual sequence map: the most items any plan makes
// (every unit one item when no context needs cutting).
int64_t map_entries(int64_t vseqs, int64_t units_per_vseq, int64_t max_context_len) {
  return pkv::max_items_bound(vseqs, units_per_vseq, max_context_len, pkv::kMaxSlots);
}
// The plan of a call: 128 bytes of scalars (items, tiles per item, groups of
// the prompt-chunk kernel, virtual sequences to merge, ...), six int32 per
// virtual sequence (context, sequence, row group, KV head, first item, items
// per row tile), the item map, the order of the prompt-chunk kernel's groups
// (one per kPrefillWaves items) and the list of virtual sequences the merge
// kernel visits (one int32 per virtual sequence).
constexpr int64_t kPlanHead = 128;
int64_t group_entries(int64_t map_cap) {
  return (map_cap + pkv::kPrefillWaves - 1) / pkv::kPrefillWaves;
}
int64_t vseq_bytes(int64_t vseqs, int64_t map_cap) {
  return (kPlanHead + 7 * 4 * vseqs + 4 * map_cap + 4 * group_entries(map_cap) + 255) / 256 * 256;
}
// Partial rows of an item: 16 x row tiles, each (max, sum) and head_dim floats.
int64_t multi_workspace(int64_t vseqs, int64_t items, int64_t head_dim, int64_t row_tiles,
                        int64_t map_cap) {
  return vseq_bytes(vseqs, map_cap) +
         (items > 0 ? seq_bytes(vseqs) + items * row_tiles * row_bytes(head_dim) : 0);
}
int64_t multi_workspace_of(int64_t batch, int64_t num_query_tokens, int64_t group,
                           int64_t kv_heads, int64_t head_dim, int64_t max_context_len,
                           const MultiShape& sh) {
  const int64_t v = multi_vseqs(batch, num_query_tokens, group, kv_heads, sh);
  return multi_workspace(v, multi_items(v, sh.waves, max_context_len), head_dim, sh.row_tiles,
                         map_entries(v, sh.waves, max_context_len));
}

// Scratch of paged_attention_decode_noalloc (partial softmax rows of split
// contexts), for callers that cannot allocate.  Each device the library runs
// on holds its own copy for the life of the process; its address is taken once
// per device with hipGetSymbolAddress (host code never uses the symbol itself,
// which on the host side is not a device address).  Calls on one device share
// it: calls that overlap there race, like calls that share a workspace.
}  // namespace

static __device__ __align__(256) uint8_t scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

pkv_status scratch_of_device(const char* fn, void** out) {
  static std::mutex mu;
  static std::map<int, void*> ptrs;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  std::lock_guard<std::mutex> lock(mu);
  auto it = ptrs.find(dev);
  if (it != ptrs.end()) {
    *out = it->second;
    return PKV_OK;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));   // (device dev is current)
  if (e != hipSuccess || ptr == nullptr) {
    (void)hipGetLastError();
    return fail(PKV_ERR_HIP, std::string(fn) + ": cannot take the scratch's device address: " +
                                 hipGetErrorString(e));
  }
  ptrs[dev] = ptr;
  *out = ptr;
  return PKV_OK;
}

// Checks, workspace layout and launch of one decode step; static_scratch: the
// workspace is the library's static scratch (sized for the launched instance).
pkv_status decode_impl(const char* fn, void* out, const void* q, int32_t q_dtype, int32_t batch,
                       int32_t num_q_heads, const void* k_cache, const void* v_cache,
                                  const float* k_scale, const float* v_scale, int32_t num_blocks,
                                  int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t kv_dtype, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t max_context_len, float scale, void* workspace,
                                  size_t workspace_bytes, bool static_scratch, void* stream) {
  if (!is_float_dtype(q_dtype))
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": q_dtype must be F32, F16 or BF16");
  if (kv_dtype != q_dtype && kv_dtype != PKV_I8 && kv_dtype != PKV_FP8_E4M3FN &&
      kv_dtype != PKV_I4)
    return fail(PKV_ERR_UNSUPPORTED,
                std::string(fn) + ": kv_dtype must equal q_dtype, or be I8, FP8_E4M3FN or I4");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": head_dim must be 64 or 128");
  if (kv_dtype == PKV_I4 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": INT4 caches need head_dim 128");
  if (block_size != 16 && block_size != 256)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": block_size must be 16 or 256");
  if (batch < 0 || batch > 65535 || num_q_heads < 1 || num_kv_heads < 1 ||
      num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG,
                std::string(fn) + ": need 0 <= batch <= 65535 and num_q_heads a multiple of "
                "num_kv_heads");
  if (num_blocks < 1 || max_blocks_per_seq < 1 || max_context_len < 0)
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": bad pool or table sizes");
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_ERR_INVALID_ARG,
                std::string(fn) + ": max_context_len exceeds max_blocks_per_seq * block_size");
  if (!(scale == scale) || __builtin_isinf(scale))
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": scale must be finite");
  if (batch == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": NULL pointer");
  if ((pkv::row_scaled(kv_dtype) || kv_dtype == PKV_FP8_E4M3FN) && (!k_scale || !v_scale))
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": quantized cache needs k_scale and v_scale");
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) ||
      (pkv::row_scaled(kv_dtype) && (!aligned(k_scale, 16) || !aligned(v_scale, 16))))
    return fail(PKV_ERR_INVALID_ARG,
                std::string(fn) + ": misaligned pointer (q, out, caches and row scales need 16 B)");

  const int32_t G = num_q_heads / num_kv_heads;
  const int32_t head_tiles = (G + 15) / 16;
  int64_t items = workspace_items(batch, num_q_heads, num_kv_heads, max_context_len);
  if (items > 0x7FFFFFF0)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": batch x heads x context too large");
  pkv::DecodeArgs a{};
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_tiles = head_tiles;
  a.plan_heads = num_kv_heads;
  a.ctx_cap = max_context_len;
  if (static_scratch && items > 0) {
    // The library's own scratch: sized by the launched instance's own slots
    // and item limit (tighter than the dtype-blind workspace size).
    const int cus = device_cus();
    if (cus <= 0) return fail(PKV_ERR_HIP, std::string(fn) + ": cannot query the device");
    const hipError_t e = pkv::decode_items_needed(a, q_dtype, kv_dtype, head_dim, block_size, cus,
                                                  &items);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  const size_t need = items > 0 ? (size_t)(seq_bytes(batch) + items * row_bytes(head_dim)) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_ERR_WORKSPACE,
                std::string(fn) + (static_scratch ? ": these sizes need " : ": workspace needs ") +
                    std::to_string(need) + " bytes of scratch, " +
                    (static_scratch ? "more than the library's static scratch of "
                                    : "got ") +
                    std::to_string(workspace_bytes));
  if (need > 0 && !aligned(workspace, 256))
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": workspace must be 256-byte aligned");

  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_items = (int32_t)items;
  a.scale = scale;
  const int cus = device_cus();
  if (cus <= 0) return fail(PKV_ERR_HIP, std::string(fn) + ": cannot query the device");
  if (need > 0) {
    uint8_t* w = static_cast<uint8_t*>(workspace);
    a.ws_seq = reinterpret_cast<int64_t*>(w);
    a.ws_ml = reinterpret_cast<float*>(w + seq_bytes(batch));
    a.ws_acc = reinterpret_cast<float*>(w + seq_bytes(batch) + items * 16 * 2 * 4);
  }
  return hip_status(pkv::launch_decode(a, q_dtype, kv_dtype, head_dim, block_size, cus,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

uint64_t kv_cache_bytes(uint64_t batch, uint64_t seq_len, uint64_t layers, uint64_t kv_heads,
                        uint64_t head_dim, uint64_t dtype_bytes) {
  uint64_t r = 2;
  const uint64_t f[6] = {batch, seq_len, layers, kv_heads, head_dim, dtype_bytes};
  for (uint64_t x : f)
    if (__builtin_mul_overflow(r, x, &r)) return 0;
  return r;
}

size_t paged_attention_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t max_context_len) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      head_dim <= 0 || max_context_len <= 0)
    return 0;
  const int64_t items = workspace_items(batch, num_q_heads, num_kv_heads, max_context_len);
  return items > 0 ? (size_t)(seq_bytes(batch) + items * row_bytes(head_dim)) : 0;
}

pkv_status kv_quantize(const void* x, int32_t x_dtype, int64_t n_rows, int32_t row_len,
                       int32_t out_dtype, void* out, float* scale, int32_t scale_given,
                       void* stream) {
  if (!is_float_dtype(x_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "kv_quantize: x_dtype must be F32, F16 or BF16");
  if (out_dtype != PKV_I8 && out_dtype != PKV_FP8_E4M3FN && out_dtype != PKV_I4)
    return fail(PKV_ERR_UNSUPPORTED, "kv_quantize: out_dtype must be I8, FP8_E4M3FN or I4");
  if (n_rows < 0 || row_len < 1)
    return fail(PKV_ERR_INVALID_ARG, "kv_quantize: n_rows must be >= 0 and row_len >= 1");
  if (out_dtype == PKV_I4 && row_len % 2)
    return fail(PKV_ERR_INVALID_ARG, "kv_quantize: INT4 rows need an even row_len");
  if (!scale) return fail(PKV_ERR_INVALID_ARG, "kv_quantize: scale is NULL");
  if (n_rows > 0 && (!x || !out)) return fail(PKV_ERR_INVALID_ARG, "kv_quantize: x or out is NULL");
  if (!aligned(x, pkv::dtype_bytes(x_dtype)) || !aligned(scale, 4))
    return fail(PKV_ERR_INVALID_ARG, "kv_quantize: misaligned pointer");
  return hip_status(pkv::launch_quantize(x, x_dtype, n_rows, row_len, out_dtype, out, scale,
                                         scale_given, static_cast<hipStream_t>(stream)),
                    "kv_quantize");
}

pkv_status kv_cache_append(const void* k, const void* v, int32_t src_dtype, int32_t num_tokens,
                           const int64_t* slot_mapping, void* k_cache, void* v_cache,
                           float* k_scale, float* v_scale, int32_t num_blocks, int32_t block_size,
                           int32_t num_kv_heads, int32_t head_dim, int32_t cache_dtype,
                           void* stream) {
  if (!is_float_dtype(src_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "kv_cache_append: src_dtype must be F32, F16 or BF16");
  if (cache_dtype != src_dtype && cache_dtype != PKV_I8 && cache_dtype != PKV_FP8_E4M3FN &&
      cache_dtype != PKV_I4)
    return fail(PKV_ERR_UNSUPPORTED,
                "kv_cache_append: cache_dtype must equal src_dtype, or be I8, FP8_E4M3FN or I4");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "kv_cache_append: head_dim must be 64 or 128");
  if (cache_dtype == PKV_I4 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "kv_cache_append: INT4 caches need head_dim 128");
  if (block_size != 16 && block_size != 256)
    return fail(PKV_ERR_UNSUPPORTED, "kv_cache_append: block_size must be 16 or 256");
  if (num_tokens < 0 || num_blocks < 1 || num_kv_heads < 1 || num_kv_heads > 65535)
    return fail(PKV_ERR_INVALID_ARG, "kv_cache_append: bad sizes");
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(PKV_ERR_INVALID_ARG, "kv_cache_append: NULL pointer");
  if ((pkv::row_scaled(cache_dtype) || cache_dtype == PKV_FP8_E4M3FN) && (!k_scale || !v_scale))
    return fail(PKV_ERR_INVALID_ARG, "kv_cache_append: quantized cache needs k_scale and v_scale");
  const int eb = pkv::dtype_bytes(src_dtype);
  if (!aligned(k, eb) || !aligned(v, eb) || !aligned(k_cache, 4) || !aligned(v_cache, 4) ||
      !aligned(slot_mapping, 8))
    return fail(PKV_ERR_INVALID_ARG, "kv_cache_append: misaligned pointer");
  return hip_status(pkv::launch_append(k, v, src_dtype, num_tokens, slot_mapping, k_cache, v_cache,
                                       k_scale, v_scale, num_blocks, block_size, num_kv_heads,
                                       head_dim, cache_dtype, static_cast<hipStream_t>(stream)),
                    "kv_cache_append");
}

pkv_status kv_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                          int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                          int32_t head_dim, int32_t kv_dtype, const int32_t* pairs,
                          int32_t n_pairs, void* stream) {
  if (kv_dtype < PKV_F32 || kv_dtype > PKV_I4)
    return fail(PKV_ERR_UNSUPPORTED, "kv_copy_blocks: unknown kv_dtype");
  if (num_blocks < 1 || block_size < 1 || num_kv_heads < 1 || head_dim < 1 || n_pairs < 0)
    return fail(PKV_ERR_INVALID_ARG, "kv_copy_blocks: bad sizes");
  if (n_pairs == 0) return ok();
  if (n_pairs > 0x3FFFFFFF) return fail(PKV_ERR_INVALID_ARG, "kv_copy_blocks: too many pairs");
  if (!k_cache || !v_cache || !pairs) return fail(PKV_ERR_INVALID_ARG, "kv_copy_blocks: NULL pointer");
  if (pkv::row_scaled(kv_dtype) && (!k_scale || !v_scale))
    return fail(PKV_ERR_INVALID_ARG, "kv_copy_blocks: an INT8 / INT4 cache needs k_scale and v_scale");
  const int64_t block_rows = (int64_t)num_kv_heads * block_size;
  const int64_t block_bytes = block_rows * pkv::row_bytes_of(kv_dtype, head_dim);
  if (block_bytes % 16 || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(pairs, 4))
    return fail(PKV_ERR_INVALID_ARG,
                "kv_copy_blocks: caches need 16-byte alignment and 16-byte-multiple blocks");
  return hip_status(pkv::launch_copy_blocks(k_cache, v_cache,
                                            pkv::row_scaled(kv_dtype) ? k_scale : nullptr,
                                            pkv::row_scaled(kv_dtype) ? v_scale : nullptr, pairs,
                                            n_pairs, block_bytes, block_rows, num_blocks,
                                            static_cast<hipStream_t>(stream)),
                    "kv_copy_blocks");
}

pkv_status paged_attention_decode(void* out, const void* q, int32_t q_dtype, int32_t batch,
                                  int32_t num_q_heads, const void* k_cache, const void* v_cache,
                                  const float* k_scale, const float* v_scale, int32_t num_blocks,
                                  int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t kv_dtype, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t max_context_len, float scale, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return decode_impl("paged_attention_decode", out, q, q_dtype, batch, num_q_heads, k_cache,
                     v_cache, k_scale, v_scale, num_blocks, block_size, num_kv_heads, head_dim,
                     kv_dtype, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                     scale, workspace, workspace_bytes, false, stream);
}

pkv_status paged_attention_decode_noalloc(void* out, const void* q, int32_t q_dtype,
                                          int32_t batch, int32_t num_q_heads, const void* k_cache,
                                          const void* v_cache, const float* k_scale,
                                          const float* v_scale, int32_t num_blocks,
                                          int32_t block_size, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t kv_dtype,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t max_context_len,
                                          float scale, void* stream) {
  const char* fn = "paged_attention_decode_noalloc";
  void* ptr = nullptr;
  const pkv_status st = scratch_of_device(fn, &ptr);
  if (st != PKV_OK) return st;
  return decode_impl(fn, out, q, q_dtype, batch, num_q_heads, k_cache, v_cache, k_scale, v_scale,
                     num_blocks, block_size, num_kv_heads, head_dim, kv_dtype, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, scale, ptr,
                     PKV_NOALLOC_SCRATCH_BYTES, true, stream);
}

size_t paged_attention_multi_workspace_size(int32_t batch, int32_t num_query_tokens,
                                            int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t max_context_len) {
  if (batch <= 0 || num_query_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads || head_dim <= 0 || max_context_len < 0)
    return 0;
  const int64_t G = num_q_heads / num_kv_heads;
  // (no dtypes here: enough for either shape the call may take)
  const int64_t a = multi_workspace_of(batch, num_query_tokens, G, num_kv_heads, head_dim,
                                       max_context_len, multi_shape(batch, num_query_tokens, G, false));
  const int64_t b = multi_workspace_of(batch, num_query_tokens, G, num_kv_heads, head_dim,
                                       max_context_len, multi_shape(batch, num_query_tokens, G, true));
  return (size_t)(a > b ? a : b);
}

pkv_status paged_attention_multi_query(void* out, const void* q, int32_t q_dtype, int32_t batch,
                                       int32_t num_query_tokens, const int32_t* query_start,
                                       int32_t num_q_heads, const void* k_cache,
                                       const void* v_cache, const float* k_scale,
                                       const float* v_scale, int32_t num_blocks,
                                       int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t kv_dtype, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                                       int32_t max_context_len, float scale, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  const char* fn = "paged_attention_multi_query";
  if (!is_float_dtype(q_dtype)) return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": q_dtype must be F32, F16 or BF16");
  if (kv_dtype != q_dtype && kv_dtype != PKV_I8 && kv_dtype != PKV_FP8_E4M3FN && kv_dtype != PKV_I4)
    return fail(PKV_ERR_UNSUPPORTED,
                std::string(fn) + ": kv_dtype must equal q_dtype, or be I8, FP8_E4M3FN or I4");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": head_dim must be 64 or 128");
  if (kv_dtype == PKV_I4 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": INT4 caches need head_dim 128");
  if (block_size != 16 && block_size != 256)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": block_size must be 16 or 256");
  if (batch < 0 || num_query_tokens < 0 || num_q_heads < 1 || num_kv_heads < 1 ||
      num_q_heads % num_kv_heads != 0 || num_kv_heads > 65535)
    return fail(PKV_ERR_INVALID_ARG,
                std::string(fn) + ": need batch, num_query_tokens >= 0 and num_q_heads a multiple of "
                "num_kv_heads");
  if (num_blocks < 1 || max_blocks_per_seq < 1 || max_context_len < 0)
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": bad pool or table sizes");
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_ERR_INVALID_ARG,
                std::string(fn) + ": max_context_len exceeds max_blocks_per_seq * block_size");
  if (!(scale == scale) || __builtin_isinf(scale))
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": scale must be finite");
  if (batch == 0 || num_query_tokens == 0) return ok();
  if (!out || !q || !query_start || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": NULL pointer");
  if ((pkv::row_scaled(kv_dtype) || kv_dtype == PKV_FP8_E4M3FN) && (!k_scale || !v_scale))
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": quantized cache needs k_scale and v_scale");
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4) ||
      (pkv::row_scaled(kv_dtype) && (!aligned(k_scale, 16) || !aligned(v_scale, 16))))
    return fail(PKV_ERR_INVALID_ARG,
                std::string(fn) + ": misaligned pointer (q, out, caches and row scales need 16 B)");
  const int32_t G = num_q_heads / num_kv_heads;
  if ((int64_t)num_query_tokens * G > 0x7FFFF000)   // rows are counted in 32 bits on the device
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": num_query_tokens x group too large");
  const MultiShape sh =
      multi_shape(batch, num_query_tokens, G, prefill_types(q_dtype, kv_dtype, head_dim));
  const int64_t vseqs = multi_vseqs(batch, num_query_tokens, G, num_kv_heads, sh);
  const int32_t wg = (int32_t)sh.waves;
  const int64_t items = multi_items(vseqs, wg, max_context_len);
  if (vseqs > 0x7FFFFFF0 || items > 0x7FFFFFF0)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": query rows x heads x context too large");
  const int64_t map_cap = map_entries(vseqs, wg, max_context_len);
  const size_t need = (size_t)multi_workspace(vseqs, items, head_dim, sh.row_tiles, map_cap);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, std::string(fn) + ": workspace needs " + std::to_string(need) +
                                       " bytes, got " + std::to_string(workspace_bytes));
  if (!aligned(workspace, 256))
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": workspace must be 256-byte aligned");
  const int cus = device_cus();
  if (cus <= 0) return fail(PKV_ERR_HIP, std::string(fn) + ": cannot query the device");

  uint8_t* w = static_cast<uint8_t*>(workspace);
  int32_t* vctx = reinterpret_cast<int32_t*>(w + kPlanHead);
  pkv::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.context_lens = vctx;
  a.batch = (int32_t)vseqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_tiles = wg;   // row tiles (waves) per virtual sequence
  a.plan_heads = 1;    // a virtual sequence is one KV head
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.ctx_cap = max_context_len;
  a.max_items = (int32_t)items;
  a.scale = scale;
  a.vseq_b = vctx + vseqs;
  a.vseq_rt = vctx + 2 * vseqs;
  a.vseq_g = vctx + 3 * vseqs;
  a.vseq_first = vctx + 4 * vseqs;
  a.vseq_m = vctx + 5 * vseqs;
  a.item_vseq = vctx + 6 * vseqs;
  a.map_cap = map_cap;
  a.group_order = a.item_vseq + map_cap;
  a.group_cap = group_entries(map_cap);
  a.merge_list = a.group_order + a.group_cap;
  a.plan_info = reinterpret_cast<int64_t*>(w);
  a.query_start = query_start;
  a.real_ctx = context_lens;
  a.q_rows = num_query_tokens;
  a.wave_rows = (int32_t)(16 * sh.row_tiles);
  a.prefill = sh.prefill ? 1 : 0;
  if (items > 0) {
    uint8_t* rest = w + vseq_bytes(vseqs, map_cap);
    a.ws_seq = reinterpret_cast<int64_t*>(rest);
    a.ws_ml = reinterpret_cast<float*>(rest + seq_bytes(vseqs));
    a.ws_acc = reinterpret_cast<float*>(rest + seq_bytes(vseqs) +
                                        items * sh.row_tiles * 16 * 2 * 4);
  }
  return hip_status(pkv::launch_multi(a, batch, vctx, q_dtype, kv_dtype, head_dim, block_size, cus,
                                      sh.prefill, static_cast<hipStream_t>(stream)),
                    fn);
}

pkv_status kv_swap_blocks(const void* src_k, const void* src_v, const float* src_k_scale,
                          const float* src_v_scale, int32_t src_num_blocks, void* dst_k,
                          void* dst_v, float* dst_k_scale, float* dst_v_scale,
                          int32_t dst_num_blocks, int32_t block_size, int32_t num_kv_heads,
                          int32_t head_dim, int32_t kv_dtype, const int32_t* pairs,
                          int32_t n_pairs, void* stream) {
  const char* fn = "kv_swap_blocks";
  if (kv_dtype < PKV_F32 || kv_dtype > PKV_I4)
    return fail(PKV_ERR_UNSUPPORTED, std::string(fn) + ": unknown kv_dtype");
  if (src_num_blocks < 1 || dst_num_blocks < 1 || block_size < 1 || num_kv_heads < 1 ||
      head_dim < 1 || n_pairs < 0 || (kv_dtype == PKV_I4 && head_dim % 2))
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": bad sizes");
  if (n_pairs == 0) return ok();
  if (!src_k || !src_v || !dst_k || !dst_v || !pairs)
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": NULL pointer");
  const bool scaled = pkv::row_scaled(kv_dtype);
  if (scaled && (!src_k_scale || !src_v_scale || !dst_k_scale || !dst_v_scale))
    return fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": INT8 / INT4 pools need their row scales");
  for (int32_t i = 0; i < n_pairs; ++i)
    if (pairs[2 * i] < 0 || pairs[2 * i] >= src_num_blocks || pairs[2 * i + 1] < 0 ||
        pairs[2 * i + 1] >= dst_num_blocks)
      return fail(PKV_ERR_INVALID_ARG,
                  std::string(fn) + ": pair " + std::to_string(i) + " is outside its pool");
  // Every pool must be device memory or pinned host memory (a DMA engine
  // cannot read pageable memory asynchronously).
  const void* pools[8] = {src_k, src_v, dst_k, dst_v,
                          src_k_scale, src_v_scale, dst_k_scale, dst_v_scale};
  for (int i = 0; i < (scaled ? 8 : 4); ++i) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, pools[i]) != hipSuccess ||
        (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeHost)) {
      (void)hipGetLastError();   // the query's error is not the caller's
      return fail(PKV_ERR_INVALID_ARG,
                  std::string(fn) + ": pools must be device memory or pinned host memory");
    }
  }
  const int64_t block_rows = (int64_t)num_kv_heads * block_size;
  const int64_t block_bytes = block_rows * pkv::row_bytes_of(kv_dtype, head_dim);
  const int64_t scale_bytes = block_rows * 4;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // Runs of consecutive blocks go to the DMA engines as single transfers (no
  // compute units taken); when the pairs make many short runs, one transfer
  // each would cost more in per-transfer overhead than the bytes take, so a
  // gather/scatter kernel moves them instead (reading and writing pinned host
  // memory directly).
  int32_t runs = 0;
  for (int32_t i = 0; i < n_pairs; ++i)
    runs += i == 0 || pairs[2 * i] != pairs[2 * i - 2] + 1 || pairs[2 * i + 1] != pairs[2 * i - 1] + 1;
  if (runs > kSwapDmaRuns) {
    pkv::SwapArrays arr{{src_k, src_v, src_k_scale, src_v_scale},
                        {dst_k, dst_v, dst_k_scale, dst_v_scale}};
    return hip_status(pkv::launch_swap_blocks(arr, scaled ? 4 : 2, pairs, n_pairs, block_bytes,
                                              scale_bytes, st),
                      fn);
  }
  auto copy = [&](const void* s, void* d, int64_t per, int32_t sb, int32_t db, int32_t n) {
    return hipMemcpyAsync(static_cast<uint8_t*>(d) + (int64_t)db * per,
                          static_cast<const uint8_t*>(s) + (int64_t)sb * per, (size_t)(n * per),
                          hipMemcpyDefault, st);
  };
  for (int32_t i = 0; i < n_pairs;) {
    // a run of pairs whose source and destination blocks both step by one
    int32_t n = 1;
    while (i + n < n_pairs && pairs[2 * (i + n)] == pairs[2 * i] + n &&
           pairs[2 * (i + n) + 1] == pairs[2 * i + 1] + n)
      ++n;
    const int32_t sb = pairs[2 * i], db = pairs[2 * i + 1];
    hipError_t e = copy(src_k, dst_k, block_bytes, sb, db, n);
    if (e == hipSuccess) e = copy(src_v, dst_v, block_bytes, sb, db, n);
    if (e == hipSuccess && scaled) e = copy(src_k_scale, dst_k_scale, scale_bytes, sb, db, n);
    if (e == hipSuccess && scaled) e = copy(src_v_scale, dst_v_scale, scale_bytes, sb, db, n);
    if (e != hipSuccess) return hip_status(e, fn);
    i += n;
  }
  return ok();
}

}  // extern "C"
