// pkv_api.hip — the C ABI: argument checks, partition choice, workspace sizing,
// dispatch, and the per-thread error text.  Declarations and the meaning of every
// argument are in include/pagedkv.h.
#include <stdlib.h>

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

// Smallest partition the decode path uses; the workspace is sized for it.
constexpr int kMinPartition = 256;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tokens per decode workgroup.  512 keeps the per-partition state (<2% of the
// KV bytes it summarises) small while giving thousands of workgroups at the
// long-context shapes; short contexts with few (sequence, head) pairs drop to
// 256 to fill the 256 compute units.  PKV_PARTITION overrides it (tuning).
int choose_partition(int32_t batch, int32_t num_kv_heads, int32_t head_tiles, int32_t block_size,
                     int32_t max_context_len) {
  const char* env = getenv("PKV_PARTITION");
  if (env) {
    const int v = atoi(env);
    if (v >= kMinPartition && v <= 1024 && v % block_size == 0 && v / block_size <= 64) return v;
  }
  int p = 512;
  const int64_t units = (int64_t)batch * num_kv_heads * head_tiles * ceil_div(max_context_len, p);
  if (units < 2048) p = 256;
  if (p % block_size != 0) p = block_size;
  return p;
}

size_t workspace_bytes_for(int64_t batch, int64_t num_q_heads, int64_t head_dim, int64_t max_parts) {
  if (max_parts <= 1) return 0;
  const int64_t rows = batch * num_q_heads * max_parts;
  const int64_t ml = ((rows * 2 * 4) + 255) / 256 * 256;
  return (size_t)(ml + rows * head_dim * 4);
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

int32_t pkv_partition_tokens(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t block_size, int32_t max_context_len) {
  if (batch < 0 || num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads ||
      (block_size != 16 && block_size != 256) || max_context_len < 0)
    return 0;
  const int32_t tiles = (num_q_heads / num_kv_heads + 15) / 16;
  return choose_partition(batch, num_kv_heads, tiles, block_size, max_context_len);
}

size_t paged_attention_workspace_size(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                      int32_t max_context_len) {
  if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  return workspace_bytes_for(batch, num_q_heads, head_dim, ceil_div(max_context_len, kMinPartition));
}

pkv_status kv_quantize(const void* x, int32_t x_dtype, int64_t n_rows, int32_t row_len,
                       int32_t out_dtype, void* out, float* scale, int32_t scale_given,
                       void* stream) {
  if (!is_float_dtype(x_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "kv_quantize: x_dtype must be F32, F16 or BF16");
  if (out_dtype != PKV_I8 && out_dtype != PKV_FP8_E4M3FN)
    return fail(PKV_ERR_UNSUPPORTED, "kv_quantize: out_dtype must be I8 or FP8_E4M3FN");
  if (n_rows < 0 || row_len < 1)
    return fail(PKV_ERR_INVALID_ARG, "kv_quantize: n_rows must be >= 0 and row_len >= 1");
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
  if (cache_dtype != src_dtype && cache_dtype != PKV_I8 && cache_dtype != PKV_FP8_E4M3FN)
    return fail(PKV_ERR_UNSUPPORTED,
                "kv_cache_append: cache_dtype must equal src_dtype, or be I8 or FP8_E4M3FN");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "kv_cache_append: head_dim must be 64 or 128");
  if (block_size != 16 && block_size != 256)
    return fail(PKV_ERR_UNSUPPORTED, "kv_cache_append: block_size must be 16 or 256");
  if (num_tokens < 0 || num_blocks < 1 || num_kv_heads < 1 || num_kv_heads > 65535)
    return fail(PKV_ERR_INVALID_ARG, "kv_cache_append: bad sizes");
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(PKV_ERR_INVALID_ARG, "kv_cache_append: NULL pointer");
  if ((cache_dtype == PKV_I8 || cache_dtype == PKV_FP8_E4M3FN) && (!k_scale || !v_scale))
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

pkv_status paged_attention_decode(void* out, const void* q, int32_t q_dtype, int32_t batch,
                                  int32_t num_q_heads, const void* k_cache, const void* v_cache,
                                  const float* k_scale, const float* v_scale, int32_t num_blocks,
                                  int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t kv_dtype, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t max_context_len, float scale, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!is_float_dtype(q_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "paged_attention_decode: q_dtype must be F32, F16 or BF16");
  if (kv_dtype != q_dtype && kv_dtype != PKV_I8 && kv_dtype != PKV_FP8_E4M3FN)
    return fail(PKV_ERR_UNSUPPORTED,
                "paged_attention_decode: kv_dtype must equal q_dtype, or be I8 or FP8_E4M3FN");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attention_decode: head_dim must be 64 or 128");
  if (block_size != 16 && block_size != 256)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attention_decode: block_size must be 16 or 256");
  if (batch < 0 || batch > 65535 || num_q_heads < 1 || num_kv_heads < 1 ||
      num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG,
                "paged_attention_decode: need 0 <= batch <= 65535 and num_q_heads a multiple of "
                "num_kv_heads");
  if (num_blocks < 1 || max_blocks_per_seq < 1 || max_context_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "paged_attention_decode: bad pool or table sizes");
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_ERR_INVALID_ARG,
                "paged_attention_decode: max_context_len exceeds max_blocks_per_seq * block_size");
  if (!(scale == scale) || __builtin_isinf(scale))
    return fail(PKV_ERR_INVALID_ARG, "paged_attention_decode: scale must be finite");
  if (batch == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "paged_attention_decode: NULL pointer");
  if ((kv_dtype == PKV_I8 || kv_dtype == PKV_FP8_E4M3FN) && (!k_scale || !v_scale))
    return fail(PKV_ERR_INVALID_ARG, "paged_attention_decode: quantized cache needs k_scale and v_scale");
  if (!aligned(out, 16) || !aligned(q, 4) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) ||
      (kv_dtype == PKV_I8 && (!aligned(k_scale, 16) || !aligned(v_scale, 16))))
    return fail(PKV_ERR_INVALID_ARG,
                "paged_attention_decode: misaligned pointer (caches/out need 16 B, INT8 scales 16 B)");

  const int32_t G = num_q_heads / num_kv_heads;
  const int32_t head_tiles = (G + 15) / 16;
  if ((int64_t)num_kv_heads * head_tiles > 65535)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attention_decode: too many KV heads");
  const int part = choose_partition(batch, num_kv_heads, head_tiles, block_size, max_context_len);
  const int64_t max_parts = max_context_len > 0 ? ceil_div(max_context_len, part) : 1;
  const size_t need = workspace_bytes_for(batch, num_q_heads, head_dim, max_parts);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_ERR_WORKSPACE, "paged_attention_decode: workspace needs " +
                                       std::to_string(need) + " bytes, got " +
                                       std::to_string(workspace_bytes));
  if (need > 0 && !aligned(workspace, 256))
    return fail(PKV_ERR_INVALID_ARG, "paged_attention_decode: workspace must be 256-byte aligned");

  pkv::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_tiles = head_tiles;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.ctx_cap = max_context_len;
  a.part_tokens = part;
  a.max_parts = (int32_t)max_parts;
  a.scale = scale;
  if (need > 0) {
    const int64_t rows = (int64_t)batch * num_q_heads * max_parts;
    const int64_t ml = ((rows * 2 * 4) + 255) / 256 * 256;
    a.ws_ml = static_cast<float*>(workspace);
    a.ws_acc = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + ml);
  }
  return hip_status(pkv::launch_decode(a, q_dtype, kv_dtype, head_dim, block_size, (int)max_parts,
                                       static_cast<hipStream_t>(stream)),
                    "paged_attention_decode");
}

}  // extern "C"
