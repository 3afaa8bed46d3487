// pkv_internal.h — argument blocks and launchers shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

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
  float* ws_ml;    // [batch][num_q_heads][max_parts][2]: running max (log2 domain), sum
  float* ws_acc;   // [batch][num_q_heads][max_parts][head_dim]: unnormalised output
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_tiles;          // ceil(G / 16): query heads of a group are taken 16 at a time
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t ctx_cap;             // context lengths are clamped to [0, ctx_cap]
  int32_t part_tokens;         // tokens per partition (multiple of block_size, <= 64 blocks)
  int32_t max_parts;           // ceil(max_context_len / part_tokens): workspace stride
  float scale;
};

hipError_t launch_decode(const DecodeArgs& a, int q_dtype, int kv_dtype, int head_dim,
                         int block_size, int grid_parts, hipStream_t st);

hipError_t launch_quantize(const void* x, int x_dtype, int64_t n_rows, int row_len, int out_dtype,
                           void* out, float* scale, int scale_given, hipStream_t st);

hipError_t launch_append(const void* k, const void* v, int src_dtype, int num_tokens,
                         const int64_t* slots, void* k_cache, void* v_cache, float* k_scale,
                         float* v_scale, int num_blocks, int block_size, int num_kv_heads,
                         int head_dim, int cache_dtype, hipStream_t st);

}  // namespace pkv
