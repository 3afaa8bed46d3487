/*
 * pagedkv.h — decode-time attention over a paged KV cache, for AMD Instinct
 * MI355X (gfx950).  Plain C ABI: device pointers, sizes, and a HIP stream
 * passed as void*.
 *
 * Pages cited:
 *  [P1] «LLM推理显存优化：KV Cache管理3大策略实测，节省60%显存开销»
 *  [P2] «生产级 LLM 推理的 KV 缓存优化» (The Ultimate Guide to KV Cache
 *       Optimization for LLM Inference)
 *  [P3] «大模型推理加速实战：KV Cache内存优化与PagedAttention分页管理方案»
 *
 * Cache layout (all entry points):
 *   k_cache, v_cache   [num_blocks][num_kv_heads][block_size][head_dim] elements in
 *                      kv_dtype, each group of 16 consecutive rows (tokens) of a
 *                      (block, head) tile stored in the order the decode kernel's
 *                      matrix instructions consume (eb = element bytes, rows of
 *                      head_dim elements, t = token within the group):
 *                        K: the row of token t is cut into 16-byte chunks; chunk c
 *                           is stored at byte (c * 16 + t) * 16 of the group;
 *                        V: element (t, d) is stored at byte
 *                           ((n / G) * 64 + (t / 4) * 16 + d % 16) * 16
 *                             + ((n % G) * 4 + t % 4) * eb,  n = d / 16, G = 4 / eb.
 *                      kv_cache_append writes this order; no caller needs to.
 *   INT4 caches        [num_blocks][num_kv_heads][block_size][head_dim / 2] bytes, head_dim
 *                      128; a row packs element 2k in the low nibble of byte k and 2k+1
 *                      in the high nibble (two's complement).  K groups: the packed row
 *                      is chunked as above (eb = 1 on the packed bytes).  V groups move
 *                      nibbles: element (t, d), n = d / 16, sits in byte
 *                        ((t / 4) * 16 + d % 16) * 16 + ((n % 8) / 2) * 4 + t % 4
 *                      of the group, low nibble for even n, high for odd (a byte holds
 *                      one token's elements d and d + 16).
 *   INT8 / INT4 scales float32 [num_blocks][num_kv_heads][block_size], one per stored row.
 *   FP8 scales         one float32 per tensor (per layer, one for K and one for V).
 *   block_tables       int32 [batch][max_blocks_per_seq]: logical block j of sequence b
 *                      lives in physical block block_tables[b][j] ([P1] §2 block table;
 *                      [P3] PagedAttention section, worked tables A = 0,3,7 / B = 1,2,5).
 *   context_lens       int32 [batch]: tokens of sequence b held in the cache.
 *   slot               physical_block * block_size + offset_in_block.
 *
 * Conventions shared by every call:
 *   - Pointers named as device pointers must point to device memory on the
 *     current HIP device; the caller owns them.  The library never allocates,
 *     frees or synchronises: every call only enqueues kernels on `stream`
 *     (a hipStream_t; NULL = the null stream) and returns.
 *   - Host-checkable problems (null pointers, unsupported sizes or dtype
 *     pairs, too small a workspace) return a non-zero pkv_status before any
 *     launch; pkv_last_error() then gives a text for the calling thread.
 *   - Contents of device arrays are preconditions, not checked (that would
 *     need a synchronisation).  For memory safety only, kernels skip — do not
 *     read through — a block-table entry outside [0, num_blocks), an INT8/FP8
 *     slot outside the pool, and clamp context_lens to
 *     [0, min(max_context_len, max_blocks_per_seq * block_size)]; the results
 *     for such inputs are unspecified but no access leaves the arrays.
 *   - Unused cache slots (free blocks, the tail of a sequence's last block)
 *     may hold any bytes, NaN included: they are never used in arithmetic.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent shapes   */
  PKV_ERR_UNSUPPORTED = 2, /* head_dim, block_size or dtype pair not built      */
  PKV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required         */
  PKV_ERR_HIP = 4          /* a kernel launch failed; the text names the call    */
} pkv_status;

/* Storage types.  FP8 is OCP E4M3FN (bias 7, 3 mantissa bits, max 448,
 * NaN = S.1111.111, no infinities): [P2] §4 and [P3] name an FP8 KV cache
 * without fixing the variant; E4M3FN is the one gfx950 converts natively. */
typedef enum {
  PKV_F32 = 0,
  PKV_F16 = 1,
  PKV_BF16 = 2,
  PKV_I8 = 3,
  PKV_FP8_E4M3FN = 4,
  PKV_I4 = 5               /* signed 4-bit codes, two per byte, per-row scale */
} pkv_dtype;

/* Text of the last non-OK status returned on this thread ("" if none). */
const char* pkv_last_error(void);

/*
 * kv_cache_bytes — closed-form size of a K+V cache:
 * 2 * batch * seq_len * layers * kv_heads * head_dim * dtype_bytes
 * ([P2] §2, estimating KV-cache memory; the same count as [P1] §1 and [P3]).
 * Host only.  Returns 0 if the product overflows 64 bits.
 */
uint64_t kv_cache_bytes(uint64_t batch, uint64_t seq_len, uint64_t layers,
                        uint64_t kv_heads, uint64_t head_dim, uint64_t dtype_bytes);

/*
 * kv_quantize — quantize rows of a float tensor for KV storage.
 *
 *   x         device, [n_rows][row_len] in x_dtype (PKV_F32 / PKV_F16 / PKV_BF16).
 *   out       device, [n_rows][row_len] bytes in out_dtype ([n_rows][row_len / 2]
 *             for PKV_I4).
 *   out_dtype PKV_I8: per-row quantizer of [P1] §4 (quantize_tensor):
 *               a = max|x_i| over the row; s = fl32(fl32(1/a) * 127) (the form
 *               PyTorch evaluates for the page's 127 / absmax);
 *               q_i = clamp(round_half_even(fl32(x_i * s)), -128, 127).
 *               scale: device float32 [n_rows], written with s (1.0 and all-zero
 *               codes for an all-zero row).  scale_given is ignored.
 *             PKV_FP8_E4M3FN: one scale for the whole tensor.  If scale_given is
 *               0, s = fl32(max|x| / 448) (1.0 if the tensor is all zero) is
 *               computed on the device and written to scale[0]; otherwise
 *               scale[0] is read.  Codes: RNE(clamp(fl32(x / s), -448, 448)).
 *             PKV_I4: the INT8 rule with 7 for 127 and [-8, 7] for the clamp
 *               (the INT4 cache of [P1] §4's quantization table, whose
 *               quantizer the page leaves open): s = fl32(fl32(1/a) * 7),
 *               q_i = clamp(round_half_even(fl32(x_i * s)), -8, 7); codes packed
 *               in row order, element 2k in the low nibble of byte k.  Scales as
 *               for PKV_I8.  row_len must be even.
 *   Errors: PKV_ERR_INVALID_ARG (null pointer, n_rows < 0, row_len < 1 or odd for I4),
 *           PKV_ERR_UNSUPPORTED (dtype pair), PKV_ERR_HIP.
 *   n_rows == 0 launches nothing (FP8 with scale_given == 0 still writes 1.0).
 */
pkv_status kv_quantize(const void* x, int32_t x_dtype, int64_t n_rows, int32_t row_len,
                       int32_t out_dtype, void* out, float* scale, int32_t scale_given,
                       void* stream);

/*
 * kv_cache_append — write the K/V rows of new tokens into their slots ([P3],
 * PagedAttention section: blocks are filled on demand through the table).
 *
 *   k, v          device, [num_tokens][num_kv_heads][head_dim] in src_dtype
 *                 (PKV_F32 / PKV_F16 / PKV_BF16), contiguous.
 *   slot_mapping  device int64 [num_tokens]; token i goes to block slot/block_size,
 *                 offset slot%block_size.  A negative slot writes nothing.
 *   k_cache, v_cache  device, cache layout above, in cache_dtype:
 *                 same as src_dtype: rows copied bit for bit;
 *                 PKV_I8: each (token, head) row quantized as kv_quantize does,
 *                   its scale written to k_scale/v_scale[block][head][offset];
 *                 PKV_FP8_E4M3FN: encoded with the tensor scale read from
 *                   k_scale[0] / v_scale[0] (saturating at +-448);
 *                 PKV_I4: quantized as kv_quantize does, scale as for PKV_I8
 *                   (head_dim 128 only).
 *   k_scale, v_scale  device float32 as above; NULL for plain float caches.
 *   Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED (head_dim not 64/128,
 *           block_size not 16/256, dtype pair, INT4 with head_dim 64), PKV_ERR_HIP.
 */
pkv_status kv_cache_append(const void* k, const void* v, int32_t src_dtype, int32_t num_tokens,
                           const int64_t* slot_mapping, void* k_cache, void* v_cache,
                           float* k_scale, float* v_scale, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                           int32_t cache_dtype, void* stream);

/*
 * paged_attention_workspace_size — bytes of device scratch paged_attention_decode
 * needs for these sizes (partial softmax state of contexts split over several
 * waves; sized for up to 256 compute units x 16 resident waves).  Host only, no
 * device needed.  0 when no context can be split (max_context_len <= 128) or
 * the sizes are invalid.
 */
size_t paged_attention_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t max_context_len);

/*
 * paged_attention_decode — one decode step: for every sequence b and query head
 * h, attention of q[b][h] over the first context_lens[b] tokens of the cache,
 * found through block_tables[b] ([P1] §2 and [P3]: the kernel locates each
 * block through the table; the result equals standard attention over the
 * stitched cache).  Query head h reads KV head h / (num_q_heads / num_kv_heads)
 * ([P1] §3, grouped-query attention: MHA, GQA and MQA are the same rule):
 *
 *   out[b][h] = sum_t softmax_t(scale * <q[b][h], K_t>) * V_t
 *
 *   out, q        device, [batch][num_q_heads][head_dim] in q_dtype
 *                 (PKV_F32 / PKV_F16 / PKV_BF16), contiguous, 16-byte aligned;
 *                 out may not alias q.
 *   k_cache, v_cache  device, cache layout above, kv_dtype = q_dtype, PKV_I8,
 *                 PKV_FP8_E4M3FN or PKV_I4.  Dequantized values: INT8 / INT4
 *                 code / scale (the inverse of [P1] §4's quantizer); FP8
 *                 decode(code) * scale.
 *   k_scale, v_scale  device: INT8 / INT4 [num_blocks][num_kv_heads][block_size];
 *                 FP8 one float each; NULL otherwise.
 *   block_tables  device int32 [batch][max_blocks_per_seq].
 *   context_lens  device int32 [batch]; a sequence of length 0 gets zeros.
 *   max_context_len  host int: an upper bound of context_lens (sizes the grid).
 *   scale         softmax scale (1/sqrt(head_dim) for the usual attention).
 *   workspace     device scratch of at least paged_attention_workspace_size(...)
 *                 bytes, 256-byte aligned (may be NULL when that
 *                 size is 0); contents are overwritten.  Calls that share a
 *                 workspace must be ordered.
 *   Supported: head_dim 64 or 128; block_size 16 or 256; num_q_heads a multiple
 *   of num_kv_heads.  INT4 caches: head_dim 128.  Pools
 *   may exceed 2^31 bytes (byte offsets are 64-bit).
 *   Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_HIP.
 */
pkv_status paged_attention_decode(void* out, const void* q, int32_t q_dtype, int32_t batch,
                                  int32_t num_q_heads, const void* k_cache, const void* v_cache,
                                  const float* k_scale, const float* v_scale, int32_t num_blocks,
                                  int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t kv_dtype, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t max_context_len, float scale, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode_noalloc — paged_attention_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, hosts that forbid allocation): the same arguments without a
 * workspace, the same kernels and the same result bit for bit.  The partial
 * rows of split contexts go to a static scratch array of
 * PKV_NOALLOC_SCRATCH_BYTES in the library, one per device, held from the first
 * call on that device until the process ends; nothing is allocated or freed.
 * The scratch needs no clearing (every byte read was written by the same call).
 * Calls on one device share the scratch: calls that may overlap there (other
 * streams, other threads) must be ordered by the caller, or they race.
 * Errors: as paged_attention_decode, and PKV_ERR_WORKSPACE when these sizes
 * need more scratch than PKV_NOALLOC_SCRATCH_BYTES (the message gives both).
 */
#define PKV_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
pkv_status paged_attention_decode_noalloc(void* out, const void* q, int32_t q_dtype,
                                          int32_t batch, int32_t num_q_heads, const void* k_cache,
                                          const void* v_cache, const float* k_scale,
                                          const float* v_scale, int32_t num_blocks,
                                          int32_t block_size, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t kv_dtype,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t max_context_len,
                                          float scale, void* stream);

/*
 * paged_attention_multi_workspace_size — bytes of device scratch
 * paged_attention_multi_query needs for these sizes (never 0 for valid sizes:
 * the call keeps its work plan there — virtual sequences, an item map — and,
 * when contexts are long enough to be cut, partial rows for the merge).  The
 * size depends on the sizes only, not on the dtypes: it covers either kernel
 * the call may take.  Host only.  0 for invalid sizes.
 */
size_t paged_attention_multi_workspace_size(int32_t batch, int32_t num_query_tokens,
                                            int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t max_context_len);

/*
 * paged_attention_multi_query — several new query tokens per sequence at once
 * (a chunk of a long prompt, or draft tokens to verify), attending through the
 * block tables ([P3], PagedAttention section: standard attention over the
 * stitched cache) with a causal mask.  The pages show only one-token decode;
 * the causal reading: the new tokens' K/V rows are appended first, so
 * context_lens[b] counts them, and query token j of the L_b new tokens of
 * sequence b sits at position p = context_lens[b] - L_b + j and attends to
 * positions 0 .. p.  Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 *   out, q        device, [num_query_tokens][num_q_heads][head_dim] in q_dtype,
 *                 sequences packed in order, 16-byte aligned; out may not alias q.
 *   query_start   device int32 [batch + 1]: sequence b's rows are
 *                 query_start[b] .. query_start[b + 1]; query_start[0] = 0,
 *                 nondecreasing, query_start[batch] = num_query_tokens
 *                 (preconditions; rows past num_query_tokens are never touched).
 *   k_cache ... max_context_len, scale  as for paged_attention_decode; a row with
 *                 p < 0 (more new tokens than cached ones) gets zeros.
 *   workspace     device scratch of paged_attention_multi_workspace_size(...) bytes,
 *                 256-byte aligned; contents overwritten; calls that share it
 *                 must be ordered.
 *   Supported: as paged_attention_decode, and num_query_tokens x (num_q_heads /
 *   num_kv_heads) < 2^31 - 4096.  Calls with several tokens per sequence and a
 *   mean of at least 128 (query token, head) rows per sequence, f16 or bf16
 *   queries and a cache of the query's type, FP8, INT8 or INT4 (prompt chunks)
 *   run on a kernel that shares each K/V step among 128 rows through LDS; all
 *   other calls (draft verification, f32 caches) on the decode kernel.
 *   L_b = 1 for every b gives exactly the decode result.
 *   Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_HIP.
 */
pkv_status paged_attention_multi_query(void* out, const void* q, int32_t q_dtype, int32_t batch,
                                       int32_t num_query_tokens, const int32_t* query_start,
                                       int32_t num_q_heads, const void* k_cache,
                                       const void* v_cache, const float* k_scale,
                                       const float* v_scale, int32_t num_blocks,
                                       int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t kv_dtype, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                                       int32_t max_context_len, float scale, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * kv_copy_blocks — copy whole physical blocks inside the pools (copy-on-write
 * of a shared block before an append, or compaction): for each pair i,
 * block pairs[2i + 1] of both caches (and, for INT8 / INT4, of both scale arrays)
 * becomes a byte-for-byte copy of block pairs[2i].
 *
 *   k_cache, v_cache, k_scale, v_scale  device, as for kv_cache_append (scales
 *                 are read only for PKV_I8 / PKV_I4; FP8's one tensor scale needs
 *                 no copy); head_dim counts elements (INT4 rows are head_dim / 2 bytes).
 *   pairs         device int32 [n_pairs][2] (src, dst).  Pairs with an index
 *                 outside [0, num_blocks) or src == dst are skipped.  The copies
 *                 of one call run concurrently: no dst may be another pair's src.
 *   Errors: PKV_ERR_INVALID_ARG (NULL pointers, misalignment, bad sizes),
 *           PKV_ERR_UNSUPPORTED (unknown dtype), PKV_ERR_HIP.
 */
pkv_status kv_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                          int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                          int32_t head_dim, int32_t kv_dtype, const int32_t* pairs,
                          int32_t n_pairs, void* stream);

/*
 * Block manager — host-side allocation of physical blocks to sequences
 * ([P1] §2: fixed-size blocks, a block table per sequence, reference counts
 * so blocks can be shared; [P3] PagedAttention section: blocks are taken on
 * demand and returned as soon as a sequence ends; [P2] §4 and [P3]: prefix
 * caching).  It only hands out block numbers; device memory is untouched.
 *
 * Rules:
 *   - A block referenced by more than one sequence is never written.  Appending
 *     into a shared, partly filled last block first gives the sequence a fresh
 *     block and reports (src, dst) so the caller can run kv_copy_blocks before
 *     writing the new rows (copy-on-write).
 *   - With prefix caching, each full block is keyed by a hash chained over all
 *     token ids from the sequence start through the block's end; a new
 *     sequence whose leading full blocks match cached blocks shares those blocks
 *     (their slots come back as -1: their rows are already stored, and
 *     kv_cache_append skips negative slots).  A key match is only a candidate:
 *     it is shared only if the cached block holds the same token ids and was
 *     sealed after the block just matched for the previous position (still
 *     holding that content), so equal keys of different prefixes are misses.
 *     Unreferenced cached blocks stay reusable until a fresh block is needed
 *     and no free block is left; then the least recently released is taken.
 *   - Failed calls change nothing.  Every call is host only and thread-safe.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* Text of the last failed block-manager call on this thread. */
const char* pkv_bm_last_error(void);

/* New manager over blocks 0 .. num_blocks-1 of block_size tokens; NULL on bad
 * sizes.  Blocks are handed out lowest number first while never used. */
pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size,
                                 int32_t enable_prefix_caching);
void pkv_bm_destroy(pkv_block_manager* bm);

/* Blocks a fresh allocation can still take (free plus unreferenced cached). */
int32_t pkv_bm_num_free(pkv_block_manager* bm);
/* References held on a block (-1 for a bad index). */
int32_t pkv_bm_ref_count(pkv_block_manager* bm, int32_t block);

/* Test hook, for tests of the content check only: keep just the bits of `mask`
 * of every lookup key, so that unrelated blocks collide (mask 0: every key is
 * the same).  Only before the manager's first sequence (PKV_ERR_INVALID_ARG
 * after).  Sharing stays exact; only the number of misses changes. */
pkv_status pkv_bm_debug_hash_mask(pkv_block_manager* bm, uint64_t mask);

/* Starts sequence seq_id with its n prompt tokens (host int32 ids; ids only
 * matter for prefix caching).  Writes the pool slot of every token to host
 * slots[n] (-1 for tokens in shared cached blocks).  PKV_ERR_INVALID_ARG if the
 * id is in use or the blocks run out. */
pkv_status pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                               int32_t n, int64_t* slots);

/* Appends n tokens to seq_id, writing their slots to host slots[n].  If the
 * last block was shared and partly filled it is replaced by a fresh block:
 * (src, dst) is written to host copies[0..1] and *n_copies = 1 (else 0); the
 * caller copies that block on the device before writing the new rows. */
pkv_status pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens, int32_t n,
                         int64_t* slots, int32_t* copies, int32_t max_copies, int32_t* n_copies);

/* child starts as a copy of parent sharing all its blocks (parallel samples,
 * beam search). */
pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);

/* Ends seq_id: every block loses one reference; blocks left unreferenced are
 * free again at once (cached ones become reusable). */
pkv_status pkv_bm_free(pkv_block_manager* bm, int64_t seq_id);

/* Host int32 tables[n_seqs][max_blocks] (-1 padded) and context_lens[n_seqs]
 * of the given sequences, ready for paged_attention_decode. */
pkv_status pkv_bm_block_tables(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n_seqs,
                               int32_t max_blocks, int32_t* tables, int32_t* context_lens);

/*
 * Swap space ([P3], vLLM configuration: swap_space moves inactive KV cache to
 * CPU memory, so more requests fit than HBM holds).
 *
 * pkv_bm_enable_swap gives the manager a host pool of num_host_blocks blocks
 * (numbered 0 ..; the caller allocates the host pools, pinned, with the device
 * pools' block layout).  Once per manager.
 *
 * pkv_bm_swap_out moves seq_id to the host pool: each of its n blocks gets a
 * host block, its device references are dropped (blocks left unreferenced are
 * free at once), and (device block, host block) pairs go to host
 * pairs[0 .. 2n) with *n_pairs = n.  The sequence cannot be appended to,
 * forked or listed in block tables until swapped in; pkv_bm_free still ends
 * it.  The caller copies the pairs with kv_swap_blocks before any later kernel
 * writes a device block handed out again (same stream, or an event).
 *
 * pkv_bm_swap_in brings it back into fresh device blocks: (host block, device
 * block) pairs as above; the host blocks are free again at once, so enqueue
 * these copies before any later swap-out's copies (one stream keeps the order).
 * Blocks swapped in are private to the sequence (not prefix-cache entries).
 *
 * Both fail without changing anything (PKV_ERR_INVALID_ARG) when the other
 * pool runs out, pairs is too small (max_pairs pairs), the sequence is
 * unknown or already in the requested place.
 */
pkv_status pkv_bm_enable_swap(pkv_block_manager* bm, int32_t num_host_blocks);
int32_t pkv_bm_num_free_host(pkv_block_manager* bm);
pkv_status pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq_id, int32_t* pairs,
                           int32_t max_pairs, int32_t* n_pairs);
pkv_status pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq_id, int32_t* pairs,
                          int32_t max_pairs, int32_t* n_pairs);

/*
 * kv_swap_blocks — copy whole blocks between two pools of the same layout,
 * device <-> pinned host (swap out / swap in) or device <-> device: for each
 * pair i, block pairs[2i + 1] of the destination pools becomes a byte-for-byte
 * copy of block pairs[2i] of the source pools (K, V and, for PKV_I8 / PKV_I4,
 * the row scales; FP8's tensor scale is shared by both pools).
 *
 *   src_*, dst_*  device memory or host memory from hipHostMalloc (pinned); the
 *                 pools are [num_blocks][num_kv_heads][block_size][head_dim] in
 *                 kv_dtype (INT4: head_dim / 2 bytes a row), scales
 *                 [num_blocks][num_kv_heads][block_size] float32.
 *   pairs         HOST int32 [n_pairs][2] (src block, dst block), each index
 *                 inside its pool (checked before anything is enqueued).
 *   stream        the copies are enqueued on it (typically a side stream, so they
 *                 overlap decode kernels).  Up to 32 runs of consecutive blocks
 *                 go as DMA transfers (no compute units taken); more, shorter
 *                 runs are moved by a copy kernel that reads and writes pinned
 *                 host memory directly (per-transfer overhead would dominate).
 *   Errors: PKV_ERR_INVALID_ARG (NULL pointers, bad sizes or pairs, pageable
 *           host memory), PKV_ERR_UNSUPPORTED (unknown dtype), PKV_ERR_HIP.
 */
pkv_status kv_swap_blocks(const void* src_k, const void* src_v, const float* src_k_scale,
                          const float* src_v_scale, int32_t src_num_blocks, void* dst_k,
                          void* dst_v, float* dst_k_scale, float* dst_v_scale,
                          int32_t dst_num_blocks, int32_t block_size, int32_t num_kv_heads,
                          int32_t head_dim, int32_t kv_dtype, const int32_t* pairs,
                          int32_t n_pairs, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
