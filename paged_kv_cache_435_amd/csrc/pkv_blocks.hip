// pkv_blocks.hip — the block manager (host) and block copies (device).
//
// [P1] «LLM推理显存优化：KV Cache管理3大策略实测，节省60%显存开销» §2: the cache is cut
// into fixed-size blocks; a per-sequence block table maps logical to physical
// blocks; blocks carry a reference count so sequences can share them.  [P3]
// «大模型推理加速实战：KV Cache内存优化与PagedAttention分页管理方案», PagedAttention
// section: blocks are taken on demand as a sequence grows and returned the
// moment it ends; [P2] «生产级 LLM 推理的 KV 缓存优化» §4 and [P3] name prefix caching.
//
// The manager hands out physical block numbers; it never touches device memory.
// Sharing follows one rule: a block with more than one reference is never
// written.  Appending into a shared, partly filled last block first moves the
// sequence to a fresh copy (copy-on-write; the caller copies the block's bytes
// on the device with kv_copy_blocks).  Full blocks are immutable, so prefix
// caching shares them by content: a full block is looked up by a hash chained
// over every token from the start of the sequence through the block's end, and
// a hit is taken only once its content is proven equal: the block's own token
// ids match, and its predecessor when it was sealed is the block just matched
// for the previous position, unchanged since (same epoch).  By induction the
// whole prefix then matches, so a hash collision costs a miss, never a wrong
// block.  Cached blocks nobody references stay reusable until a fresh block is
// needed and the free list is empty; then the least recently released one is
// taken.
//
// Swap space ([P3], vLLM configuration: swap_space moves inactive KV cache to
// CPU memory so more requests fit than HBM holds): with a host pool enabled, a
// sequence can be swapped out (each of its blocks gets a host block, its device
// references are dropped) and swapped back in (fresh device blocks).  The
// manager returns the block pairs to copy; kv_swap_blocks moves the bytes.
#include <stdint.h>
#include <string.h>

#include <list>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "pkv_common.h"
#include "pkv_internal.h"

namespace {

constexpr uint64_t kNoHash = 0;

// 64-bit FNV-1a over the previous block's key and this block's token ids,
// keeping the bits of `mask` (all of them, except under the test hook
// pkv_bm_debug_hash_mask).  Only a lookup key: hits are checked by content.
uint64_t chain_hash(uint64_t prev, const int32_t* tokens, int n, uint64_t mask) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&h](uint64_t x) {
    for (int i = 0; i < 8; ++i) {
      h ^= (x >> (8 * i)) & 0xFFu;
      h *= 1099511628211ull;
    }
  };
  mix(prev);
  for (int i = 0; i < n; ++i) mix((uint32_t)tokens[i]);
  h &= mask;
  return h == kNoHash ? 1 : h;
}

struct Sequence {
  std::vector<int32_t> blocks;   // physical block of each logical block (host block when swapped)
  bool swapped = false;
  int64_t tokens = 0;            // tokens held
  uint64_t last_full_key = kNoHash;   // key of the last full block (chain)
  std::vector<int32_t> pending;  // token ids of the partly filled last block
};

}  // namespace

struct pkv_block_manager {
  int32_t num_blocks;
  int32_t block_size;
  bool prefix_caching;
  std::vector<int32_t> ref;                    // references per block
  std::vector<uint64_t> key;                   // content key of a cached full block (0: none)
  // Prefix caching: what a keyed block holds, to check a hit by content.
  std::vector<int32_t> key_tokens;             // [num_blocks][block_size] token ids
  std::vector<int32_t> key_parent;             // predecessor block when sealed (-1: first)
  std::vector<uint32_t> key_parent_epoch;      // that predecessor's epoch then
  std::vector<uint32_t> epoch;                 // bumped each time a block is handed out fresh
  uint64_t hash_mask = ~0ull;
  std::vector<int32_t> free_list;              // blocks with no references and no key
  std::list<int32_t> evictable;                // cached blocks with no references, oldest first
  std::vector<std::list<int32_t>::iterator> evict_pos;
  std::vector<bool> in_evictable;
  std::unordered_map<uint64_t, int32_t> cache;   // key -> block
  std::unordered_map<int64_t, Sequence> seqs;
  int32_t num_host_blocks = 0;                 // swap space (0: none)
  std::vector<int32_t> host_free;
  std::mutex mu;
};

namespace {

thread_local std::string g_bm_error;

pkv_status bm_fail(pkv_status s, const std::string& m) {
  g_bm_error = m;
  return s;
}

int32_t free_count(const pkv_block_manager* bm) {
  return (int32_t)(bm->free_list.size() + bm->evictable.size());
}

// A fresh block for writing: from the free list, else the oldest unreferenced
// cached block (its key is dropped).  -1 if none.
int32_t take_fresh(pkv_block_manager* bm) {
  if (!bm->free_list.empty()) {
    const int32_t b = bm->free_list.back();
    bm->free_list.pop_back();
    bm->ref[b] = 1;
    ++bm->epoch[b];
    return b;
  }
  if (bm->evictable.empty()) return -1;
  const int32_t b = bm->evictable.front();
  bm->evictable.pop_front();
  bm->in_evictable[b] = false;
  bm->cache.erase(bm->key[b]);
  bm->key[b] = kNoHash;
  bm->ref[b] = 1;
  ++bm->epoch[b];   // its content is about to change: blocks sealed after it stop matching
  return b;
}

// Is cached block x, found under the key of logical block j of a new
// sequence, that sequence's block?  Its token ids must equal `tokens` (the
// block's bs ids) and its predecessor when sealed must be `prev` (the block
// matched for j - 1, -1 for j = 0) in its current epoch.
bool same_content(const pkv_block_manager* bm, int32_t x, const int32_t* tokens, int32_t prev) {
  const int bs = bm->block_size;
  if (memcmp(&bm->key_tokens[(size_t)x * bs], tokens, sizeof(int32_t) * bs) != 0) return false;
  if (bm->key_parent[x] != prev) return false;
  return prev < 0 || bm->key_parent_epoch[x] == bm->epoch[prev];
}

void take_ref(pkv_block_manager* bm, int32_t b) {
  if (bm->ref[b] == 0 && bm->in_evictable[b]) {
    bm->evictable.erase(bm->evict_pos[b]);
    bm->in_evictable[b] = false;
  }
  ++bm->ref[b];
}

void drop_ref(pkv_block_manager* bm, int32_t b) {
  if (--bm->ref[b] > 0) return;
  if (bm->key[b] != kNoHash) {   // keep the cached content reusable
    bm->evictable.push_back(b);
    bm->evict_pos[b] = std::prev(bm->evictable.end());
    bm->in_evictable[b] = true;
  } else {
    bm->free_list.push_back(b);
  }
}

// The sequence's last block just filled: give it its content key and, with
// prefix caching, offer it for sharing (a block already holding that key wins).
void seal_block(pkv_block_manager* bm, Sequence& s) {
  const uint64_t k =
      chain_hash(s.last_full_key, s.pending.data(), (int)s.pending.size(), bm->hash_mask);
  s.last_full_key = k;
  if (bm->prefix_caching) {
    const int32_t b = s.blocks.back();
    if (bm->ref[b] == 1 && bm->key[b] == kNoHash && bm->cache.find(k) == bm->cache.end()) {
      bm->key[b] = k;
      bm->cache[k] = b;
      const size_t bs = (size_t)bm->block_size;
      memcpy(&bm->key_tokens[(size_t)b * bs], s.pending.data(), sizeof(int32_t) * bs);
      const int32_t prev = s.blocks.size() >= 2 ? s.blocks[s.blocks.size() - 2] : -1;
      bm->key_parent[b] = prev;
      bm->key_parent_epoch[b] = prev >= 0 ? bm->epoch[prev] : 0u;
    }
  }
  s.pending.clear();
}

int64_t slot_of(const pkv_block_manager* bm, const Sequence& s, int64_t pos) {
  return (int64_t)s.blocks[pos / bm->block_size] * bm->block_size + pos % bm->block_size;
}

}  // namespace

extern "C" {

const char* pkv_bm_last_error(void) { return g_bm_error.c_str(); }

pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size,
                                 int32_t enable_prefix_caching) {
  if (num_blocks < 1 || block_size < 1) {
    g_bm_error = "pkv_bm_create: num_blocks and block_size must be >= 1";
    return nullptr;
  }
  pkv_block_manager* bm = new (std::nothrow) pkv_block_manager();
  if (!bm) return nullptr;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->prefix_caching = enable_prefix_caching != 0;
  bm->ref.assign(num_blocks, 0);
  bm->key.assign(num_blocks, kNoHash);
  bm->epoch.assign(num_blocks, 0u);
  if (bm->prefix_caching) {
    bm->key_tokens.assign((size_t)num_blocks * block_size, 0);
    bm->key_parent.assign(num_blocks, -1);
    bm->key_parent_epoch.assign(num_blocks, 0u);
  }
  bm->evict_pos.resize(num_blocks);
  bm->in_evictable.assign(num_blocks, false);
  bm->free_list.reserve(num_blocks);
  for (int32_t b = num_blocks - 1; b >= 0; --b) bm->free_list.push_back(b);   // 0 first
  return bm;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int32_t pkv_bm_num_free(pkv_block_manager* bm) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lock(bm->mu);
  return free_count(bm);
}

int32_t pkv_bm_ref_count(pkv_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  std::lock_guard<std::mutex> lock(bm->mu);
  return bm->ref[block];
}

pkv_status pkv_bm_debug_hash_mask(pkv_block_manager* bm, uint64_t mask) {
  if (!bm) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_debug_hash_mask: NULL manager");
  std::lock_guard<std::mutex> lock(bm->mu);
  if (!bm->seqs.empty() || !bm->cache.empty())
    return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_debug_hash_mask: only before the first sequence");
  bm->hash_mask = mask;
  return PKV_OK;
}

pkv_status pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                               int32_t n, int64_t* slots) {
  if (!bm) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_add_sequence: NULL manager");
  if (n < 0 || (n > 0 && (!tokens || !slots)))
    return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_add_sequence: bad token arrays");
  std::lock_guard<std::mutex> lock(bm->mu);
  if (bm->seqs.count(seq_id)) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_add_sequence: id in use");
  const int bs = bm->block_size;
  const int64_t nblk = ((int64_t)n + bs - 1) / bs;
  // Plan first (no state change until it is known to fit).
  std::vector<int32_t> hits;   // cached blocks for the leading full blocks
  uint64_t k = kNoHash;
  if (bm->prefix_caching) {
    for (int64_t j = 0; j < n / bs; ++j) {
      const uint64_t kj = chain_hash(k, tokens + j * bs, bs, bm->hash_mask);
      auto it = bm->cache.find(kj);
      if (it == bm->cache.end()) break;
      // (a key match that is not this content is a collision: a miss)
      if (!same_content(bm, it->second, tokens + j * bs, hits.empty() ? -1 : hits.back())) break;
      hits.push_back(it->second);
      k = kj;
    }
  }
  int64_t need = nblk - (int64_t)hits.size();
  int64_t reusable_hits_evictable = 0;   // hits sitting in the evictable list stop being free
  for (int32_t b : hits) reusable_hits_evictable += (bm->ref[b] == 0);
  if (need > (int64_t)free_count(bm) - reusable_hits_evictable)
    return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_add_sequence: out of blocks");

  Sequence s;
  for (int32_t b : hits) {
    take_ref(bm, b);
    s.blocks.push_back(b);
  }
  s.last_full_key = k;
  const int64_t shared_tokens = (int64_t)hits.size() * bs;
  for (int64_t i = 0; i < n; ++i) slots[i] = -1;   // rows of shared blocks are already stored
  s.tokens = shared_tokens;
  for (int64_t i = shared_tokens; i < n; ++i) {
    if (s.tokens % bs == 0) s.blocks.push_back(take_fresh(bm));
    slots[i] = slot_of(bm, s, s.tokens);
    s.pending.push_back(tokens[i]);
    ++s.tokens;
    if (s.tokens % bs == 0) seal_block(bm, s);
  }
  bm->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

pkv_status pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens, int32_t n,
                         int64_t* slots, int32_t* copies, int32_t max_copies,
                         int32_t* n_copies) {
  if (!bm || !n_copies) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_append: NULL argument");
  *n_copies = 0;
  if (n < 0 || (n > 0 && (!tokens || !slots)))
    return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_append: bad token arrays");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_append: unknown sequence");
  Sequence& s = it->second;
  if (s.swapped) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_append: sequence is swapped out");
  const int bs = bm->block_size;
  const bool cow = s.tokens % bs != 0 && bm->ref[s.blocks.back()] > 1;
  const int64_t room = s.tokens % bs == 0 ? 0 : bs - s.tokens % bs;
  const int64_t need = (n > room ? (n - room + bs - 1) / bs : 0) + (cow && n > 0 ? 1 : 0);
  if (need > free_count(bm)) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_append: out of blocks");
  if (cow && n > 0) {
    if (!copies || max_copies < 1)
      return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_append: copy-on-write needs room in copies");
    const int32_t src = s.blocks.back();
    const int32_t dst = take_fresh(bm);
    drop_ref(bm, src);
    s.blocks.back() = dst;
    copies[0] = src;
    copies[1] = dst;
    *n_copies = 1;
  }
  for (int64_t i = 0; i < n; ++i) {
    if (s.tokens % bs == 0) s.blocks.push_back(take_fresh(bm));
    slots[i] = slot_of(bm, s, s.tokens);
    s.pending.push_back(tokens[i]);
    ++s.tokens;
    if (s.tokens % bs == 0) seal_block(bm, s);
  }
  return PKV_OK;
}

pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_fork: NULL manager");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_fork: unknown parent");
  if (bm->seqs.count(child)) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_fork: child id in use");
  if (it->second.swapped) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_fork: parent is swapped out");
  Sequence c = it->second;   // same blocks, same tokens
  for (int32_t b : c.blocks) take_ref(bm, b);
  bm->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

pkv_status pkv_bm_free(pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_free: NULL manager");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_free: unknown sequence");
  // Release from the last block back, so the oldest-released cached blocks are
  // the deepest ones of a prefix (evicted first).
  if (it->second.swapped) {
    for (int32_t h : it->second.blocks) bm->host_free.push_back(h);
  } else {
    for (auto b = it->second.blocks.rbegin(); b != it->second.blocks.rend(); ++b) drop_ref(bm, *b);
  }
  bm->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_bm_block_tables(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n_seqs,
                               int32_t max_blocks, int32_t* tables, int32_t* context_lens) {
  if (!bm || n_seqs < 0 || max_blocks < 1 || (n_seqs > 0 && (!seq_ids || !tables || !context_lens)))
    return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_block_tables: bad arguments");
  std::lock_guard<std::mutex> lock(bm->mu);
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end())
      return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_block_tables: unknown sequence");
    if (it->second.swapped)
      return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_block_tables: sequence is swapped out");
    if ((int64_t)it->second.blocks.size() > max_blocks)
      return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_block_tables: max_blocks too small");
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    const Sequence& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = tables + (int64_t)i * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j)
      row[j] = j < (int32_t)s.blocks.size() ? s.blocks[j] : -1;
    context_lens[i] = (int32_t)s.tokens;
  }
  return PKV_OK;
}

pkv_status pkv_bm_enable_swap(pkv_block_manager* bm, int32_t num_host_blocks) {
  if (!bm || num_host_blocks < 1)
    return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_enable_swap: need a manager and >= 1 host block");
  std::lock_guard<std::mutex> lock(bm->mu);
  if (bm->num_host_blocks > 0)
    return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_enable_swap: swap space already set");
  bm->num_host_blocks = num_host_blocks;
  bm->host_free.reserve(num_host_blocks);
  for (int32_t h = num_host_blocks - 1; h >= 0; --h) bm->host_free.push_back(h);   // 0 first
  return PKV_OK;
}

int32_t pkv_bm_num_free_host(pkv_block_manager* bm) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lock(bm->mu);
  return (int32_t)bm->host_free.size();
}

pkv_status pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq_id, int32_t* pairs,
                           int32_t max_pairs, int32_t* n_pairs) {
  if (!bm || !n_pairs) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_swap_out: NULL argument");
  *n_pairs = 0;
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_swap_out: unknown sequence");
  Sequence& s = it->second;
  if (s.swapped) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_swap_out: already swapped out");
  const int32_t n = (int32_t)s.blocks.size();
  if (n > 0 && (!pairs || max_pairs < n))
    return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_swap_out: pairs holds fewer than the sequence's blocks");
  if (n > (int32_t)bm->host_free.size())
    return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_swap_out: out of host blocks");
  for (int32_t j = 0; j < n; ++j) {
    const int32_t h = bm->host_free.back();
    bm->host_free.pop_back();
    pairs[2 * j] = s.blocks[j];
    pairs[2 * j + 1] = h;
  }
  for (int32_t j = n - 1; j >= 0; --j) drop_ref(bm, s.blocks[j]);
  for (int32_t j = 0; j < n; ++j) s.blocks[j] = pairs[2 * j + 1];
  s.swapped = true;
  *n_pairs = n;
  return PKV_OK;
}

pkv_status pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq_id, int32_t* pairs,
                          int32_t max_pairs, int32_t* n_pairs) {
  if (!bm || !n_pairs) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_swap_in: NULL argument");
  *n_pairs = 0;
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_swap_in: unknown sequence");
  Sequence& s = it->second;
  if (!s.swapped) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_swap_in: not swapped out");
  const int32_t n = (int32_t)s.blocks.size();
  if (n > 0 && (!pairs || max_pairs < n))
    return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_swap_in: pairs holds fewer than the sequence's blocks");
  if (n > free_count(bm)) return bm_fail(PKV_ERR_INVALID_ARG, "pkv_bm_swap_in: out of blocks");
  for (int32_t j = 0; j < n; ++j) {
    const int32_t d = take_fresh(bm);
    pairs[2 * j] = s.blocks[j];
    pairs[2 * j + 1] = d;
    bm->host_free.push_back(s.blocks[j]);
    s.blocks[j] = d;
  }
  s.swapped = false;
  *n_pairs = n;
  return PKV_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Device: whole-block copies (copy-on-write, defragmentation).  One workgroup
// per (pair, K or V); 16 bytes per lane per step over the block's
// num_kv_heads * block_size rows.  INT8 row scales are copied alongside.
// ---------------------------------------------------------------------------
namespace pkv {

__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ k_cache,
                                                          uint8_t* __restrict__ v_cache,
                                                          float* __restrict__ k_scale,
                                                          float* __restrict__ v_scale,
                                                          const int32_t* __restrict__ pairs,
                                                          int64_t block_bytes, int64_t block_rows,
                                                          int32_t num_blocks) {
  const int pair = blockIdx.x >> 1;
  const int which = blockIdx.x & 1;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks || src == dst) return;
  uint8_t* base = which == 0 ? k_cache : v_cache;
  const u32x4* s = reinterpret_cast<const u32x4*>(base + (int64_t)src * block_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(base + (int64_t)dst * block_bytes);
  for (int64_t i = threadIdx.x; i < block_bytes / 16; i += blockDim.x) d[i] = s[i];
  float* sc = which == 0 ? k_scale : v_scale;
  if (sc)
    for (int64_t i = threadIdx.x; i < block_rows; i += blockDim.x)
      sc[(int64_t)dst * block_rows + i] = sc[(int64_t)src * block_rows + i];
}

// Swap copies between two pools (device and pinned host memory, which the
// kernel reads and writes directly over the host link).  One workgroup per
// (pair, array); the pairs of a launch travel in the kernel arguments, so the
// host's pair list needs no device copy.
__global__ __launch_bounds__(256) void swap_blocks_kernel(SwapArrays arr, SwapChunk chunk,
                                                          int64_t block_bytes,
                                                          int64_t scale_bytes) {
  const int pair = blockIdx.x;
  const int which = blockIdx.y;            // 0 K, 1 V, 2 K scales, 3 V scales
  if (pair >= chunk.n) return;
  const int64_t per = which < 2 ? block_bytes : scale_bytes;
  const uint8_t* s = static_cast<const uint8_t*>(arr.src[which]) + (int64_t)chunk.src[pair] * per;
  uint8_t* d = static_cast<uint8_t*>(arr.dst[which]) + (int64_t)chunk.dst[pair] * per;
  if (((per | (int64_t)(uintptr_t)s | (int64_t)(uintptr_t)d) & 15) == 0) {
    const u32x4* s4 = reinterpret_cast<const u32x4*>(s);
    u32x4* d4 = reinterpret_cast<u32x4*>(d);
    for (int64_t i = threadIdx.x; i < per / 16; i += blockDim.x) d4[i] = s4[i];
  } else {
    for (int64_t i = threadIdx.x; i < per; i += blockDim.x) d[i] = s[i];
  }
}

hipError_t launch_swap_blocks(const SwapArrays& arr, int arrays, const int32_t* pairs,
                              int32_t n_pairs, int64_t block_bytes, int64_t scale_bytes,
                              hipStream_t st) {
  for (int32_t i0 = 0; i0 < n_pairs; i0 += kSwapChunk) {
    SwapChunk c;
    c.n = n_pairs - i0 < kSwapChunk ? n_pairs - i0 : kSwapChunk;
    for (int j = 0; j < c.n; ++j) {
      c.src[j] = pairs[2 * (i0 + j)];
      c.dst[j] = pairs[2 * (i0 + j) + 1];
    }
    hipLaunchKernelGGL(swap_blocks_kernel, dim3(c.n, arrays), dim3(256), 0, st, arr, c,
                       block_bytes, scale_bytes);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* pairs, int32_t n_pairs, int64_t block_bytes,
                              int64_t block_rows, int32_t num_blocks, hipStream_t st) {
  if (n_pairs == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(2 * n_pairs), dim3(256), 0, st,
                     static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), k_scale,
                     v_scale, pairs, block_bytes, block_rows, num_blocks);
  return hipGetLastError();
}

}  // namespace pkv
