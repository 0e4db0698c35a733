// Host block pool: the control plane that hands out the physical blocks whose
// ids fill the block tables the kernels read.
//
// Follows "vLLM 架构概述" §5.1 (the block pool: a doubly linked free list with O(1)
// allocation and release, a prefix-cache map from block hash to block, and per-block
// reference counts and hashes) and the reading note on "Inside vLLM", core points 1
// (allocate_slots: ceil(new tokens / 16) blocks taken from the head of the free list,
// after checking there are enough, and recorded per request) and 3 (a block's hash
// chains the previous block's hash, the block's tokens and optional extra identity;
// find_longest_cache_hit scans for the longest cached prefix).  "vLLM：从 KV Cache 到高吞吐
// 推理服务", tutorial 3, names the null block and eviction of cached free blocks, and
// tutorial 4 several physical copies of one hash.
//
// Design: block ids index flat arrays (prev/next links of the intrusive free list, ref
// counts, hashes), so every list operation is O(1) with no allocation; requests and the
// hash map are hash tables.  Block 0 is the null block: never handed out, never counted,
// the placeholder of released table entries.
#include <stdint.h>

#include <algorithm>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

struct pa_block_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  // intrusive free list over block ids; kNil ends it
  static constexpr int32_t kNil = -1;
  std::vector<int32_t> prev, next;
  std::vector<uint8_t> in_queue;
  int32_t head = kNil, tail = kNil, num_free = 0;
  std::vector<int32_t> ref;
  std::vector<uint64_t> hash;
  std::vector<uint8_t> has_hash;
  std::unordered_map<uint64_t, std::vector<int32_t>> cached;  // hash -> physical copies, oldest first
  struct Request {
    std::vector<int32_t> blocks;
    int32_t num_cached = 0;  // leading blocks whose hash is committed (or were hits)
  };
  std::unordered_map<int64_t, Request> requests;

  void push_tail(int32_t b) {
    prev[b] = tail;
    next[b] = kNil;
    if (tail != kNil) next[tail] = b; else head = b;
    tail = b;
    in_queue[b] = 1;
    ++num_free;
  }
  void unlink(int32_t b) {
    if (prev[b] != kNil) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] != kNil) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = kNil;
    in_queue[b] = 0;
    --num_free;
  }
  // drops a cached block's hash (eviction, when the block is handed out again)
  void evict(int32_t b) {
    if (!has_hash[b]) return;
    auto it = cached.find(hash[b]);
    if (it != cached.end()) {
      auto& v = it->second;
      v.erase(std::remove(v.begin(), v.end(), b), v.end());
      if (v.empty()) cached.erase(it);
    }
    has_hash[b] = 0;
    hash[b] = 0;
  }
  int32_t pop_head() {
    const int32_t b = head;
    unlink(b);
    evict(b);
    return b;
  }
  void release(int32_t b) {
    if (b == 0) return;
    if (--ref[b] == 0) push_tail(b);
  }
};

namespace {

// 64-bit FNV-1a (Fowler, Noll, Vo): offset basis 14695981039346656037, prime 1099511628211.
struct Fnv1a64 {
  uint64_t h = 14695981039346656037ull;
  void bytes(const void* p, size_t n) {
    const auto* c = static_cast<const unsigned char*>(p);
    for (size_t i = 0; i < n; ++i) {
      h ^= c[i];
      h *= 1099511628211ull;
    }
  }
  void u64(uint64_t v) {
    unsigned char b[8];
    for (int i = 0; i < 8; ++i) b[i] = (unsigned char)(v >> (8 * i));
    bytes(b, 8);
  }
  void i32(int32_t v) {
    unsigned char b[4];
    for (int i = 0; i < 4; ++i) b[i] = (unsigned char)((uint32_t)v >> (8 * i));
    bytes(b, 4);
  }
};

pa_status_t bad(pa_status_t st, const char* msg) { return pa::set_error(st, "%s", msg); }

}  // namespace

extern "C" {

pa_status_t pa_pool_create(int32_t num_blocks, int32_t block_size, pa_block_pool_t** pool) {
  if (!pool) return bad(PA_ERR_NULL, "pa_pool_create: pool is NULL");
  *pool = nullptr;
  if (num_blocks < 2) return pa::set_error(PA_ERR_SHAPE, "pa_pool_create: num_blocks %d < 2", num_blocks);
  if (block_size < 1) return pa::set_error(PA_ERR_SHAPE, "pa_pool_create: block_size %d < 1", block_size);
  auto* p = new pa_block_pool;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->prev.assign(num_blocks, pa_block_pool::kNil);
  p->next.assign(num_blocks, pa_block_pool::kNil);
  p->in_queue.assign(num_blocks, 0);
  p->ref.assign(num_blocks, 0);
  p->hash.assign(num_blocks, 0);
  p->has_hash.assign(num_blocks, 0);
  for (int32_t b = 1; b < num_blocks; ++b) p->push_tail(b);
  *pool = p;
  return PA_OK;
}

void pa_pool_destroy(pa_block_pool_t* pool) { delete pool; }

int32_t pa_pool_num_free(const pa_block_pool_t* pool) { return pool ? pool->num_free : -1; }

int32_t pa_pool_hash_blocks(const int32_t* tokens, int32_t num_tokens, int32_t block_size, uint64_t extra_key,
                            uint64_t* hashes) {
  if (!tokens || !hashes || num_tokens < 0 || block_size < 1) return -1;
  const int32_t full = num_tokens / block_size;
  uint64_t parent = 0;  // the chain's root
  for (int32_t i = 0; i < full; ++i) {
    Fnv1a64 f;
    f.u64(parent);
    for (int32_t t = 0; t < block_size; ++t) f.i32(tokens[(size_t)i * block_size + t]);
    f.u64(extra_key);
    hashes[i] = parent = f.h;
  }
  return full;
}

int32_t pa_pool_find_longest_cache_hit(const pa_block_pool_t* pool, const uint64_t* hashes, int32_t num_hashes,
                                       int32_t* blocks) {
  if (!pool || (num_hashes > 0 && (!hashes || !blocks)) || num_hashes < 0) return -1;
  int32_t n = 0;
  for (; n < num_hashes; ++n) {
    auto it = pool->cached.find(hashes[n]);
    if (it == pool->cached.end()) break;
    blocks[n] = it->second.front();
  }
  return n;
}

pa_status_t pa_pool_allocate_slots(pa_block_pool_t* pool, int64_t request_id, int32_t num_tokens,
                                   const int32_t* hit_blocks, int32_t num_hit_blocks, int32_t* num_blocks) {
  if (!pool) return bad(PA_ERR_NULL, "pa_pool_allocate_slots: pool is NULL");
  if (num_tokens < 0 || num_hit_blocks < 0 || (num_hit_blocks > 0 && !hit_blocks))
    return bad(PA_ERR_SHAPE, "pa_pool_allocate_slots: negative count or missing hit_blocks");
  auto it = pool->requests.find(request_id);
  const bool known = it != pool->requests.end();
  if (known && num_hit_blocks > 0)
    return bad(PA_ERR_STATE, "pa_pool_allocate_slots: cache hits are only taken when a request is first allocated");
  const int32_t have = known ? (int32_t)it->second.blocks.size() : 0;
  const int64_t want = ((int64_t)num_tokens + pool->block_size - 1) / pool->block_size;
  if (num_hit_blocks > want)
    return bad(PA_ERR_SHAPE, "pa_pool_allocate_slots: more hit blocks than the tokens need");
  // hits that sit in the free list leave it when touched
  int32_t hits_free = 0;
  for (int32_t i = 0; i < num_hit_blocks; ++i) {
    const int32_t b = hit_blocks[i];
    if (b < 1 || b >= pool->num_blocks || !pool->has_hash[b])
      return pa::set_error(PA_ERR_SHAPE, "pa_pool_allocate_slots: hit block %d is not a cached block", b);
    hits_free += pool->in_queue[b];
  }
  if (num_hit_blocks > 1) {
    std::vector<int32_t> sorted(hit_blocks, hit_blocks + num_hit_blocks);
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
      return bad(PA_ERR_SHAPE, "pa_pool_allocate_slots: repeated hit block");
  }
  const int64_t fresh = std::max<int64_t>(0, want - have - num_hit_blocks);
  if (fresh + hits_free > pool->num_free)
    return pa::set_error(PA_ERR_NO_SPACE, "pa_pool_allocate_slots: %lld blocks needed, %d free",
                         (long long)(fresh + hits_free), pool->num_free);
  pa_block_pool::Request& r = pool->requests[request_id];
  for (int32_t i = 0; i < num_hit_blocks; ++i) {  // touch
    const int32_t b = hit_blocks[i];
    if (pool->in_queue[b]) pool->unlink(b);
    ++pool->ref[b];
    r.blocks.push_back(b);
  }
  if (!known) r.num_cached = num_hit_blocks;
  for (int64_t i = 0; i < fresh; ++i) {
    const int32_t b = pool->pop_head();
    pool->ref[b] = 1;
    r.blocks.push_back(b);
  }
  if (num_blocks) *num_blocks = (int32_t)r.blocks.size();
  return PA_OK;
}

pa_status_t pa_pool_cache_blocks(pa_block_pool_t* pool, int64_t request_id, const uint64_t* hashes,
                                 int32_t num_full_blocks) {
  if (!pool) return bad(PA_ERR_NULL, "pa_pool_cache_blocks: pool is NULL");
  auto it = pool->requests.find(request_id);
  if (it == pool->requests.end()) return bad(PA_ERR_STATE, "pa_pool_cache_blocks: unknown request");
  pa_block_pool::Request& r = it->second;
  if (num_full_blocks < 0 || num_full_blocks > (int32_t)r.blocks.size() || (num_full_blocks > 0 && !hashes))
    return bad(PA_ERR_SHAPE, "pa_pool_cache_blocks: num_full_blocks outside the request's blocks");
  for (int32_t i = r.num_cached; i < num_full_blocks; ++i) {
    const int32_t b = r.blocks[i];
    if (b == 0 || pool->has_hash[b]) continue;  // released entry, or already cached
    pool->hash[b] = hashes[i];
    pool->has_hash[b] = 1;
    pool->cached[hashes[i]].push_back(b);
  }
  r.num_cached = std::max(r.num_cached, num_full_blocks);
  return PA_OK;
}

pa_status_t pa_pool_release_before(pa_block_pool_t* pool, int64_t request_id, int32_t position) {
  if (!pool) return bad(PA_ERR_NULL, "pa_pool_release_before: pool is NULL");
  auto it = pool->requests.find(request_id);
  if (it == pool->requests.end()) return bad(PA_ERR_STATE, "pa_pool_release_before: unknown request");
  auto& blocks = it->second.blocks;
  const int32_t n = std::min<int64_t>(std::max(position, 0) / pool->block_size, (int64_t)blocks.size());
  for (int32_t j = 0; j < n; ++j) {
    pool->release(blocks[j]);
    blocks[j] = 0;
  }
  return PA_OK;
}

pa_status_t pa_pool_free(pa_block_pool_t* pool, int64_t request_id) {
  if (!pool) return bad(PA_ERR_NULL, "pa_pool_free: pool is NULL");
  auto it = pool->requests.find(request_id);
  if (it == pool->requests.end()) return bad(PA_ERR_STATE, "pa_pool_free: unknown request");
  // the last blocks first: they are the least likely to be shared, so they are evicted first
  const auto& blocks = it->second.blocks;
  for (auto b = blocks.rbegin(); b != blocks.rend(); ++b) pool->release(*b);
  pool->requests.erase(it);
  return PA_OK;
}

int32_t pa_pool_block_table(const pa_block_pool_t* pool, int64_t request_id, int32_t* out, int32_t max_blocks) {
  if (!pool) return -1;
  auto it = pool->requests.find(request_id);
  if (it == pool->requests.end()) return -1;
  const auto& blocks = it->second.blocks;
  if (out) std::copy_n(blocks.begin(), std::min<size_t>(blocks.size(), (size_t)std::max(max_blocks, 0)), out);
  return (int32_t)blocks.size();
}

pa_status_t pa_pool_block_state(const pa_block_pool_t* pool, int32_t block, int32_t* ref_count, int32_t* is_free,
                                int32_t* has_hash, uint64_t* hash) {
  if (!pool) return bad(PA_ERR_NULL, "pa_pool_block_state: pool is NULL");
  if (block < 0 || block >= pool->num_blocks) return bad(PA_ERR_SHAPE, "pa_pool_block_state: block out of range");
  if (ref_count) *ref_count = pool->ref[block];
  if (is_free) *is_free = pool->in_queue[block];
  if (has_hash) *has_hash = pool->has_hash[block];
  if (hash) *hash = pool->hash[block];
  return PA_OK;
}

int32_t pa_pool_free_queue(const pa_block_pool_t* pool, int32_t* out, int32_t max_blocks) {
  if (!pool) return -1;
  int32_t n = 0;
  for (int32_t b = pool->head; b != pa_block_pool::kNil; b = pool->next[b], ++n)
    if (out && n < max_blocks) out[n] = b;
  return n;
}

}  // extern "C"
