// Host block pool of libpagedkv: the physical KV blocks' free list and reference
// counts, fork, the copy-on-write decision for a sequence's next token, and prefix
// caching.
//
// Semantics (page "vllm源码分析：我是如何一步步读懂PagedAttention核心实现的？", 第一讲,
// the BlockAllocator: a first-in first-out list of free ids, allocation takes the
// front and sets the count to 1, an empty list is an error, a block returns to the
// back of the list when its count reaches 0; page "读一个真实 serving 系统 · vLLM 架构
// 巡礼", the ref_cnt paragraph: shared blocks are copied before they are changed; page
// "vLLM PagedAttention 原理与源码深度解析", sections 3.3 and 5.2: a full last block
// means a new block).
//
// Prefix caching (page "vllm源码剖析", the BlockPool paragraphs: a full block's hash
// covers its tokens and its predecessor's hash and maps to the block; a hit raises the
// block's count; a block at count 0 rejoins the free queue and its hash is cleared
// when it is handed out again; page "读一个真实 serving 系统 · vLLM 架构巡礼", section 2,
// the _block_hash field and touch()).  The pages name no hash function: this pool
// uses 64-bit FNV-1a over the parent hash (8 bytes, little-endian; 0 for the first
// block) and the block's token ids (4 bytes each).  A hit also compares the stored
// tokens and parent hash, so a hash collision never shares a block.
//
// The free list is intrusive and doubly linked (prev/next per block), so allocate,
// release and the removal of a free block hit by a lookup are O(1).  A pool is not
// thread-safe; callers serialise the calls on one pool.
#include <climits>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"

namespace {

constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

uint64_t fnv_bytes(uint64_t h, const unsigned char* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

// Hash of one full block: FNV-1a of the parent hash then the tokens, little-endian.
uint64_t block_hash(uint64_t parent, const int32_t* tokens, int32_t n) {
  unsigned char b[8];
  for (int k = 0; k < 8; ++k) b[k] = static_cast<unsigned char>(parent >> (8 * k));
  uint64_t h = fnv_bytes(kFnvOffset, b, 8);
  for (int32_t i = 0; i < n; ++i) {
    const uint32_t t = static_cast<uint32_t>(tokens[i]);
    for (int k = 0; k < 4; ++k) b[k] = static_cast<unsigned char>(t >> (8 * k));
    h = fnv_bytes(h, b, 4);
  }
  return h;
}

}  // namespace

struct pkv_block_pool {
  std::vector<int32_t> prev, next;   // free list links; -1 ends it
  std::vector<int32_t> ref;          // reference count per block
  std::vector<int32_t> pending;      // release(): references asked per block; 0 between calls
  std::vector<uint8_t> is_free;
  int32_t head = -1, tail = -1;      // front and back of the free list
  int64_t count = 0;                 // free blocks
  // prefix cache
  int32_t block_size = 0;            // fixed by the first prefix-cache call
  std::vector<uint8_t> cached_flag;  // the block holds a hash in the map
  std::vector<uint64_t> hash, parent;
  std::vector<int32_t> tokens;       // [num_blocks][block_size] of cached blocks
  std::unordered_map<uint64_t, int32_t> cached;

  explicit pkv_block_pool(int32_t n)
      : prev(n), next(n), ref(n, 0), pending(n, 0), is_free(n, 1), cached_flag(n, 0), hash(n, 0),
        parent(n, 0) {
    for (int32_t i = 0; i < n; ++i) {
      prev[i] = i - 1;
      next[i] = i + 1 < n ? i + 1 : -1;
    }
    head = 0;
    tail = n - 1;
    count = n;
  }
  int32_t size() const { return static_cast<int32_t>(ref.size()); }
  bool valid(int32_t b) const { return b >= 0 && b < size(); }

  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    is_free[b] = 0;
    --count;
  }
  void push(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    is_free[b] = 1;
    ++count;
  }
  // A reallocated block leaves the prefix cache.
  void evict(int32_t b) {
    if (!cached_flag[b]) return;
    auto it = cached.find(hash[b]);
    if (it != cached.end() && it->second == b) cached.erase(it);
    cached_flag[b] = 0;
  }
  bool pop(int32_t* b) {
    if (count == 0) return false;
    *b = head;
    unlink(head);
    evict(*b);
    ref[*b] = 1;
    return true;
  }
  // Drops one reference; the block goes back to the free list at zero (keeping its
  // hash until it is handed out again).
  void drop(int32_t b) {
    if (--ref[b] == 0) push(b);
  }
  bool set_block_size(int32_t bs) {
    if (block_size == 0) {
      block_size = bs;
      tokens.assign(static_cast<size_t>(size()) * bs, 0);
    }
    return block_size == bs;
  }
  const int32_t* block_tokens(int32_t b) const {
    return tokens.data() + static_cast<size_t>(b) * block_size;
  }
};

extern "C" {

pkv_status pkv_block_pool_create(int32_t num_blocks, pkv_block_pool** pool) {
  if (!pool || num_blocks <= 0) return PKV_ERR_INVALID_ARG;
  *pool = new (std::nothrow) pkv_block_pool(num_blocks);
  return *pool ? PKV_OK : PKV_ERR_INVALID_ARG;
}

void pkv_block_pool_destroy(pkv_block_pool* pool) { delete pool; }

int32_t pkv_block_pool_num_free(const pkv_block_pool* pool) {
  return pool ? static_cast<int32_t>(pool->count) : -1;
}

int32_t pkv_block_pool_ref_count(const pkv_block_pool* pool, int32_t block) {
  return pool && pool->valid(block) ? pool->ref[block] : -1;
}

pkv_status pkv_block_pool_allocate(pkv_block_pool* pool, int32_t* block) {
  if (!pool || !block) return PKV_ERR_INVALID_ARG;
  return pool->pop(block) ? PKV_OK : PKV_ERR_NO_BLOCKS;
}

pkv_status pkv_block_pool_release(pkv_block_pool* pool, const int32_t* blocks, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !blocks)) return PKV_ERR_INVALID_ARG;
  // check first, so that a bad list changes nothing (a block listed k times must
  // hold at least k references)
  for (int32_t i = 0; i < n; ++i) {
    if (!pool->valid(blocks[i])) return PKV_ERR_INVALID_ARG;
  }
  // count the references asked per block in the pool's reusable array, then clear
  // only the entries this list touched: O(n), whatever the pool's size
  int32_t counted = 0;
  bool ok = true;
  for (; counted < n; ++counted) {
    const int32_t b = blocks[counted];
    if (++pool->pending[b] > pool->ref[b]) {
      ok = false;
      ++counted;
      break;
    }
  }
  for (int32_t i = 0; i < counted; ++i) pool->pending[blocks[i]] = 0;
  if (!ok) return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) pool->drop(blocks[i]);
  return PKV_OK;
}

pkv_status pkv_block_pool_fork(pkv_block_pool* pool, const int32_t* blocks, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !blocks)) return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (!pool->valid(blocks[i]) || pool->ref[blocks[i]] <= 0) return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) ++pool->ref[blocks[i]];
  return PKV_OK;
}

pkv_status pkv_block_pool_append_slots(pkv_block_pool* pool, int32_t* tables,
                                       int32_t* table_lens, int32_t table_capacity,
                                       const int32_t* num_tokens, int32_t num_seqs,
                                       int32_t block_size, int32_t* slots, int32_t* copies,
                                       int32_t* num_copies, int32_t* done) {
  if (!pool || num_seqs < 0 || table_capacity <= 0 || block_size <= 0 || !num_copies || !done)
    return PKV_ERR_INVALID_ARG;
  *num_copies = 0;
  *done = 0;
  if (num_seqs == 0) return PKV_OK;
  if (!tables || !table_lens || !num_tokens || !slots || !copies) return PKV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(pool->size()) * block_size > INT32_MAX)
    return PKV_ERR_INVALID_ARG;   // slots are int32
  for (int32_t i = 0; i < num_seqs; ++i) {
    int32_t* table = tables + static_cast<int64_t>(i) * table_capacity;
    const int32_t n = num_tokens[i];
    const int32_t len = table_lens[i];
    if (n < 0 || len < 0 || len > table_capacity) return PKV_ERR_INVALID_ARG;
    const int32_t logical = n / block_size, offset = n % block_size;
    if (offset == 0) {
      // the token opens a new logical block
      if (logical != len || len == table_capacity) return PKV_ERR_INVALID_ARG;
      int32_t b;
      if (!pool->pop(&b)) return PKV_ERR_NO_BLOCKS;
      table[len] = b;
      table_lens[i] = len + 1;
    } else {
      if (logical != len - 1 || !pool->valid(table[len - 1]) || pool->ref[table[len - 1]] <= 0)
        return PKV_ERR_INVALID_ARG;
      const int32_t last = table[len - 1];
      if (pool->ref[last] > 1) {
        // shared: copy it before the token is written
        int32_t fresh;
        if (!pool->pop(&fresh)) return PKV_ERR_NO_BLOCKS;
        copies[2 * *num_copies] = last;
        copies[2 * *num_copies + 1] = fresh;
        ++*num_copies;
        pool->drop(last);
        table[len - 1] = fresh;
      }
    }
    slots[i] = table[logical] * block_size + offset;
    *done = i + 1;
  }
  return PKV_OK;
}

// ---- prefix caching ---------------------------------------------------------------

pkv_status pkv_prefix_block_hashes(const int32_t* tokens, int32_t num_tokens,
                                   int32_t block_size, uint64_t* hashes) {
  if (num_tokens < 0 || block_size <= 0) return PKV_ERR_INVALID_ARG;
  const int32_t nb = num_tokens / block_size;
  if (nb == 0) return PKV_OK;
  if (!tokens || !hashes) return PKV_ERR_INVALID_ARG;
  uint64_t h = 0;
  for (int32_t j = 0; j < nb; ++j) {
    h = block_hash(h, tokens + static_cast<int64_t>(j) * block_size, block_size);
    hashes[j] = h;
  }
  return PKV_OK;
}

int32_t pkv_block_pool_num_cached(const pkv_block_pool* pool) {
  return pool ? static_cast<int32_t>(pool->cached.size()) : -1;
}

pkv_status pkv_block_pool_match_prefix(pkv_block_pool* pool, const int32_t* tokens,
                                       int32_t num_tokens, int32_t block_size,
                                       int32_t* blocks, int32_t max_blocks, int32_t* num_hit) {
  if (!pool || num_tokens < 0 || block_size <= 0 || max_blocks < 0 || !num_hit)
    return PKV_ERR_INVALID_ARG;
  *num_hit = 0;
  if (num_tokens > 0 && !tokens) return PKV_ERR_INVALID_ARG;
  if (max_blocks > 0 && !blocks) return PKV_ERR_INVALID_ARG;
  if (!pool->set_block_size(block_size)) return PKV_ERR_INVALID_ARG;
  const int32_t nb = num_tokens / block_size;
  const size_t row = static_cast<size_t>(block_size) * sizeof(int32_t);
  int32_t hits = 0;
  uint64_t parent = 0;
  for (int32_t j = 0; j < nb && hits < max_blocks; ++j) {
    const int32_t* t = tokens + static_cast<int64_t>(j) * block_size;
    const uint64_t h = block_hash(parent, t, block_size);
    const auto it = pool->cached.find(h);
    if (it == pool->cached.end()) break;
    const int32_t b = it->second;
    if (pool->parent[b] != parent || std::memcmp(pool->block_tokens(b), t, row) != 0) break;
    blocks[hits++] = b;
    parent = h;
  }
  for (int32_t k = 0; k < hits; ++k) {   // touch
    const int32_t b = blocks[k];
    if (pool->ref[b] == 0) pool->unlink(b);
    ++pool->ref[b];
  }
  *num_hit = hits;
  return PKV_OK;
}

pkv_status pkv_block_pool_register_prefix(pkv_block_pool* pool, const int32_t* tokens,
                                          int32_t num_tokens, int32_t block_size,
                                          const int32_t* table, int32_t table_len,
                                          int32_t* num_registered) {
  if (!pool || num_tokens < 0 || block_size <= 0 || table_len < 0 || !num_registered)
    return PKV_ERR_INVALID_ARG;
  *num_registered = 0;
  const int32_t nb = num_tokens / block_size;
  if (nb == 0) return pool->set_block_size(block_size) ? PKV_OK : PKV_ERR_INVALID_ARG;
  if (!tokens || !table || table_len < nb) return PKV_ERR_INVALID_ARG;
  if (!pool->set_block_size(block_size)) return PKV_ERR_INVALID_ARG;
  for (int32_t j = 0; j < nb; ++j)   // check first: a bad table changes nothing
    if (!pool->valid(table[j]) || pool->ref[table[j]] <= 0) return PKV_ERR_INVALID_ARG;
  const size_t row = static_cast<size_t>(block_size) * sizeof(int32_t);
  int32_t n = 0;
  uint64_t parent = 0;
  for (int32_t j = 0; j < nb; ++j) {
    const int32_t b = table[j];
    const int32_t* t = tokens + static_cast<int64_t>(j) * block_size;
    const uint64_t h = block_hash(parent, t, block_size);
    if (!pool->cached_flag[b] && pool->cached.find(h) == pool->cached.end()) {
      pool->cached.emplace(h, b);
      pool->cached_flag[b] = 1;
      pool->hash[b] = h;
      pool->parent[b] = parent;
      std::memcpy(pool->tokens.data() + static_cast<size_t>(b) * block_size, t, row);
      ++n;
    }
    parent = h;
  }
  *num_registered = n;
  return PKV_OK;
}

}  // extern "C"
