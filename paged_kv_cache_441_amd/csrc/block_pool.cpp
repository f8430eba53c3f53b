// Host block pool of libpagedkv: the physical KV blocks' free list and reference
// counts, fork, and the copy-on-write decision for a sequence's next token.
//
// Semantics (page "vllm源码分析：我是如何一步步读懂PagedAttention核心实现的？", 第一讲,
// the BlockAllocator: a first-in first-out list of free ids, allocation takes the
// front and sets the count to 1, an empty list is an error, a block returns to the
// back of the list when its count reaches 0; page "读一个真实 serving 系统 · vLLM 架构
// 巡礼", the ref_cnt paragraph: shared blocks are copied before they are changed; page
// "vLLM PagedAttention 原理与源码深度解析", sections 3.3 and 5.2: a full last block
// means a new block).  The free list is a ring buffer, so allocate and release are
// O(1).  A pool is not thread-safe; callers serialise the calls on one pool.
#include <climits>
#include <cstdint>
#include <new>
#include <vector>

#include "../../include/pagedkv.h"

struct pkv_block_pool {
  std::vector<int32_t> ring;   // free ids, first in first out
  std::vector<int32_t> ref;    // reference count per block
  int64_t head = 0;            // index of the first free id in ring
  int64_t count = 0;           // free ids in ring

  explicit pkv_block_pool(int32_t n) : ring(n), ref(n, 0), count(n) {
    for (int32_t i = 0; i < n; ++i) ring[i] = i;
  }
  int32_t size() const { return static_cast<int32_t>(ref.size()); }
  bool valid(int32_t b) const { return b >= 0 && b < size(); }
  bool pop(int32_t* b) {
    if (count == 0) return false;
    *b = ring[head];
    head = (head + 1) % size();
    --count;
    ref[*b] = 1;
    return true;
  }
  void push(int32_t b) {
    ring[(head + count) % size()] = b;
    ++count;
  }
  // Drops one reference; the block goes back to the free list at zero.
  void drop(int32_t b) {
    if (--ref[b] == 0) push(b);
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
  std::vector<int32_t> need;
  for (int32_t i = 0; i < n; ++i) {
    if (!pool->valid(blocks[i])) return PKV_ERR_INVALID_ARG;
  }
  need.assign(pool->size(), 0);
  for (int32_t i = 0; i < n; ++i)
    if (++need[blocks[i]] > pool->ref[blocks[i]]) return PKV_ERR_INVALID_ARG;
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

}  // extern "C"
