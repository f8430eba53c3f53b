"""CPU oracle of the paged KV block pool: allocation, reference counts, fork,
copy-on-write append, and the block copy that copy-on-write needs.

TEST INFRASTRUCTURE.  Only the tests may import this module.  It shares no code with
the library's C++ pool or its HIP kernels; it is written to be read against the pages.

What it models, from the pages:

  P1  allocate.  The free blocks form a first-in first-out list that starts as block ids
      0 .. num_blocks-1; allocation takes the first id and sets its reference count to
      1; an empty list is an error.  (Page "vllm源码分析：我是如何一步步读懂PagedAttention
      核心实现的？", 第一讲, the BlockAllocator of v0.4.2: a deque of free ids, allocate
      takes from the left and raises when there is none.)
  P2  free.  The reference count drops by one; at zero the block goes to the back of
      the free list.  (Same passage, BlockAllocator.free; page "vllm源码剖析", the
      BlockPool paragraph: a block whose count reaches 0 goes back to the free queue.)
  P3  fork.  A new sequence shares every block of its parent: its table is a copy of
      the parent's and every shared block's count grows by one.  (Same 第一讲, the
      copy-on-write paragraph on beam search and try_fork; page "读一个真实 serving 系统 ·
      vLLM 架构巡礼", the ref_cnt paragraph: requests that share a prefix point at the same
      blocks and touch() raises the count.)
  P4  append slot.  The slot of a sequence's next token, at position n (the number of
      tokens it already has).  When n is a multiple of block_size the token opens a new
      logical block: allocate one and append it to the table.  Otherwise the token goes
      into the last block; if that block is shared (count > 1) it is copied first:
      allocate a fresh block, record the copy (old -> new), drop one reference to the old
      block and put the new one in the table.  The slot is
      table[n // block_size] * block_size + n % block_size.  (Page "vLLM PagedAttention
      原理与源码深度解析", section 3.3 and section 5.2 append_slot: a full last block means a
      new block; 架构巡礼: a shared block is copied before it is changed.)  Reading: the
      sketch in section 3.3 writes the token into the old last block after allocating a
      new one; here the token goes to the block that holds its position.
  P5  copy blocks.  For each (src, dst) pair the rows of block dst in the key and value
      caches become bitwise copies of block src's rows.

Pins (tests/test_block_pool.py): first-in first-out order of fresh and freed ids; the
exhaustion error; reference counts equal to the number of live tables that hold each
block and a free list of exactly the unreferenced blocks, after random operation
sequences (counted by scanning the tables, not by the pool's own bookkeeping); a worked
beam-search scenario whose slots and copies are derived by hand from P1-P4; bitwise
block copies.
"""

from __future__ import annotations

from collections import deque

import numpy as np


class PoolExhausted(Exception):
    """No free block is left (P1)."""


class BlockPool:
    """P1-P3: the free list and the reference counts of num_blocks physical blocks."""

    def __init__(self, num_blocks: int):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        self.num_blocks = num_blocks
        self.free = deque(range(num_blocks))
        self.ref = [0] * num_blocks

    def allocate(self) -> int:
        if not self.free:
            raise PoolExhausted("No free blocks available")
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def release(self, block: int) -> None:
        if self.ref[block] <= 0:
            raise ValueError(f"block {block} is not in use")
        self.ref[block] -= 1
        if self.ref[block] == 0:
            self.free.append(block)

    def fork(self, table: list) -> list:
        for b in table:
            if self.ref[b] <= 0:
                raise ValueError(f"block {b} is not in use")
            self.ref[b] += 1
        return list(table)

    def release_table(self, table: list) -> None:
        for b in table:
            self.release(b)

    def append_slot(self, table: list, n_tokens: int, block_size: int):
        """P4.  Updates ``table`` in place; returns (slot, copies) with copies a list of
        (src, dst) block pairs to copy before the token is written."""
        copies = []
        logical, offset = divmod(n_tokens, block_size)
        if offset == 0:
            if logical != len(table):
                raise ValueError("table length does not match the token count")
            table.append(self.allocate())
        else:
            if logical != len(table) - 1:
                raise ValueError("table length does not match the token count")
            last = table[-1]
            if self.ref[last] > 1:
                fresh = self.allocate()
                copies.append((last, fresh))
                self.release(last)
                table[-1] = fresh
        return table[logical] * block_size + offset, copies


def copy_blocks(key_cache: np.ndarray, value_cache: np.ndarray, pairs):
    """P5: copies of the caches with block dst replaced by block src for every pair
    (applied in order)."""
    kc = key_cache.copy()
    vc = value_cache.copy()
    for src, dst in pairs:
        kc[int(dst)] = kc[int(src)]
        vc[int(dst)] = vc[int(src)]
    return kc, vc
