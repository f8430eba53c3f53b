"""CPU oracle of prefix caching on the block pool: chained block hashes, the
hash-to-block lookup, touch on a hit, and eviction when a cached free block is
reallocated.

TEST INFRASTRUCTURE.  Only the tests may import this module.  It shares no code with
the library's C++ pool.

What it models, from the pages:

  H1  block hash.  Only full blocks are cached.  A block's hash covers its tokens and
      the hash of the block before it, so equal hashes mean equal whole prefixes.
      (Page "vllm源码剖析", the BlockPool paragraphs: the hash of a logical block is
      computed from its token content and its predecessor's hash, and
      cached_block_hash_to_block maps it to the block; page "读一个真实 serving 系统 ·
      vLLM 架构巡礼", section 2: _block_hash is the key for prefix-cache lookups.)
      The pages name no hash function.  Reading: 64-bit FNV-1a (Fowler, Noll, Vo)
      over the little-endian bytes of the parent hash (8 bytes; 0 for the first
      block) followed by the block's token ids (4 bytes each).
  H2  lookup.  A new request's prompt is hashed block by block from the start; the
      longest run of leading blocks found in the map is reused.  A hit must also match
      the stored tokens and parent hash, so that two prefixes never share a block
      through a hash collision (the pages do not discuss collisions; this check makes
      a hit exact).
  H3  touch.  A reused block's reference count grows by one; if it was free (count 0)
      it leaves the free list.  (Same BlockPool paragraphs: on a hit only the count is
      raised; 架构巡礼: touch() raises the count on a shared-prefix hit.)
  H4  register.  After a request's full blocks hold their K/V, their hashes enter the
      map; a hash already mapped to another block keeps its first block.
  H5  eviction.  A block whose count drops to 0 goes back to the end of the free list
      and keeps its hash, so it can still be hit; when the free list hands it out
      again, its hash leaves the map.  (Same page: a block at count 0 rejoins the free
      queue, and its hash mapping is cleared when it is reallocated.)

Pins (tests/test_prefix_cache.py): FNV-1a against its published test vectors; the
chain property (a change in one token changes that block's hash and every later one,
equal prefixes give equal hashes); a worked scenario of two requests sharing a
system prompt, derived by hand from H1-H5; collision safety with the hash forced to
a constant; invariants under random operation sequences (counts equal the holders,
free and referenced blocks partition the pool, every cached hash names a block with
the right content).
"""

from __future__ import annotations

from .block_pool import BlockPool

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes) -> int:
    """64-bit FNV-1a: for each byte, xor it in, then multiply by the prime mod 2^64."""
    h = FNV_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_hash(parent: int, tokens) -> int:
    """H1 for one full block."""
    data = int(parent).to_bytes(8, "little")
    for t in tokens:
        data += (int(t) & 0xFFFFFFFF).to_bytes(4, "little")
    return fnv1a64(data)


def chain_hashes(tokens, block_size: int) -> list:
    """H1 for every full block of a token sequence, in order."""
    out = []
    parent = 0
    for j in range(len(tokens) // block_size):
        parent = block_hash(parent, tokens[j * block_size:(j + 1) * block_size])
        out.append(parent)
    return out


class PrefixCachingPool(BlockPool):
    """The block pool (P1-P4 of block_pool.py) with H2-H5."""

    def __init__(self, num_blocks: int, hash_fn=block_hash):
        super().__init__(num_blocks)
        self.hash_fn = hash_fn
        self.cached = {}            # hash -> block
        self.meta = {}              # block -> (hash, parent hash, tokens)

    def _evict(self, b: int) -> None:
        if b in self.meta:
            h = self.meta.pop(b)[0]
            if self.cached.get(h) == b:
                del self.cached[h]

    def allocate(self) -> int:
        b = super().allocate()          # front of the free list
        self._evict(b)                  # H5
        return b

    def match_prefix(self, tokens, block_size: int) -> list:
        """H2 + H3: the reused leading blocks of ``tokens`` (their counts raised)."""
        hits = []
        parent = 0
        for j in range(len(tokens) // block_size):
            blk = tuple(int(t) for t in tokens[j * block_size:(j + 1) * block_size])
            h = self.hash_fn(parent, blk)
            b = self.cached.get(h)
            if b is None or self.meta[b][1] != parent or self.meta[b][2] != blk:
                break
            hits.append(b)
            parent = h
        for b in hits:                  # touch
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
        return hits

    def register(self, tokens, table, block_size: int) -> int:
        """H4: enter the full blocks of a sequence whose K/V are stored in ``table``;
        returns how many new hashes entered the map."""
        n = 0
        parent = 0
        for j in range(len(tokens) // block_size):
            b = int(table[j])
            if self.ref[b] <= 0:
                raise ValueError(f"block {b} is not in use")
            blk = tuple(int(t) for t in tokens[j * block_size:(j + 1) * block_size])
            h = self.hash_fn(parent, blk)
            if b not in self.meta and h not in self.cached:
                self.meta[b] = (h, parent, blk)
                self.cached[h] = b
                n += 1
            parent = h
        return n
