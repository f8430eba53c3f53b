"""CPU fp64 oracle for one PagedAttention decode step.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU-baseline
leg may import this module.  It shares no code with the HIP path; it is written to be
read against the pages, not to be fast.

What it computes, step by step, for a batch of decode sequences:

  O1  slot of the new token.  A sequence's token at 0-based position ``pos`` lives in
      logical block ``pos // block_size`` at offset ``pos % block_size``; the block
      table turns the logical block into a physical one, and the flat slot is
      ``physical * block_size + offset``.  (Page "vllm源码剖析", section 一.3
      "请求和显存块的映射", the worked example of how a token's offset is found:
      block size 4, tokens 1-4 in block 0, 5-8 in block 1, offset by the modulus.)
      Reading adopted: ``context_lens`` counts the new token, so the new token sits
      at ``pos = ctx - 1``.
  O2  cache write (reshape_and_cache).  The new token's K and V rows are copied, bit
      for bit, into ``cache[slot // block_size, slot % block_size]`` -- the cache
      ``[num_blocks, block_size, num_kv_heads, head_dim]`` seen as a flat array of
      slots.  (Same page, section 一.2 "为什么要reshape": the first two dims merged so
      each token's row is contiguous.)  A negative slot means "no token" and is
      skipped.
  O3  gather.  For sequence i and kv head g, walk the block table in logical order,
      take rows ``[0, block_size)`` of each physical block, concatenate, keep the
      first ``ctx`` rows.  (Page "vllm源码分析：我是如何一步步读懂PagedAttention核心
      实现的？", 第三讲: the block-table indirection from logical block i to the
      physical block; page "vLLM PagedAttention 原理与源码深度解析", 5.3 注意力计算:
      gather K/V through ``block_tables`` up to ``context_lens``.)
  O4  scores ``s_t = scale * <q_h, k_t>`` in fp64, with q head h reading kv head
      ``h // (num_heads // num_kv_heads)``.  (5.3 注意力计算 on the deep-dive page
      divides by sqrt(head_dim); here the scale is an argument.)
  O5  softmax over the context with the maximum subtracted first.
  O6  ``out_h = sum_t p_t v_t / sum_t p_t``.
  O7  (formula check only) the same result through fixed-size context partitions,
      each giving (max m_k, sum l_k, normalised partial o_k), merged by
      ``M = max m_k``, ``w_k = l_k * exp(m_k - M)``, ``out = sum w_k o_k / sum w_k``.
      The pages do not print this merge; it is the log-sum-exp identity.

Storage: f32 caches are float32 arrays; bf16 caches are uint16 arrays of raw
bfloat16 bit patterns.  Values are widened to fp64 exactly before any arithmetic.

Pins (tests/test_oracle.py): the worked slot example; bitwise invariance under any
relabelling of physical blocks; equality with torch's scaled-dot-product attention in
fp64 (a library routine) on the gathered dense K/V; brute-force pure-Python loops on
tiny inputs; closed forms (one-token context gives V exactly, zero query or equal keys
give the mean of V, one dominant key gives its V); the partition merge against the
unpartitioned result.
"""

from __future__ import annotations

import math

import numpy as np


# ----------------------------------------------------------------------------------
# storage decoding
# ----------------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the top half of a float32: shift the 16 bits up and reinterpret."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_f64(arr: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(arr)
    raise ValueError(kv_dtype)


# ----------------------------------------------------------------------------------
# O1, O2
# ----------------------------------------------------------------------------------

def token_place(pos: int, block_size: int):
    """(logical block, offset) of the token at 0-based position ``pos``."""
    return pos // block_size, pos % block_size


def slot_mapping(block_tables: np.ndarray, context_lens: np.ndarray, block_size: int) -> np.ndarray:
    """O1: flat cache slot of each sequence's new token (the one at ctx - 1)."""
    B = context_lens.shape[0]
    slots = np.empty(B, dtype=np.int64)
    for i in range(B):
        pos = int(context_lens[i]) - 1
        logical, offset = token_place(pos, block_size)
        physical = int(block_tables[i, logical])
        slots[i] = physical * block_size + offset
    return slots


def cache_write(key_cache: np.ndarray, value_cache: np.ndarray, key: np.ndarray,
                value: np.ndarray, slots: np.ndarray, block_size: int):
    """O2: copies of the caches with each token's K/V rows stored at its slot."""
    kc = key_cache.copy()
    vc = value_cache.copy()
    for t in range(slots.shape[0]):
        s = int(slots[t])
        if s < 0:
            continue
        kc[s // block_size, s % block_size] = key[t]
        vc[s // block_size, s % block_size] = value[t]
    return kc, vc


# ----------------------------------------------------------------------------------
# O3 .. O6
# ----------------------------------------------------------------------------------

def gather_context(cache: np.ndarray, table_row: np.ndarray, ctx: int, kv_head: int,
                   kv_dtype: str) -> np.ndarray:
    """O3: the sequence's first ``ctx`` rows for one kv head, in logical order, fp64."""
    block_size = cache.shape[1]
    nblk = -(-ctx // block_size)
    pieces = [cache[int(table_row[j]), :, kv_head, :] for j in range(nblk)]
    return to_f64(np.concatenate(pieces, axis=0)[:ctx], kv_dtype)


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """O4-O6 for one query vector over a contiguous context (all fp64)."""
    s = scale * (K @ q)
    m = s.max()
    p = np.exp(s - m)
    return (p @ V) / p.sum()


def paged_attention_decode(query: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                           block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                           kv_dtype: str, seqs=None) -> np.ndarray:
    """Decode attention of one query token per sequence over its paged context.

    ``query`` is [B, H, D] storage; caches are [NB, BS, Hkv, D] storage.  Returns
    fp64 [len(seqs), H, D] (all sequences when ``seqs`` is None).
    """
    B, H, D = query.shape
    Hkv = key_cache.shape[2]
    group = H // Hkv
    seqs = range(B) if seqs is None else seqs
    seqs = list(seqs)
    out = np.empty((len(seqs), H, D), dtype=np.float64)
    q64 = to_f64(query, kv_dtype)
    for n, i in enumerate(seqs):
        ctx = int(context_lens[i])
        for g in range(Hkv):
            K = gather_context(key_cache, block_tables[i], ctx, g, kv_dtype)
            V = gather_context(value_cache, block_tables[i], ctx, g, kv_dtype)
            for h in range(g * group, (g + 1) * group):
                out[n, h] = softmax_attention(q64[i, h], K, V, scale)
    return out


def decode_step(query, key, value, key_cache, value_cache, block_tables, context_lens,
                scale, kv_dtype, seqs=None):
    """O1 + O2 + O3..O6: write the new tokens, then attend.  Returns (slots, kc, vc, out)."""
    block_size = key_cache.shape[1]
    slots = slot_mapping(block_tables, context_lens, block_size)
    kc, vc = cache_write(key_cache, value_cache, key, value, slots, block_size)
    out = paged_attention_decode(query, kc, vc, block_tables, context_lens, scale, kv_dtype,
                                 seqs=seqs)
    return slots, kc, vc, out


# ----------------------------------------------------------------------------------
# O7: partitions and their log-sum-exp merge
# ----------------------------------------------------------------------------------

def partition_stats(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                    partition_size: int):
    """Per partition k of the context: (m_k, l_k, o_k) with o_k already divided by l_k."""
    stats = []
    for start in range(0, K.shape[0], partition_size):
        s = scale * (K[start:start + partition_size] @ q)
        m = s.max()
        p = np.exp(s - m)
        lsum = p.sum()
        stats.append((m, lsum, (p @ V[start:start + partition_size]) / lsum))
    return stats


def merge_partitions(stats) -> np.ndarray:
    M = max(m for m, _, _ in stats)
    weights = [lsum * math.exp(m - M) for m, lsum, _ in stats]
    num = sum(w * o for w, (_, _, o) in zip(weights, stats))
    return num / sum(weights)


def partitioned_attention_decode(query, key_cache, value_cache, block_tables, context_lens,
                                 scale, kv_dtype, partition_size, seqs=None):
    B, H, D = query.shape
    Hkv = key_cache.shape[2]
    group = H // Hkv
    seqs = list(range(B) if seqs is None else seqs)
    out = np.empty((len(seqs), H, D), dtype=np.float64)
    q64 = to_f64(query, kv_dtype)
    for n, i in enumerate(seqs):
        ctx = int(context_lens[i])
        for g in range(Hkv):
            K = gather_context(key_cache, block_tables[i], ctx, g, kv_dtype)
            V = gather_context(value_cache, block_tables[i], ctx, g, kv_dtype)
            for h in range(g * group, (g + 1) * group):
                out[n, h] = merge_partitions(partition_stats(q64[i, h], K, V, scale,
                                                             partition_size))
    return out
