"""CPU fp64 oracle for a step with several new tokens per sequence: chunked prefill and
the verification of speculated tokens, over the paged cache, with a causal mask.

TEST INFRASTRUCTURE.  Only the tests and the bench's CPU-baseline leg may import this
module.  It shares no code with the HIP path.

The pages describe one scheduler for every kind of step: a request has a number of
tokens already computed and a number it must reach, and each step hands it some new
tokens (page "读一个真实 serving 系统 · vLLM 架构巡礼", section 3 on schedule(): no
separate prefill and decode phases, chunked prefill and speculative decoding fall
under the same rule; page "vLLM PagedAttention 原理与源码深度解析", sections 8.1 and
8.2: a long prompt is cut into chunks, and a draft model proposes 5 tokens that the
main model verifies).  The new tokens of all requests are packed into one flat batch
that records where each request starts and how many tokens it has (page
"vllm源码剖析", section 一.3, the mapping of requests onto one-dimensional data).
The pages print no kernel for this step; what follows is the plainest reading:

  M1  layout.  Sequence i owns the new tokens query_start_loc[i] ..
      query_start_loc[i+1] - 1 of the flat batch (q_len_i of them).  context_lens[i]
      counts every token of the sequence after the step, the new ones included (as
      for decode), so new token j sits at position p = ctx_i - q_len_i + j.
  M2  slots and write.  The token at position p has slot
      table[i][p // block_size] * block_size + p % block_size (the decode step's O1 at
      every new position); its K/V rows are stored there (O2).
  M3  causal attention.  New token j of sequence i attends to positions 0 .. p of its
      sequence (its own row included, nothing after it): scores scale * <q, k_t>,
      softmax over t <= p, weighted sum of v_t (the decode step's O3-O6 over the
      first p + 1 positions).  Decode is the case q_len_i = 1.
  M4  invalid input.  A sequence with ctx_i < q_len_i or ctx_i beyond its table gets
      no slots (-1) and NaN outputs; q_len_i = 0 contributes nothing.

Pins (tests/test_multi_query.py): q_len = 1 equals the decode oracle (pinned on its
own); equality with torch's scaled-dot-product attention in fp64 with an explicit
causal mask on the dense K/V; invariance under relabelling of physical blocks;
brute-force loops on tiny inputs; chunking invariance (a prompt processed in two
chunks, the second after the first chunk's rows were written, equals one chunk
covering both); the worked slot example of the decode pins at several positions.
"""

from __future__ import annotations

import numpy as np

from .paged_decode import gather_context, softmax_attention, to_f64, token_place


def _layout(query_start_loc: np.ndarray, context_lens: np.ndarray, i: int):
    q0 = int(query_start_loc[i])
    q_len = int(query_start_loc[i + 1]) - q0
    ctx = int(context_lens[i])
    return q0, q_len, ctx


def _valid(ctx: int, q_len: int, max_ctx: int) -> bool:
    return q_len <= ctx <= max_ctx


def slot_mapping_multi(block_tables: np.ndarray, context_lens: np.ndarray,
                       query_start_loc: np.ndarray, block_size: int) -> np.ndarray:
    """M1/M2: slot of every new token of the flat batch (-1 for M4)."""
    B = context_lens.shape[0]
    T = int(query_start_loc[B])
    max_ctx = block_tables.shape[1] * block_size
    slots = np.full(T, -1, dtype=np.int64)
    for i in range(B):
        q0, q_len, ctx = _layout(query_start_loc, context_lens, i)
        if not _valid(ctx, q_len, max_ctx):
            continue
        for j in range(q_len):
            p = ctx - q_len + j
            logical, offset = token_place(p, block_size)
            slots[q0 + j] = int(block_tables[i, logical]) * block_size + offset
    return slots


def paged_attention_multi_query(query: np.ndarray, key_cache: np.ndarray,
                                value_cache: np.ndarray, block_tables: np.ndarray,
                                context_lens: np.ndarray, query_start_loc: np.ndarray,
                                scale: float, kv_dtype: str, seqs=None,
                                tokens=None) -> np.ndarray:
    """M3/M4: fp64 outputs [T, H, D] for the flat batch.  ``seqs`` / ``tokens``
    restrict the work to some sequences / flat token indices; the other rows are
    left as NaN."""
    T, H, D = query.shape
    B = context_lens.shape[0]
    Hkv = key_cache.shape[2]
    block_size = key_cache.shape[1]
    group = H // Hkv
    max_ctx = block_tables.shape[1] * block_size
    out = np.full((T, H, D), np.nan)
    q64 = to_f64(query, kv_dtype)
    want = None if tokens is None else set(int(t) for t in tokens)
    for i in (range(B) if seqs is None else seqs):
        q0, q_len, ctx = _layout(query_start_loc, context_lens, i)
        if q_len == 0 or not _valid(ctx, q_len, max_ctx):
            continue
        js = [j for j in range(q_len) if want is None or q0 + j in want]
        if not js:
            continue
        for g in range(Hkv):
            K = gather_context(key_cache, block_tables[i], ctx, g, kv_dtype)
            V = gather_context(value_cache, block_tables[i], ctx, g, kv_dtype)
            for j in js:
                p = ctx - q_len + j
                for h in range(g * group, (g + 1) * group):
                    out[q0 + j, h] = softmax_attention(q64[q0 + j, h], K[:p + 1], V[:p + 1],
                                                       scale)
    return out


def multi_query_step(query, key, value, key_cache, value_cache, block_tables, context_lens,
                     query_start_loc, scale, kv_dtype, seqs=None, tokens=None):
    """M2 then M3: write every new token's rows, then attend.  Returns
    (slots, kc, vc, out)."""
    from .paged_decode import cache_write
    block_size = key_cache.shape[1]
    slots = slot_mapping_multi(block_tables, context_lens, query_start_loc, block_size)
    kc, vc = cache_write(key_cache, value_cache, key, value, slots, block_size)
    out = paged_attention_multi_query(query, kc, vc, block_tables, context_lens,
                                      query_start_loc, scale, kv_dtype, seqs=seqs,
                                      tokens=tokens)
    return slots, kc, vc, out
