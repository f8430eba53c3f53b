"""Seeded synthetic decode batches for the paged KV cache.

Each batch is one decode step: every sequence has ``ctx`` tokens of context, of which
the first ``ctx - 1`` are already in the paged cache and the last one (the new token)
is handed over separately as ``key``/``value`` rows.  The cache layout is
``[num_blocks, block_size, num_kv_heads, head_dim]``; physical block ids are dealt to
sequences from a seeded random permutation of the pool.

What the generator fixes, and nothing more:
  * context lengths drawn from the workload's distribution;
  * block tables (unused entries are -1);
  * N(0, 1) fp32 values, rounded to nearest-even into the storage dtype;
  * poison: every cache row that holds no history (unreferenced blocks, the tail of
    each sequence's last block, the row the new token is about to take) is a NaN
    with a recognisable payload, so that any read outside the context shows up as
    NaN in the result.

The workloads follow the shapes named for the method: a tiny fp32 case, a
Llama-2-7B-shaped MHA layer, a Llama-3-8B-shaped GQA layer, a long-context batch,
and a prefix-shared batch whose groups point at the same physical prefix blocks.
No dataset is involved; these synthetic draws stand in for serving traffic.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np
import torch

BF16_POISON = 0x7FA5          # a quiet NaN in bfloat16 with a payload
F32_POISON = 0x7FC0DEAD       # a quiet NaN in float32 with a payload
FP8_POISON = 0x7F             # the E4M3 NaN code

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
_INT_VIEW = {"f32": torch.int32, "bf16": torch.int16}


# partition_size of the balanced split (the library's PKV_PARTITION_BALANCED); 0 is
# the library's default of 512-token partitions
PARTITION_BALANCED = -1


def poison_bits(kv_dtype: str) -> int:
    return {"f32": F32_POISON, "bf16": BF16_POISON}[kv_dtype]


@dataclass(frozen=True)
class ConfigSpec:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    kv_dtype: str
    max_context: int            # upper end of the context distribution
    ctx: tuple                  # ("fixed", lens) | ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi)
                                # | ("prefix", shared_tokens, suffix_lo, suffix_hi)
    seed: int
    partition_size: int = 512   # tokens per fixed partition, or PARTITION_BALANCED
    share_group: int = 0        # sequences per group sharing a prefix (0: no sharing)
    shared_blocks: int = 0      # physical blocks each group shares
    per_head: bool = False      # fixed partitions in the per-head layout (shared prefixes)

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.max_context // self.block_size)

    @property
    def description(self) -> str:
        return (f"{self.name}: B={self.num_seqs} H={self.num_heads} Hkv={self.num_kv_heads} "
                f"D={self.head_dim} BS={self.block_size} NB={self.num_blocks} {self.kv_dtype} "
                f"ctx={self.ctx}")


CONFIGS = {
    # 4 sequences, MHA 4/4, D=64, fp32, contexts {17, 33, 64, 100}, 64-block pool.
    "tiny": ConfigSpec("tiny", 4, 4, 4, 64, 16, 64, "f32", 100, ("fixed", (17, 33, 64, 100)), 0),
    # One Llama-2-7B layer: MHA 32/32, D=128, bf16, contexts uniform in [128, 2048].  The
    # workload fixes no partition size either; the balanced split measured faster than
    # 512-token partitions on MI355X (5.97 vs 5.38 TB/s).
    "llama2_7b": ConfigSpec("llama2_7b", 64, 32, 32, 128, 16, 16384, "bf16", 2048,
                            ("uniform", 128, 2048), 1, partition_size=PARTITION_BALANCED),
    # One Llama-3-8B layer: GQA 32/8, D=128, bf16, lognormal contexts (median 1024,
    # sigma 1.0 in log space), clipped to [16, 8192], 200k-block pool.  The workload
    # fixes no partition size; it runs in the balanced split, which measured fastest
    # on MI355X.
    "llama3_8b": ConfigSpec("llama3_8b", 256, 32, 8, 128, 16, 200_000, "bf16", 8192,
                            ("lognormal", 1024, 1.0, 16, 8192), 2,
                            partition_size=PARTITION_BALANCED),
    # Long-context split decode: 8 sequences of 32k..128k tokens, partition 512.
    "long_ctx": ConfigSpec("long_ctx", 8, 32, 8, 128, 16, 65536, "bf16", 131072,
                           ("uniform", 32768, 131072), 3),
    # Prefix sharing: 32 groups of 4 sequences; each group shares its first 64
    # physical blocks (2048 tokens at block size 32); unique suffixes of 16..512 tokens.
    # 512-token partitions in the per-head layout, whose workgroups of sharing
    # sequences meet on the shared blocks in the caches.
    "prefix_shared": ConfigSpec("prefix_shared", 128, 32, 8, 128, 32, 16384, "bf16", 2048 + 512,
                                ("prefix", 2048, 16, 512), 4, share_group=4, shared_blocks=64,
                                per_head=True),
}


@dataclass
class DecodeBatch:
    spec: ConfigSpec
    context_lens: np.ndarray        # int32 [B]; includes the new token
    block_tables: np.ndarray        # int32 [B, max_blocks_per_seq]; -1 where unused
    query: torch.Tensor             # [B, H, D]        storage dtype
    key: torch.Tensor               # [B, Hkv, D]      new token K, storage dtype
    value: torch.Tensor             # [B, Hkv, D]      new token V
    key_cache: torch.Tensor         # [NB, BS, Hkv, D] history; poison elsewhere
    value_cache: torch.Tensor       # [NB, BS, Hkv, D]
    scale: float
    extra: dict = field(default_factory=dict)

    # --- shape shorthands -------------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def kv_dtype(self) -> str:
        return self.spec.kv_dtype

    def kv_bytes(self) -> int:
        """Bytes of K and V one decode step must read: sum(ctx) * Hkv * D * 2 * elem."""
        elem = {"f32": 4, "bf16": 2, "fp8": 1}[self.spec.kv_dtype]
        return int(self.context_lens.astype(np.int64).sum()) * self.spec.num_kv_heads * \
            self.spec.head_dim * 2 * elem

    def referenced_blocks(self) -> np.ndarray:
        bt = self.block_tables
        return np.unique(bt[bt >= 0])

    # --- host views for the CPU side -------------------------------------------
    def numpy_storage(self, t: torch.Tensor) -> np.ndarray:
        """Raw storage of a tensor as numpy: float32 for f32, uint16 bit patterns for
        bf16, uint8 codes for an E4M3 cache."""
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.float32:
            return t.numpy()
        if t.dtype == torch.uint8:
            return t.numpy()
        return t.view(torch.int16).numpy().view(np.uint16)


# -----------------------------------------------------------------------------------
# context lengths and block tables
# -----------------------------------------------------------------------------------

def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream]))


def draw_context_lens(spec: ConfigSpec, seed: Optional[int] = None) -> np.ndarray:
    seed = spec.seed if seed is None else seed
    rng = _rng(seed, 0)
    kind = spec.ctx[0]
    B = spec.num_seqs
    if kind == "fixed":
        lens = np.asarray(spec.ctx[1], dtype=np.int64)
        assert lens.shape == (B,)
    elif kind == "uniform":
        lens = rng.integers(spec.ctx[1], spec.ctx[2], size=B, endpoint=True)
    elif kind == "lognormal":
        median, sigma, lo, hi = spec.ctx[1:]
        lens = np.clip(np.rint(np.exp(rng.normal(math.log(median), sigma, size=B))), lo, hi)
    elif kind == "prefix":
        shared, lo, hi = spec.ctx[1:]
        lens = shared + rng.integers(lo, hi, size=B, endpoint=True)
    else:
        raise ValueError(kind)
    return lens.astype(np.int32)


def deal_block_tables(spec: ConfigSpec, context_lens: np.ndarray,
                      seed: Optional[int] = None, max_blocks_per_seq: Optional[int] = None
                      ) -> np.ndarray:
    """Physical ids from a seeded permutation of the pool, dealt to sequences in order.

    With sharing, each group first takes ``shared_blocks`` ids that all its members
    list first; every member then takes its own ids for the rest of its context.
    """
    seed = spec.seed if seed is None else seed
    BS = spec.block_size
    MB = spec.max_blocks_per_seq if max_blocks_per_seq is None else max_blocks_per_seq
    B = context_lens.shape[0]
    nblk = -(-context_lens.astype(np.int64) // BS)
    assert nblk.max() <= MB, "context longer than the block table allows"
    perm = _rng(seed, 1).permutation(spec.num_blocks)
    tables = np.full((B, MB), -1, dtype=np.int32)
    cursor = 0
    if spec.share_group:
        S = spec.shared_blocks
        assert (nblk > S).all(), "every sharer must own at least one block past the prefix"
        assert B % spec.share_group == 0
        for g0 in range(0, B, spec.share_group):
            shared = perm[cursor:cursor + S]
            cursor += S
            for i in range(g0, g0 + spec.share_group):
                own = int(nblk[i]) - S
                tables[i, :S] = shared
                tables[i, S:S + own] = perm[cursor:cursor + own]
                cursor += own
    else:
        for i in range(B):
            n = int(nblk[i])
            tables[i, :n] = perm[cursor:cursor + n]
            cursor += n
    assert cursor <= spec.num_blocks, "pool too small for this batch"
    return tables


# -----------------------------------------------------------------------------------
# values
# -----------------------------------------------------------------------------------

def _randn(gen: torch.Generator, shape, kv_dtype: str, device) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    return x.to(_TORCH_DTYPE[kv_dtype])     # round to nearest even


def _poisoned(shape, kv_dtype: str, device) -> torch.Tensor:
    t = torch.empty(shape, dtype=_TORCH_DTYPE[kv_dtype], device=device)
    t.view(_INT_VIEW[kv_dtype]).fill_(poison_bits(kv_dtype))
    return t


def build_batch(spec: ConfigSpec, context_lens: Sequence[int], device="cpu",
                seed: Optional[int] = None, block_tables: Optional[np.ndarray] = None,
                max_blocks_per_seq: Optional[int] = None) -> DecodeBatch:
    """Make one decode batch for ``spec`` with the given context lengths."""
    seed = spec.seed if seed is None else seed
    ctx = np.asarray(context_lens, dtype=np.int32)
    assert ctx.ndim == 1 and (ctx >= 1).all()
    spec = replace(spec, num_seqs=int(ctx.shape[0]),
                   max_context=max(spec.max_context, int(ctx.max())))
    if block_tables is None:
        block_tables = deal_block_tables(spec, ctx, seed, max_blocks_per_seq)
    B, H, Hkv, D = spec.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_dim
    BS, NB = spec.block_size, spec.num_blocks
    dt = spec.kv_dtype
    device = torch.device(device)

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1_000_003 + 17)
    query = _randn(gen, (B, H, D), dt, device)
    key = _randn(gen, (B, Hkv, D), dt, device)
    value = _randn(gen, (B, Hkv, D), dt, device)

    key_cache = _poisoned((NB, BS, Hkv, D), dt, device)
    value_cache = _poisoned((NB, BS, Hkv, D), dt, device)
    ids = block_tables[block_tables >= 0]
    _, first = np.unique(ids, return_index=True)
    ids = ids[np.sort(first)]                       # referenced ids, first-use order
    chunk = 4096
    for c0 in range(0, ids.shape[0], chunk):
        idx = torch.as_tensor(ids[c0:c0 + chunk].astype(np.int64), device=device)
        n = int(idx.shape[0])
        key_cache[idx] = _randn(gen, (n, BS, Hkv, D), dt, device)
        value_cache[idx] = _randn(gen, (n, BS, Hkv, D), dt, device)

    # Rows at and after the new token's place hold no history yet: poison them.
    # Block j of a sequence holds its tokens j*BS .. j*BS+BS-1.
    kv_int = (key_cache.view(_INT_VIEW[dt]), value_cache.view(_INT_VIEW[dt]))
    for i in range(B):
        history = int(ctx[i]) - 1
        nblk = -(-int(ctx[i]) // BS)
        j = nblk - 1
        live_rows = history - j * BS
        assert 0 <= live_rows < BS
        b = int(block_tables[i, j])
        for t in kv_int:
            t[b, live_rows:].fill_(poison_bits(dt))

    return DecodeBatch(spec=spec, context_lens=ctx, block_tables=block_tables.astype(np.int32),
                       query=query, key=key, value=value, key_cache=key_cache,
                       value_cache=value_cache, scale=1.0 / math.sqrt(D))


# -----------------------------------------------------------------------------------
# several new tokens per sequence (chunked prefill, verification of speculated tokens)
# -----------------------------------------------------------------------------------
# A step hands sequence i q_len_i new tokens, packed into one flat batch in sequence
# order (query_start_loc[i] .. query_start_loc[i+1]); context_lens[i] counts them, so
# the cache holds ctx_i - q_len_i tokens of history.  Values and poison as for decode:
# every row at or after the first new position is poisoned until the step writes it.

def build_multi_batch(spec: ConfigSpec, context_lens: Sequence[int], query_lens: Sequence[int],
                      device="cpu", seed: Optional[int] = None,
                      block_tables: Optional[np.ndarray] = None) -> DecodeBatch:
    """A multi-token step; query/key/value are [T, ...] over the flat token batch and
    ``extra`` holds query_lens and query_start_loc (int32 numpy arrays)."""
    seed = spec.seed if seed is None else seed
    ctx = np.asarray(context_lens, dtype=np.int32)
    ql = np.asarray(query_lens, dtype=np.int32)
    assert ctx.ndim == 1 and ql.shape == ctx.shape and (ql >= 0).all() and (ctx >= 1).all()
    assert (ql <= ctx).all()
    spec = replace(spec, num_seqs=int(ctx.shape[0]),
                   max_context=max(spec.max_context, int(ctx.max())))
    if block_tables is None:
        block_tables = deal_block_tables(spec, ctx, seed)
    B, H, Hkv, D = spec.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_dim
    BS, NB = spec.block_size, spec.num_blocks
    dt = spec.kv_dtype
    T = int(ql.sum())
    qsl = np.zeros(B + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(ql)
    device = torch.device(device)

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1_000_003 + 41)
    query = _randn(gen, (T, H, D), dt, device)
    key = _randn(gen, (T, Hkv, D), dt, device)
    value = _randn(gen, (T, Hkv, D), dt, device)

    key_cache = _poisoned((NB, BS, Hkv, D), dt, device)
    value_cache = _poisoned((NB, BS, Hkv, D), dt, device)
    ids = block_tables[block_tables >= 0]
    _, first = np.unique(ids, return_index=True)
    ids = ids[np.sort(first)]
    chunk = 4096
    for c0 in range(0, ids.shape[0], chunk):
        idx = torch.as_tensor(ids[c0:c0 + chunk].astype(np.int64), device=device)
        n = int(idx.shape[0])
        key_cache[idx] = _randn(gen, (n, BS, Hkv, D), dt, device)
        value_cache[idx] = _randn(gen, (n, BS, Hkv, D), dt, device)
    # history ends at ctx - q_len: poison every row from there to the end of the table
    kv_int = (key_cache.view(_INT_VIEW[dt]), value_cache.view(_INT_VIEW[dt]))
    for i in range(B):
        hist = int(ctx[i]) - int(ql[i])
        nblk = -(-int(ctx[i]) // BS)
        for j in range(hist // BS, nblk):
            b = int(block_tables[i, j])
            r0 = max(0, hist - j * BS)
            for t in kv_int:
                t[b, r0:].fill_(poison_bits(dt))
    return DecodeBatch(spec=spec, context_lens=ctx, block_tables=block_tables.astype(np.int32),
                       query=query, key=key, value=value, key_cache=key_cache,
                       value_cache=value_cache, scale=1.0 / math.sqrt(D),
                       extra={"query_lens": ql, "query_start_loc": qsl})


# Multi-token workloads on the Llama-3-8B layer shape (GQA 32/8, D = 128, bf16, block
# size 16):
#  - spec_verify: 256 sequences with lognormal contexts (as llama3_8b), each verifying
#    5 speculated tokens (the draft length on the pages);
#  - chunked_prefill: a 2048-token step budget (the pages' default) spent on 4
#    prompts' 512-token chunks, after histories uniform in [0, 8192];
#  - chunked_prefill_skewed: the same budget with one long history beside short ones
#    (16000 and 3 x 1000 tokens), where a few long units would set the step's time.
MULTI_CONFIGS = {
    "tiny_multi": (ConfigSpec("tiny_multi", 4, 4, 4, 64, 16, 64, "f32", 100,
                              ("fixed", (17, 33, 64, 100)), 5), ("fixed", (1, 5, 16, 40))),
    "spec_verify": (replace(CONFIGS["llama3_8b"], name="spec_verify", seed=6),
                    ("fixed_all", 5)),
    "chunked_prefill": (ConfigSpec("chunked_prefill", 4, 32, 8, 128, 16, 16384, "bf16",
                                   8192 + 512, ("uniform", 512, 8192 + 512), 7,
                                   partition_size=PARTITION_BALANCED), ("fixed_all", 512)),
    "chunked_prefill_skewed": (ConfigSpec("chunked_prefill_skewed", 4, 32, 8, 128, 16, 16384,
                                          "bf16", 16000 + 512,
                                          ("fixed", (16512, 1512, 1512, 1512)), 7,
                                          partition_size=PARTITION_BALANCED),
                               ("fixed_all", 512)),
}


def make_multi_config(name: str, device="cpu", seed: Optional[int] = None) -> DecodeBatch:
    spec, qdist = MULTI_CONFIGS[name]
    ctx = draw_context_lens(spec, seed)
    if qdist[0] == "fixed":
        ql = np.asarray(qdist[1], dtype=np.int32)
    else:
        ql = np.full(ctx.shape, qdist[1], dtype=np.int32)
    ctx = np.maximum(ctx, ql)        # a sequence holds at least its new tokens
    tables = deal_block_tables(spec, ctx, seed)
    return build_multi_batch(spec, ctx, ql, device=device, seed=seed, block_tables=tables)


# -----------------------------------------------------------------------------------
# E4M3 (FP8) caches
# -----------------------------------------------------------------------------------
# The history rows hold codes drawn uniformly from the 254 finite E4M3 codes (every
# sign, exponent and mantissa), so that every decode case is exercised; with the
# cache scales below the values they stand for span about 1e-6 .. 4 in magnitude.
# Queries and the new tokens' rows are bfloat16 N(0, 1); the write quantises the new
# rows.  The scales are not powers of two, so the fp32 quotient x / scale rounds.
FP8_K_SCALE = 0.0089
FP8_V_SCALE = 0.0113


def _finite_codes(gen: torch.Generator, shape, device) -> torch.Tensor:
    r = torch.randint(0, 254, shape, generator=gen, dtype=torch.int32, device=device)
    return (r + (r >= FP8_POISON).to(torch.int32)).to(torch.uint8)   # skip 0x7F; 0xFF unreachable


def build_fp8_batch(spec: ConfigSpec, context_lens: Sequence[int], device="cpu",
                    seed: Optional[int] = None, block_tables: Optional[np.ndarray] = None,
                    max_blocks_per_seq: Optional[int] = None) -> DecodeBatch:
    """One decode batch with E4M3 caches (uint8 codes) for ``spec`` (kv_dtype "fp8");
    ``extra`` holds k_scale and v_scale."""
    assert spec.kv_dtype == "fp8"
    seed = spec.seed if seed is None else seed
    ctx = np.asarray(context_lens, dtype=np.int32)
    assert ctx.ndim == 1 and (ctx >= 1).all()
    spec = replace(spec, num_seqs=int(ctx.shape[0]),
                   max_context=max(spec.max_context, int(ctx.max())))
    if block_tables is None:
        block_tables = deal_block_tables(spec, ctx, seed, max_blocks_per_seq)
    B, H, Hkv, D = spec.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_dim
    BS, NB = spec.block_size, spec.num_blocks
    device = torch.device(device)

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1_000_003 + 29)
    query = _randn(gen, (B, H, D), "bf16", device)
    key = _randn(gen, (B, Hkv, D), "bf16", device)
    value = _randn(gen, (B, Hkv, D), "bf16", device)

    key_cache = torch.full((NB, BS, Hkv, D), FP8_POISON, dtype=torch.uint8, device=device)
    value_cache = torch.full((NB, BS, Hkv, D), FP8_POISON, dtype=torch.uint8, device=device)
    ids = block_tables[block_tables >= 0]
    _, first = np.unique(ids, return_index=True)
    ids = ids[np.sort(first)]
    chunk = 8192
    for c0 in range(0, ids.shape[0], chunk):
        idx = torch.as_tensor(ids[c0:c0 + chunk].astype(np.int64), device=device)
        n = int(idx.shape[0])
        key_cache[idx] = _finite_codes(gen, (n, BS, Hkv, D), device)
        value_cache[idx] = _finite_codes(gen, (n, BS, Hkv, D), device)
    for i in range(B):
        history = int(ctx[i]) - 1
        j = -(-int(ctx[i]) // BS) - 1
        b = int(block_tables[i, j])
        key_cache[b, history - j * BS:].fill_(FP8_POISON)
        value_cache[b, history - j * BS:].fill_(FP8_POISON)
    return DecodeBatch(spec=spec, context_lens=ctx, block_tables=block_tables.astype(np.int32),
                       query=query, key=key, value=value, key_cache=key_cache,
                       value_cache=value_cache, scale=1.0 / math.sqrt(D),
                       extra={"k_scale": FP8_K_SCALE, "v_scale": FP8_V_SCALE})


# E4M3-cache forms of the named workloads: same shapes, context draws and tables.
FP8_CONFIGS = {
    "tiny_fp8": replace(CONFIGS["tiny"], name="tiny_fp8", kv_dtype="fp8",
                        partition_size=PARTITION_BALANCED),
    "llama3_8b_fp8": replace(CONFIGS["llama3_8b"], name="llama3_8b_fp8", kv_dtype="fp8"),
    "long_ctx_fp8": replace(CONFIGS["long_ctx"], name="long_ctx_fp8", kv_dtype="fp8",
                            partition_size=PARTITION_BALANCED),
}


def make_fp8_config(name: str, device="cpu", seed: Optional[int] = None,
                    num_seqs: Optional[int] = None) -> DecodeBatch:
    spec = FP8_CONFIGS[name]
    ctx = draw_context_lens(spec, seed)
    tables = deal_block_tables(spec, ctx, seed)
    if num_seqs is not None:
        ctx, tables = ctx[:num_seqs], tables[:num_seqs]
    return build_fp8_batch(spec, ctx, device=device, seed=seed, block_tables=tables)


def make_config(name: str, device="cpu", seed: Optional[int] = None,
                num_seqs: Optional[int] = None) -> DecodeBatch:
    """The named workload; ``num_seqs`` keeps only the first sequences (same draws)."""
    spec = CONFIGS[name]
    ctx = draw_context_lens(spec, seed)
    tables = deal_block_tables(spec, ctx, seed)
    if num_seqs is not None:
        ctx, tables = ctx[:num_seqs], tables[:num_seqs]
    return build_batch(spec, ctx, device=device, seed=seed, block_tables=tables)


# -----------------------------------------------------------------------------------
# relabelling helpers for the invariance checks
# -----------------------------------------------------------------------------------

def permute_physical_blocks(batch: DecodeBatch, perm: np.ndarray) -> DecodeBatch:
    """Move block b to ``perm[b]`` and relabel the tables: same logical content."""
    NB = batch.spec.num_blocks
    perm = np.asarray(perm, dtype=np.int64)
    assert sorted(perm.tolist()) == list(range(NB))
    p = torch.as_tensor(perm, device=batch.key_cache.device)
    kc = torch.empty_like(batch.key_cache)
    vc = torch.empty_like(batch.value_cache)
    kc[p] = batch.key_cache
    vc[p] = batch.value_cache
    bt = batch.block_tables
    new_bt = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    return replace(batch, block_tables=new_bt, key_cache=kc, value_cache=vc)


def unshare_prefix_blocks(batch: DecodeBatch) -> DecodeBatch:
    """Give every sequence of a sharing group private copies of the shared blocks."""
    spec = batch.spec
    assert spec.share_group and spec.shared_blocks
    S, G = spec.shared_blocks, spec.share_group
    bt = batch.block_tables.copy()
    free = np.setdiff1d(np.arange(spec.num_blocks), batch.referenced_blocks())
    kc = batch.key_cache.clone()
    vc = batch.value_cache.clone()
    cursor = 0
    dev = kc.device
    for g0 in range(0, batch.num_seqs, G):
        for i in range(g0 + 1, g0 + G):
            src = torch.as_tensor(bt[i, :S].astype(np.int64), device=dev)
            dst_np = free[cursor:cursor + S]
            cursor += S
            assert dst_np.shape[0] == S, "pool too small to unshare"
            dst = torch.as_tensor(dst_np.astype(np.int64), device=dev)
            kc[dst] = kc[src]
            vc[dst] = vc[src]
            bt[i, :S] = dst_np
    return replace(batch, block_tables=bt, key_cache=kc, value_cache=vc)
