"""The seeded input generators: determinism, table structure, poison placement."""

import numpy as np
import pytest
import torch

from workloads import CONFIGS, make_config, poison_bits
from workloads.decode_batches import deal_block_tables, draw_context_lens


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).numpy()


def test_same_seed_same_batch():
    a, b = make_config("tiny"), make_config("tiny")
    assert (a.context_lens == b.context_lens).all()
    assert (a.block_tables == b.block_tables).all()
    for x, y in ((a.query, b.query), (a.key_cache, b.key_cache), (a.value, b.value)):
        assert (_bits(x) == _bits(y)).all()
    c = make_config("tiny", seed=5)
    assert not (_bits(a.query) == _bits(c.query)).all()


@pytest.mark.parametrize("name", list(CONFIGS))
def test_tables_and_context_distribution(name):
    spec = CONFIGS[name]
    ctx = draw_context_lens(spec)
    bt = deal_block_tables(spec, ctx)
    assert bt.shape == (spec.num_seqs, spec.max_blocks_per_seq)
    nblk = -(-ctx.astype(np.int64) // spec.block_size)
    for i in range(spec.num_seqs):
        assert (bt[i, :nblk[i]] >= 0).all() and (bt[i, nblk[i]:] == -1).all()
    used = bt[bt >= 0]
    assert used.max() < spec.num_blocks
    if spec.share_group:
        S, G = spec.shared_blocks, spec.share_group
        for g0 in range(0, spec.num_seqs, G):
            for i in range(g0 + 1, g0 + G):
                assert (bt[i, :S] == bt[g0, :S]).all()
        # suffix blocks are private, and the new token lands past the shared prefix
        private = np.concatenate([bt[i, S:nblk[i]] for i in range(spec.num_seqs)])
        assert np.unique(private).size == private.size
        assert ((ctx - 1) // spec.block_size >= S).all()
    else:
        assert np.unique(used).size == used.size          # no block is referenced twice
    lo_hi = {"tiny": (17, 100), "llama2_7b": (128, 2048), "llama3_8b": (16, 8192),
             "long_ctx": (32768, 131072), "prefix_shared": (2048 + 16, 2048 + 512)}[name]
    assert ctx.min() >= lo_hi[0] and ctx.max() <= lo_hi[1]
    if name == "llama3_8b":
        assert 800 <= np.median(ctx) <= 1300


def test_poison_placement_tiny():
    b = make_config("tiny")
    BS = b.spec.block_size
    P = poison_bits("f32")
    kbits = _bits(b.key_cache)
    used = set(b.referenced_blocks().tolist())
    for blk in range(b.spec.num_blocks):
        if blk not in used:
            assert (kbits[blk] == P).all()
    for i in range(b.num_seqs):
        ctx = int(b.context_lens[i])
        for t in range(-(-ctx // BS) * BS):
            row = kbits[b.block_tables[i, t // BS], t % BS]
            if t < ctx - 1:
                assert (row != P).all()
            else:
                assert (row == P).all()


def test_fp8_batch_codes_and_poison():
    from workloads import make_fp8_config
    from workloads.decode_batches import FP8_POISON
    b = make_fp8_config("tiny_fp8")
    a = make_fp8_config("tiny_fp8")
    assert b.key_cache.dtype == torch.uint8 and b.query.dtype == torch.bfloat16
    assert torch.equal(a.key_cache, b.key_cache) and torch.equal(a.value, b.value)
    assert b.kv_bytes() == int(b.context_lens.sum()) * 4 * 64 * 2
    BS = b.spec.block_size
    used = set(b.referenced_blocks().tolist())
    for cache in (b.key_cache.numpy(), b.value_cache.numpy()):
        for blk in range(b.spec.num_blocks):
            if blk not in used:
                assert (cache[blk] == FP8_POISON).all()
        hist = []
        for i in range(b.num_seqs):
            ctx = int(b.context_lens[i])
            for t in range(-(-ctx // BS) * BS):
                row = cache[b.block_tables[i, t // BS], t % BS]
                if t < ctx - 1:
                    hist.append(row)
                else:
                    assert (row == FP8_POISON).all()
        hist = np.concatenate(hist)
        # history rows: finite codes only (no 0x7F / 0xFF), every sign and exponent
        assert not np.isin(hist, [0x7F, 0xFF]).any()
        assert len(np.unique(hist >> 3)) == 32
    # same context draws and tables as the bf16/f32 form of the workload
    c = make_config("tiny")
    assert (c.context_lens == b.context_lens).all() and (c.block_tables == b.block_tables).all()
