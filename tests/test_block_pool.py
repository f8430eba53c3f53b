"""The block pool oracle against what the pages fix (CPU)."""

import random

import numpy as np
import pytest

from oracle.block_pool import BlockPool, PoolExhausted, copy_blocks


# ----------------------------------------------------------------------------------
# the oracle's pins
# ----------------------------------------------------------------------------------

def test_fresh_ids_in_order_and_freed_ids_go_to_the_back():
    p = BlockPool(5)
    assert [p.allocate() for _ in range(3)] == [0, 1, 2]
    p.release(1)
    p.release(0)
    # free list is now 3, 4, 1, 0 (first in, first out)
    assert [p.allocate() for _ in range(4)] == [3, 4, 1, 0]


def test_exhaustion_is_an_error():
    p = BlockPool(2)
    p.allocate(), p.allocate()
    with pytest.raises(PoolExhausted):
        p.allocate()


def test_block_returns_only_when_its_last_reference_goes():
    p = BlockPool(3)
    t = [p.allocate()]
    u = p.fork(t)
    assert p.ref[t[0]] == 2
    p.release_table(t)
    assert p.ref[u[0]] == 1 and list(p.free) == [1, 2]
    p.release_table(u)
    assert list(p.free) == [1, 2, 0]


def test_worked_beam_scenario():
    # Derived by hand from P1-P4 with block_size 16: sequence A holds 20 tokens in
    # blocks [0, 1]; B is forked from A; both then append.
    bs = 16
    p = BlockPool(8)
    a = []
    for n in range(20):
        p.append_slot(a, n, bs)
    assert a == [0, 1] and p.ref[:2] == [1, 1]
    b = p.fork(a)
    assert p.ref[:2] == [2, 2]
    # A's token 20 lands in shared block 1 at offset 4: copy 1 -> 2 first
    slot, copies = p.append_slot(a, 20, bs)
    assert (slot, copies, a, b) == (2 * 16 + 4, [(1, 2)], [0, 2], [0, 1])
    assert p.ref[:3] == [2, 1, 1]
    # B's token 20: block 1 is B's alone now, no copy
    slot, copies = p.append_slot(b, 20, bs)
    assert (slot, copies) == (1 * 16 + 4, [])
    # B fills block 1 and opens a new block at token 32
    for n in range(21, 32):
        assert p.append_slot(b, n, bs)[1] == []
    slot, copies = p.append_slot(b, 32, bs)
    assert (slot, copies, b) == (3 * 16 + 0, [], [0, 1, 3])
    # block 0 (the shared prefix) is never copied: appends never touch it
    assert p.ref[0] == 2


def _check_consistent(p, tables):
    counts = [0] * p.num_blocks
    for t in tables:
        for blk in t:
            counts[blk] += 1
    assert counts == p.ref
    free = list(p.free)
    assert len(free) == len(set(free))
    assert set(free) == {i for i in range(p.num_blocks) if counts[i] == 0}


def _random_ops(p, rng, bs, steps, record=None):
    """Random forks, appends and finishes; the reference counts are checked against a
    scan of the live tables after every operation."""
    seqs = []          # [table, n_tokens]
    for _ in range(steps):
        r = rng.random()
        try:
            if r < 0.15 or not seqs:
                t = []
                slot, cp = p.append_slot(t, 0, bs)
                seqs.append([t, 1])
                out = ("new", slot, cp)
            elif r < 0.3:
                i = rng.randrange(len(seqs))
                seqs.append([p.fork(seqs[i][0]), seqs[i][1]])
                out = ("fork", i)
            elif r < 0.4:
                i = rng.randrange(len(seqs))
                t, _ = seqs.pop(i)
                p.release_table(t)
                out = ("finish", i)
            else:
                i = rng.randrange(len(seqs))
                slot, cp = p.append_slot(seqs[i][0], seqs[i][1], bs)
                seqs[i][1] += 1
                out = ("append", i, slot, cp)
        except PoolExhausted:
            out = ("exhausted",)
        if record is not None:
            record.append(out)
        _check_consistent(p, [t for t, _ in seqs])
    return seqs


@pytest.mark.parametrize("seed", range(6))
def test_reference_counts_match_the_live_tables(seed):
    rng = random.Random(seed)
    p = BlockPool(rng.choice([4, 16, 64]))
    _random_ops(p, rng, rng.choice([1, 2, 4, 16]), 400)


def test_copy_on_write_preserves_every_sequence_contents():
    # Brute force: keep a token list per sequence; after copy-on-write appends, each
    # table's slots must hold exactly its own tokens (a fake one-element cache).
    rng = random.Random(7)
    bs, nb = 4, 64
    p = BlockPool(nb)
    cache = np.full(nb * bs, -1, np.int64)
    seqs = []      # [table, tokens]
    for step in range(300):
        if not seqs or rng.random() < 0.2:
            t, toks = [], []
            seqs.append([t, toks])
        elif rng.random() < 0.2:
            i = rng.randrange(len(seqs))
            seqs.append([p.fork(seqs[i][0]), list(seqs[i][1])])
            continue
        i = rng.randrange(len(seqs))
        t, toks = seqs[i]
        try:
            slot, copies = p.append_slot(t, len(toks), bs)
        except PoolExhausted:
            break
        for src, dst in copies:
            cache[dst * bs:(dst + 1) * bs] = cache[src * bs:(src + 1) * bs]
        cache[slot] = step
        toks.append(step)
        for t2, toks2 in seqs:
            got = [int(cache[t2[n // bs] * bs + n % bs]) for n in range(len(toks2))]
            assert got == toks2


def test_copy_blocks_copies_whole_blocks_only():
    rng = np.random.default_rng(0)
    kc = rng.integers(0, 2**16, (8, 4, 2, 3), dtype=np.uint16)
    vc = rng.integers(0, 2**16, (8, 4, 2, 3), dtype=np.uint16)
    k2, v2 = copy_blocks(kc, vc, [(1, 5), (1, 6), (3, 0)])
    for src, dst in [(1, 5), (1, 6), (3, 0)]:
        assert (k2[dst] == kc[src]).all() and (v2[dst] == vc[src]).all()
    for b in (1, 2, 3, 4, 7):
        assert (k2[b] == kc[b]).all() and (v2[b] == vc[b]).all()


def test_planted_mistakes_fail_the_pins(monkeypatch):
    # copy-on-write also for unshared blocks: the worked scenario catches it
    orig = BlockPool.append_slot

    def cow_always(self, table, n, bs):
        if n % bs and self.ref[table[-1]] >= 1:
            self.ref[table[-1]] += 1
        return orig(self, table, n, bs)

    monkeypatch.setattr(BlockPool, "append_slot", cow_always)
    with pytest.raises((AssertionError, PoolExhausted)):
        test_worked_beam_scenario()
    monkeypatch.setattr(BlockPool, "append_slot", orig)

    # a free that forgets the free list: the table scan catches it
    def leaky(self, b):
        self.ref[b] -= 1

    monkeypatch.setattr(BlockPool, "release", leaky)
    with pytest.raises(AssertionError):
        test_reference_counts_match_the_live_tables(0)
