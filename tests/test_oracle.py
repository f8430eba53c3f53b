"""Pins for the CPU fp64 oracle: each checks it against something other than itself.

Every test here runs on the CPU.  A plausible mistake anywhere in the oracle (a
dropped scale, a wrong head mapping, an off-by-one context, a wrong slot formula, a
missing max subtraction, a wrong merge weight) fails at least one of them; the
planted-mistake tests at the bottom show that for the main ones.
"""

import json
import math
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, DecodeBatch, build_batch, make_config, permute_physical_blocks
from workloads.decode_batches import ConfigSpec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(batch, t):
    return batch.numpy_storage(t)


def _small_gqa(ctx=(1, 15, 16, 17, 40, 97), seed=11, dtype="bf16", D=128, G=4, Hkv=2, BS=16,
               NB=128):
    spec = ConfigSpec("small", len(ctx), G * Hkv, Hkv, D, BS, NB, dtype, max(ctx),
                      ("fixed", tuple(ctx)), seed)
    return build_batch(spec, ctx, device="cpu", seed=seed)


# --------------------------------------------------------------------------------
# O1: the worked example on the pages
# --------------------------------------------------------------------------------

def test_worked_example_slots():
    g = json.load(open(os.path.join(GOLDEN, "slot_worked_example.json")))
    bs = g["block_size"]
    table = np.array([g["block_table"]], dtype=np.int32)
    for k, tok in enumerate(g["tokens"]):
        pos = tok - 1
        assert oracle.token_place(pos, bs) == (g["logical_block"][k], g["offset"][k])
        # token ``tok`` is the new token of a context of length ``tok``
        slots = oracle.slot_mapping(table, np.array([tok], dtype=np.int32), bs)
        assert int(slots[0]) == g["slot"][k]
    for tok in g["stated_entries"]["offset"]:
        assert oracle.token_place(tok - 1, bs)[1] == g["offset"][tok - 1]


def test_worked_example_with_scattered_blocks():
    # Same example, but the request's three logical blocks live in physical blocks
    # 5, 2, 9: the offset within a block is unchanged, only the block moves.
    g = json.load(open(os.path.join(GOLDEN, "slot_worked_example.json")))
    bs = g["block_size"]
    phys = [5, 2, 9]
    table = np.array([phys], dtype=np.int32)
    got = [int(oracle.slot_mapping(table, np.array([t], np.int32), bs)[0]) for t in g["tokens"]]
    assert got == [20, 21, 22, 23, 8, 9, 10, 11, 36]


# --------------------------------------------------------------------------------
# O2: the cache write is a bit copy into exactly the target rows
# --------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cache_write_touches_only_target_rows(dtype):
    b = _small_gqa(dtype=dtype)
    kc0, vc0 = _np(b, b.key_cache), _np(b, b.value_cache)
    k, v = _np(b, b.key), _np(b, b.value)
    BS = b.spec.block_size
    slots = oracle.slot_mapping(b.block_tables, b.context_lens, BS)
    kc, vc = oracle.cache_write(kc0, vc0, k, v, slots, BS)
    # Brute force over every (block, row) of the pool, naming rows by block*BS+row.
    where = {int(s): t for t, s in enumerate(slots)}
    for blk in range(kc.shape[0]):
        for row in range(BS):
            flat = blk * BS + row
            for new, old, src in ((kc, kc0, k), (vc, vc0, v)):
                if flat in where:
                    assert new[blk, row].tobytes() == src[where[flat]].tobytes()
                else:
                    assert new[blk, row].tobytes() == old[blk, row].tobytes()


def test_cache_write_skips_negative_slots():
    b = _small_gqa()
    kc0, vc0 = _np(b, b.key_cache), _np(b, b.value_cache)
    slots = np.full(b.num_seqs, -1, dtype=np.int64)
    kc, vc = oracle.cache_write(kc0, vc0, _np(b, b.key), _np(b, b.value), slots, 16)
    assert kc.tobytes() == kc0.tobytes() and vc.tobytes() == vc0.tobytes()


# --------------------------------------------------------------------------------
# O3-O6: equality with a library routine on dense, unpaged K/V
# --------------------------------------------------------------------------------

def _dense_then_paged(ctx, Hkv, G, D, BS, NB, seed):
    """Dense per-sequence K/V, then placed into a pool by walking each table block."""
    rng = np.random.default_rng(seed)
    B = len(ctx)
    H = Hkv * G
    nblk = [-(-c // BS) for c in ctx]
    ids = rng.permutation(NB)[: sum(nblk)]
    tables = np.full((B, max(nblk)), -1, dtype=np.int32)
    kpool = np.full((NB, BS, Hkv, D), np.nan, dtype=np.float32)
    vpool = np.full((NB, BS, Hkv, D), np.nan, dtype=np.float32)
    dense_k, dense_v = [], []
    cur = 0
    for i, c in enumerate(ctx):
        K = rng.standard_normal((c, Hkv, D)).astype(np.float32)
        V = rng.standard_normal((c, Hkv, D)).astype(np.float32)
        dense_k.append(K)
        dense_v.append(V)
        for j in range(nblk[i]):
            b = int(ids[cur])
            cur += 1
            tables[i, j] = b
            rows = K[j * BS:(j + 1) * BS]
            kpool[b, :rows.shape[0]] = rows
            vpool[b, :rows.shape[0]] = V[j * BS:(j + 1) * BS]
    q = rng.standard_normal((B, H, D)).astype(np.float32)
    return q, kpool, vpool, tables, np.array(ctx, np.int32), dense_k, dense_v


@pytest.mark.parametrize("Hkv,G,D,BS", [(4, 1, 64, 16), (2, 4, 128, 16), (1, 8, 64, 32)])
def test_equals_torch_sdpa_on_dense_kv(Hkv, G, D, BS):
    ctx = [1, 5, 16, 33, 100, 257]
    q, kp, vp, bt, cl, dk, dv = _dense_then_paged(ctx, Hkv, G, D, BS, 128, seed=7)
    scale = 1.0 / math.sqrt(D)
    got = oracle.paged_attention_decode(q, kp, vp, bt, cl, scale, "f32")
    for i, c in enumerate(ctx):
        qt = torch.from_numpy(q[i]).double()[None, :, None, :]                  # [1,H,1,D]
        kt = torch.from_numpy(dk[i]).double().permute(1, 0, 2).repeat_interleave(G, 0)[None]
        vt = torch.from_numpy(dv[i]).double().permute(1, 0, 2).repeat_interleave(G, 0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        np.testing.assert_allclose(got[i], ref[0, :, 0, :].numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------------
# O3: physical placement does not matter
# --------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_permutation_invariance_bitwise(dtype):
    b = _small_gqa(dtype=dtype)
    perm = np.random.default_rng(3).permutation(b.spec.num_blocks)
    pb = permute_physical_blocks(b, perm)
    args = lambda x: (_np(x, x.query), _np(x, x.key), _np(x, x.value), _np(x, x.key_cache),
                      _np(x, x.value_cache), x.block_tables, x.context_lens, x.scale, dtype)
    _, _, _, out0 = oracle.decode_step(*args(b))
    _, _, _, out1 = oracle.decode_step(*args(pb))
    assert out0.tobytes() == out1.tobytes()
    assert np.isfinite(out0).all()


def test_prefix_sharing_equals_private_copies():
    from workloads import unshare_prefix_blocks
    spec = replace(CONFIGS["prefix_shared"], num_kv_heads=2, num_heads=8, head_dim=64,
                   num_blocks=1024)
    from workloads.decode_batches import draw_context_lens, deal_block_tables
    ctx = draw_context_lens(spec)[:8]
    spec = replace(spec, num_seqs=8)
    bt = deal_block_tables(spec, ctx)
    b = build_batch(spec, ctx, device="cpu", block_tables=bt)
    u = unshare_prefix_blocks(b)
    assert (b.block_tables[0, :64] == b.block_tables[1, :64]).all()
    assert not np.intersect1d(u.block_tables[0, :64], u.block_tables[1, :64]).size
    args = lambda x: (_np(x, x.query), _np(x, x.key), _np(x, x.value), _np(x, x.key_cache),
                      _np(x, x.value_cache), x.block_tables, x.context_lens, x.scale, "bf16")
    assert oracle.decode_step(*args(b))[3].tobytes() == oracle.decode_step(*args(u))[3].tobytes()


# --------------------------------------------------------------------------------
# brute force on the tiny workload
# --------------------------------------------------------------------------------

def test_brute_force_tiny():
    b = make_config("tiny")
    q, k, v = _np(b, b.query), _np(b, b.key), _np(b, b.value)
    kc, vc = _np(b, b.key_cache), _np(b, b.value_cache)
    slots, kc2, vc2, out = oracle.decode_step(q, k, v, kc, vc, b.block_tables, b.context_lens,
                                              b.scale, "f32")
    BS = b.spec.block_size
    H, D = q.shape[1], q.shape[2]
    for i in range(b.num_seqs):
        ctx = int(b.context_lens[i])
        # the context: history rows from the pool, new token from the inputs
        rows_k, rows_v = [], []
        for t in range(ctx):
            if t == ctx - 1:
                rows_k.append(k[i]); rows_v.append(v[i])
            else:
                blk = int(b.block_tables[i][t // BS])
                rows_k.append(kc[blk, t % BS]); rows_v.append(vc[blk, t % BS])
        for h in range(H):
            s = [b.scale * math.fsum(float(q[i, h, d]) * float(rk[h, d]) for d in range(D))
                 for rk in rows_k]
            m = max(s)
            p = [math.exp(x - m) for x in s]
            l = math.fsum(p)
            for d in range(0, D, 7):
                ref = math.fsum(p[t] * float(rows_v[t][h, d]) for t in range(ctx)) / l
                assert abs(out[i, h, d] - ref) <= 1e-12


# --------------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------------

def test_context_of_one_returns_new_value_exactly():
    b = _small_gqa(ctx=(1, 1, 1), dtype="bf16")
    _, _, _, out = oracle.decode_step(_np(b, b.query), _np(b, b.key), _np(b, b.value),
                                      _np(b, b.key_cache), _np(b, b.value_cache),
                                      b.block_tables, b.context_lens, b.scale, "bf16")
    G = b.spec.num_heads // b.spec.num_kv_heads
    v = oracle.to_f64(_np(b, b.value), "bf16")
    for h in range(b.spec.num_heads):
        assert (out[:, h] == v[:, h // G]).all()


def test_zero_query_and_equal_keys_give_mean_value():
    q, kp, vp, bt, cl, dk, dv = _dense_then_paged([37, 64], 2, 4, 64, 16, 32, seed=5)
    q0 = np.zeros_like(q)
    out = oracle.paged_attention_decode(q0, kp, vp, bt, cl, 0.125, "f32")
    for i in range(2):
        mean = dv[i].astype(np.float64).mean(axis=0)          # [Hkv, D]
        np.testing.assert_allclose(out[i], np.repeat(mean, 4, axis=0), rtol=0, atol=1e-14)
    # equal keys: any query
    one_key = np.broadcast_to(kp[bt[0, 0], 0][None, None], kp.shape)
    kp_eq = np.where(np.isfinite(kp), one_key, kp)
    out = oracle.paged_attention_decode(q, kp_eq, vp, bt, cl, 0.125, "f32")
    mean = dv[0].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(out[0], np.repeat(mean, 4, axis=0), rtol=0, atol=1e-14)


def test_dominant_key_selects_its_value_without_overflow():
    # One key scores 2000 above the rest: exp without subtracting the maximum would
    # overflow to inf/inf; the stable softmax gives that key's value.
    q, kp, vp, bt, cl, dk, dv = _dense_then_paged([50], 1, 1, 64, 16, 8, seed=9)
    q[:] = 0.0
    q[0, 0, 0] = 1.0
    kp[np.isfinite(kp)] = 0.0
    b, r = int(bt[0, 1]), 3                                  # token 19
    kp[b, r, 0, 0] = 2000.0
    out = oracle.paged_attention_decode(q, kp, vp, bt, cl, 1.0, "f32")
    np.testing.assert_array_equal(out[0, 0], vp[b, r, 0].astype(np.float64))


# --------------------------------------------------------------------------------
# O7: the partition merge equals the single softmax
# --------------------------------------------------------------------------------

@pytest.mark.parametrize("psize", [16, 48, 64, 512])
def test_partition_merge_identity(psize):
    ctx = [1, 16, 17, 100, 513, 1100]
    q, kp, vp, bt, cl, dk, dv = _dense_then_paged(ctx, 2, 4, 64, 16, 256, seed=21)
    full = oracle.paged_attention_decode(q, kp, vp, bt, cl, 0.125, "f32")
    part = oracle.partitioned_attention_decode(q, kp, vp, bt, cl, 0.125, "f32", psize)
    np.testing.assert_allclose(part, full, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------------
# storage decoding and byte accounting
# --------------------------------------------------------------------------------

def test_bf16_widening_matches_torch():
    bits = np.random.default_rng(0).integers(0, 1 << 16, size=200_000, dtype=np.uint32)
    bits = bits.astype(np.uint16)
    bits = bits[~(((bits & 0x7F80) == 0x7F80) & ((bits & 0x7F) != 0))]     # drop NaNs
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(bits), ref)
    assert oracle.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0000], np.uint16)).tolist() == \
        [1.0, -2.0, 0.0]


def test_kv_bytes_closed_form():
    g = json.load(open(os.path.join(GOLDEN, "kv_bytes_per_token.json")))
    spec = ConfigSpec("kvb", 1, g["heads"], g["heads"], g["head_dim"], 16, 4, "bf16", 2048,
                      ("fixed", (2048,)), 0)
    ctx = np.array([g["tokens_per_sequence"]], np.int32)
    per_layer = DecodeBatch(spec, ctx, None, None, None, None, None, None, 1.0).kv_bytes()
    assert per_layer * g["layers"] == g["bytes_per_sequence"]
    assert per_layer * g["layers"] // g["tokens_per_sequence"] == g["bytes_per_token_all_layers"]


# --------------------------------------------------------------------------------
# planted mistakes: a broken oracle must fail the pins above
# --------------------------------------------------------------------------------

def _sdpa_case():
    ctx = [3, 40, 70]
    q, kp, vp, bt, cl, dk, dv = _dense_then_paged(ctx, 2, 4, 64, 16, 64, seed=31)
    refs = []
    for i in range(len(ctx)):
        qt = torch.from_numpy(q[i]).double()[None, :, None, :]
        kt = torch.from_numpy(dk[i]).double().permute(1, 0, 2).repeat_interleave(4, 0)[None]
        vt = torch.from_numpy(dv[i]).double().permute(1, 0, 2).repeat_interleave(4, 0)[None]
        refs.append(torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, scale=0.125)[0, :, 0, :].numpy())
    return (q, kp, vp, bt, cl), np.stack(refs)


def _sdpa_ok(out, ref):
    return np.isfinite(out).all() and np.abs(out - ref).max() <= 1e-12


def test_planted_mistakes_fail_the_library_pin(monkeypatch):
    (q, kp, vp, bt, cl), ref = _sdpa_case()
    assert _sdpa_ok(oracle.paged_attention_decode(q, kp, vp, bt, cl, 0.125, "f32"), ref)

    import oracle.paged_decode as od
    good_attn, good_gather = od.softmax_attention, od.gather_context

    def no_scale(qv, K, V, scale):
        return good_attn(qv, K, V, 1.0)

    def off_by_one(cache, row, ctx, g, dt):
        return good_gather(cache, row, max(ctx - 1, 1), g, dt)

    def wrong_head(cache, row, ctx, g, dt):
        return good_gather(cache, row, ctx, cache.shape[2] - 1 - g, dt)

    def no_normalise(qv, K, V, scale):
        s = scale * (K @ qv)
        p = np.exp(s - s.max())
        return p @ V

    for name, fn in (("softmax_attention", no_scale), ("gather_context", off_by_one),
                     ("gather_context", wrong_head), ("softmax_attention", no_normalise)):
        with monkeypatch.context() as m:
            m.setattr(od, name, fn)
            out = od.paged_attention_decode(q, kp, vp, bt, cl, 0.125, "f32")
            assert not _sdpa_ok(out, ref), f"planted mistake in {name} went unnoticed"


def test_planted_slot_mistake_fails_worked_example(monkeypatch):
    import oracle.paged_decode as od
    g = json.load(open(os.path.join(GOLDEN, "slot_worked_example.json")))
    table = np.array([g["block_table"]], dtype=np.int32)
    monkeypatch.setattr(od, "token_place", lambda pos, bs: (pos // bs, (pos + 1) % bs))
    got = [int(od.slot_mapping(table, np.array([t], np.int32), 4)[0]) for t in g["tokens"]]
    assert got != g["slot"]


def test_planted_merge_mistake_fails_identity(monkeypatch):
    import oracle.paged_decode as od
    ctx = [100, 513]
    q, kp, vp, bt, cl, _, _ = _dense_then_paged(ctx, 1, 4, 64, 16, 64, seed=2)
    full = od.paged_attention_decode(q, kp, vp, bt, cl, 0.125, "f32")

    def bad_merge(stats):             # forgets the l_k factor in the weights
        M = max(m for m, _, _ in stats)
        w = [math.exp(m - M) for m, _, _ in stats]
        return sum(wi * o for wi, (_, _, o) in zip(w, stats)) / sum(w)

    monkeypatch.setattr(od, "merge_partitions", bad_merge)
    part = od.partitioned_attention_decode(q, kp, vp, bt, cl, 0.125, "f32", 64)
    assert np.abs(part - full).max() > 1e-6
