"""Several new tokens per sequence (chunked prefill, verification of speculated
tokens): pins for the CPU oracle (each against something other than itself), and the
HIP path against the oracle (GPU)."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import multi_query as omq
from workloads import build_multi_batch, make_multi_config, permute_physical_blocks
from workloads.decode_batches import ConfigSpec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _spec(D=64, G=2, Hkv=2, BS=16, NB=128, dtype="f32", seed=3):
    return ConfigSpec("mq", 1, G * Hkv, Hkv, D, BS, NB, dtype, 1, ("fixed", (1,)), seed)


def _np(b, t):
    return b.numpy_storage(t)


def _run_oracle(b, **kw):
    qsl = b.extra["query_start_loc"]
    return omq.multi_query_step(_np(b, b.query), _np(b, b.key), _np(b, b.value),
                                _np(b, b.key_cache), _np(b, b.value_cache), b.block_tables,
                                b.context_lens, qsl, b.scale, b.kv_dtype, **kw)


def _dense(b, kc, vc, i, g, kv_dtype):
    ctx = int(b.context_lens[i])
    K = oracle.gather_context(kc, b.block_tables[i], ctx, g, kv_dtype)
    V = oracle.gather_context(vc, b.block_tables[i], ctx, g, kv_dtype)
    return K, V


# --------------------------------------------------------------------------------
# oracle pins (CPU)
# --------------------------------------------------------------------------------

def test_one_new_token_equals_the_decode_oracle_bitwise():
    ctx = [1, 16, 17, 40, 97]
    b = build_multi_batch(_spec(dtype="bf16", D=128, G=4), ctx, [1] * len(ctx))
    _, kc, vc, out = _run_oracle(b)
    _, kc2, vc2, ref = oracle.decode_step(_np(b, b.query), _np(b, b.key), _np(b, b.value),
                                          _np(b, b.key_cache), _np(b, b.value_cache),
                                          b.block_tables, b.context_lens, b.scale, "bf16")
    assert (kc == kc2).all() and (vc == vc2).all()
    assert (out == ref).all()


@pytest.mark.parametrize("G,Hkv,dtype", [(1, 4, "f32"), (4, 2, "bf16"), (8, 1, "bf16")])
def test_equals_torch_sdpa_with_a_causal_mask(G, Hkv, dtype):
    ctx = [5, 20, 33, 64]
    ql = [5, 3, 17, 1]
    b = build_multi_batch(_spec(G=G, Hkv=Hkv, dtype=dtype), ctx, ql)
    _, kc, vc, out = _run_oracle(b)
    qsl = b.extra["query_start_loc"]
    q64 = oracle.to_f64(_np(b, b.query), dtype)
    for i in range(len(ctx)):
        c, n = ctx[i], ql[i]
        # key t is visible to new token j when t <= c - n + j
        mask = torch.as_tensor(np.arange(c)[None, :] <= (c - n + np.arange(n))[:, None])
        for g in range(Hkv):
            K, V = _dense(b, kc, vc, i, g, dtype)
            q = torch.as_tensor(q64[qsl[i]:qsl[i + 1], g * G:(g + 1) * G]).permute(1, 0, 2)
            ref = torch.nn.functional.scaled_dot_product_attention(
                q, torch.as_tensor(K)[None].expand(G, -1, -1),
                torch.as_tensor(V)[None].expand(G, -1, -1), attn_mask=mask,
                scale=b.scale).permute(1, 0, 2).numpy()
            got = out[qsl[i]:qsl[i + 1], g * G:(g + 1) * G]
            assert np.abs(got - ref).max() < 1e-12


def test_brute_force_tiny():
    ctx, ql = [3, 6], [2, 4]
    b = build_multi_batch(_spec(D=4, G=2, Hkv=1, BS=2, NB=16), ctx, ql)
    _, kc, vc, out = _run_oracle(b)
    qsl = b.extra["query_start_loc"]
    q = _np(b, b.query).astype(np.float64)
    for i in range(2):
        for j in range(ql[i]):
            p = ctx[i] - ql[i] + j
            for h in range(2):
                s = []
                for t in range(p + 1):
                    blk = b.block_tables[i][t // 2]
                    s.append(sum(q[qsl[i] + j, h, d] * float(kc[blk, t % 2, 0, d])
                                 for d in range(4)) * b.scale)
                m = max(s)
                w = [np.exp(x - m) for x in s]
                for d in range(4):
                    num = sum(w[t] * float(vc[b.block_tables[i][t // 2], t % 2, 0, d])
                              for t in range(p + 1))
                    assert abs(out[qsl[i] + j, h, d] - num / sum(w)) < 1e-12


def test_block_relabelling_invariance_bitwise():
    b = build_multi_batch(_spec(dtype="bf16", NB=64), [7, 40, 90], [7, 5, 16])
    pb = permute_physical_blocks(b, np.random.default_rng(1).permutation(64))
    assert (_run_oracle(b)[3] == _run_oracle(pb)[3]).all()


def test_chunking_invariance():
    # a 40-token prompt in one step equals a 23-token chunk and then a 17-token chunk
    b = build_multi_batch(_spec(dtype="bf16", NB=32), [40], [40])
    qsl = b.extra["query_start_loc"]
    slots, kc, vc, whole = _run_oracle(b)
    st = lambda t: _np(b, t)  # noqa: E731
    s1, kc1, vc1, first = omq.multi_query_step(
        st(b.query)[:23], st(b.key)[:23], st(b.value)[:23], st(b.key_cache),
        st(b.value_cache), b.block_tables, np.array([23]), np.array([0, 23]), b.scale, "bf16")
    s2, kc2, vc2, second = omq.multi_query_step(
        st(b.query)[23:], st(b.key)[23:], st(b.value)[23:], kc1, vc1, b.block_tables,
        np.array([40]), np.array([0, 17]), b.scale, "bf16")
    assert (np.concatenate([s1, s2]) == slots).all()
    assert (kc2 == kc).all() and (vc2 == vc).all()
    assert (np.concatenate([first, second]) == whole).all()
    assert qsl.tolist() == [0, 40]


def test_worked_example_slots_for_a_chunk():
    # the pages' worked example (block size 4, tokens 1..9): one 9-token chunk gets the
    # nine slots of the example; a 4-token chunk after 5 tokens gets the last four
    g = json.load(open(os.path.join(GOLDEN, "slot_worked_example.json")))
    table = np.array([g["block_table"]], dtype=np.int32)
    s = omq.slot_mapping_multi(table, np.array([9]), np.array([0, 9]), g["block_size"])
    assert s.tolist() == g["slot"]
    s = omq.slot_mapping_multi(table, np.array([9]), np.array([0, 4]), g["block_size"])
    assert s.tolist() == g["slot"][5:]


def test_invalid_lengths_give_no_slots_and_nan_rows():
    b = build_multi_batch(_spec(NB=64), [10, 20, 30], [3, 4, 5])
    ctx = b.context_lens.copy()
    ctx[1] = 2                              # fewer tokens than new tokens
    qsl = b.extra["query_start_loc"]
    s = omq.slot_mapping_multi(b.block_tables, ctx, qsl, 16)
    assert (s[3:7] == -1).all() and (s[:3] >= 0).all() and (s[7:] >= 0).all()
    _, _, _, out = omq.multi_query_step(_np(b, b.query), _np(b, b.key), _np(b, b.value),
                                        _np(b, b.key_cache), _np(b, b.value_cache),
                                        b.block_tables, ctx, qsl, b.scale, "f32")
    assert np.isnan(out[3:7]).all()
    assert not np.isnan(out[:3]).any() and not np.isnan(out[7:]).any()


def test_planted_off_by_one_mask_fails_the_library_pin(monkeypatch):
    real = oracle.softmax_attention

    def strict(q, K, V, scale):          # drops the token's own key
        return real(q, K[:-1], V[:-1], scale) if K.shape[0] > 1 else real(q, K, V, scale)

    monkeypatch.setattr(omq, "softmax_attention", strict)
    with pytest.raises(AssertionError):
        test_equals_torch_sdpa_with_a_causal_mask(4, 2, "bf16")


def test_workloads_shapes():
    b = make_multi_config("tiny_multi")
    assert b.extra["query_start_loc"].tolist() == [0, 1, 6, 22, 62]
    assert (b.extra["query_lens"] <= b.context_lens).all()
    c = make_multi_config("chunked_prefill")
    assert int(c.extra["query_start_loc"][-1]) == 2048
