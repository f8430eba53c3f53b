"""FP8 (E4M3) KV cache: the oracle against the format and a library implementation
of it (CPU), and the HIP path against the oracle (GPU)."""

import math

import numpy as np
import pytest
import torch

from oracle import fp8 as of8


def _torch_decode(codes):
    return torch.as_tensor(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def _torch_encode(x):
    return torch.as_tensor(np.asarray(x, np.float64)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = of8.e4m3_decode_array(codes)
    ref = _torch_decode(codes)
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all() and nan.sum() == 2          # 0x7F and 0xFF
    assert (ours[~nan] == ref[~nan]).all()


def test_values_the_format_fixes():
    enc = of8.e4m3_encode
    assert (enc(1.0), enc(448.0), enc(2.0 ** -6), enc(2.0 ** -9), enc(-2.0)) == \
        (0x38, 0x7E, 0x08, 0x01, 0xC0)
    assert of8.e4m3_decode(0x7E) == 448.0 and math.isnan(of8.e4m3_decode(0x7F))
    assert enc(-0.0) == 0x80 and enc(0.0) == 0x00


def test_every_finite_code_round_trips():
    for c in range(256):
        v = of8.e4m3_decode(c)
        if not math.isnan(v):
            assert of8.e4m3_encode(v) == c


def test_midpoints_go_to_the_even_code():
    for c in range(0x7E):                   # neighbours c, c + 1 among non-negative codes
        mid = (of8.e4m3_decode(c) + of8.e4m3_decode(c + 1)) / 2
        want = c if c % 2 == 0 else c + 1
        assert of8.e4m3_encode(mid) == want
        assert of8.e4m3_encode(-mid) == 0x80 | want


def test_encode_matches_torch_up_to_464_and_saturates_beyond():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 1, 4000), rng.normal(0, 100, 4000),
                        rng.uniform(-464, 464, 2000), rng.normal(0, 2 ** -8, 2000)])
    assert (of8.e4m3_encode_array(x) == _torch_encode(x)).all()
    assert of8.e4m3_encode(1e6) == 0x7E and of8.e4m3_encode(-500.0) == 0xFE
    assert of8.e4m3_encode(float("nan")) == 0x7F


def test_quantised_write_is_bitwise():
    rng = np.random.default_rng(1)
    kc = rng.integers(0, 256, (6, 4, 2, 8), dtype=np.uint8)
    vc = rng.integers(0, 256, (6, 4, 2, 8), dtype=np.uint8)
    k = rng.normal(0, 3, (3, 2, 8)).astype(np.float32)
    v = rng.normal(0, 3, (3, 2, 8)).astype(np.float32)
    slots = np.array([5, -1, 22])
    k2, v2 = of8.cache_write_fp8(kc, vc, k, v, slots, 4, 0.5, 2.0)
    # the quotient is taken in fp32; scales 0.5 and 2 make it exact here
    assert (k2[1, 1] == of8.e4m3_encode_array(k[0].astype(np.float32) / 0.5)).all()
    assert (v2[5, 2] == of8.e4m3_encode_array(v[2].astype(np.float32) / 2.0)).all()
    changed = (k2 != kc).any(axis=(2, 3))
    assert set(zip(*np.nonzero(changed))) <= {(1, 1), (5, 2)}


def test_fp8_attention_equals_dense_attention_on_dequantised_values():
    rng = np.random.default_rng(2)
    B, H, Hkv, D, BS, NB = 3, 8, 2, 16, 4, 40
    kc = rng.integers(0, 0x7E, (NB, BS, Hkv, D), dtype=np.uint8) | \
        (rng.integers(0, 2, (NB, BS, Hkv, D), dtype=np.uint8) << 7)
    vc = rng.integers(0, 0x7E, (NB, BS, Hkv, D), dtype=np.uint8)
    ctx = np.array([1, 9, 30])
    tables = rng.permutation(NB)[:B * 8].reshape(B, 8).astype(np.int32)
    q = rng.normal(0, 1, (B, H, D))
    ks, vs, scale = 0.02, 0.5, 0.25
    out = of8.paged_attention_decode_fp8(q, kc, vc, tables, ctx, scale, ks, vs)
    for i in range(B):
        rows = [tables[i, t // BS] * BS + t % BS for t in range(ctx[i])]
        K = torch.as_tensor(_torch_decode(kc.reshape(NB * BS, Hkv, D)[rows]) * ks)
        V = torch.as_tensor(_torch_decode(vc.reshape(NB * BS, Hkv, D)[rows]) * vs)
        K = K.repeat_interleave(H // Hkv, dim=1).permute(1, 0, 2)
        V = V.repeat_interleave(H // Hkv, dim=1).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.as_tensor(q[i])[:, None, :], K, V, scale=scale)[:, 0, :].numpy()
        assert np.abs(out[i] - ref).max() < 1e-12


def test_planted_rounding_mistake_fails_the_pins(monkeypatch):
    # ties away from zero instead of to even: the midpoint pin must catch it
    orig = of8.e4m3_encode

    def half_up(x):
        c = orig(x)
        for d in (c - 1, c + 1):
            if 0 <= (d & 0x7F) <= 0x7E and (d & 0x80) == (c & 0x80):
                a, b = abs(of8.e4m3_decode(c)), abs(of8.e4m3_decode(d))
                if abs(abs(x) - a) == abs(abs(x) - b) and b > a:
                    return d
        return c

    monkeypatch.setattr(of8, "e4m3_encode", half_up)
    with pytest.raises(AssertionError):
        test_midpoints_go_to_the_even_code()


def test_quotient_is_rounded_to_fp32_before_encoding():
    # x / s rounds (in fp32) onto the midpoint 1.0625 of codes 0x38 and 0x39, which then
    # goes to the even code; the exact quotient lies above the midpoint (-> 0x39 in fp64)
    from fractions import Fraction
    s = np.float32(0.3)
    x = np.float32(0.31875002)
    assert Fraction(float(x)) / Fraction(float(s)) > Fraction(1.0625)
    assert x / s == np.float32(1.0625)
    assert of8.e4m3_encode(float(x) / float(s)) == 0x39
    assert of8.quantize(np.array([x]), s)[0] == 0x38


# ----------------------------------------------------------------------------
# GPU: the HIP path against the oracle
# ----------------------------------------------------------------------------

FP8_ATOL = 2e-3     # attention outputs, as for bf16 caches (decoding is exact on both sides)


def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import paged_kv_cache_441_amd as pkv
    pkv.load_library()
    return pkv


def _spec(D=128, G=4, Hkv=2, BS=16, NB=4096, seed=7):
    from workloads.decode_batches import ConfigSpec
    return ConfigSpec("custom_fp8", 1, G * Hkv, Hkv, D, BS, NB, "fp8", 1, ("fixed", (1,)), seed,
                      partition_size=-1)


def _bf16_f64(t):
    from oracle import bf16_bits_to_f64
    return bf16_bits_to_f64(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def _meta(b):
    return (torch.as_tensor(b.block_tables, device="cuda"),
            torch.as_tensor(b.context_lens, device="cuda"))


def _step(pkv, b, out_dtype=torch.float32, fused=False):
    """Slot mapping, E4M3 write (into copies) and attention; returns (slots, kc, vc, out)."""
    kc, vc = b.key_cache.clone(), b.value_cache.clone()
    bt, cl = _meta(b)
    ks, vs = b.extra["k_scale"], b.extra["v_scale"]
    NB, BS = kc.shape[:2]
    if fused:
        ws = pkv.alloc_workspace(b.query, bt, BS, pkv.PARTITION_BALANCED)
        slots = pkv.decode_prologue_fp8(bt, cl, b.key, b.value, kc, vc, ws, ks, vs)
        out, _ = pkv.paged_attention_partition_fp8(b.query, kc, vc, bt, cl, b.scale, ks, vs,
                                                   out_dtype=out_dtype, workspace=ws)
        pkv.paged_attention_reduce(out, cl, ws, BS, bt.shape[1], pkv.PARTITION_BALANCED)
    else:
        slots = pkv.slot_mapping(bt, cl, BS, NB)
        pkv.kv_cache_write_fp8(b.key, b.value, kc, vc, slots, ks, vs)
        out = pkv.paged_attention_decode_fp8(b.query, kc, vc, bt, cl, b.scale, ks, vs,
                                             out_dtype=out_dtype)
    torch.cuda.synchronize()
    return slots, kc, vc, out


def _oracle_step(b, seqs=None):
    """The oracle's write (on the pre-step caches) and attention for ``seqs``."""
    import oracle
    seqs = np.arange(b.num_seqs) if seqs is None else np.asarray(list(seqs))
    bt = b.block_tables[seqs]
    ids = np.unique(bt[bt >= 0])
    idx = torch.as_tensor(ids.astype(np.int64), device=b.key_cache.device)
    kc = b.key_cache.index_select(0, idx).cpu().numpy()
    vc = b.value_cache.index_select(0, idx).cpu().numpy()
    cbt = np.where(bt >= 0, np.searchsorted(ids, np.maximum(bt, 0)), -1).astype(np.int32)
    ctx = b.context_lens[seqs]
    BS = b.spec.block_size
    slots = oracle.slot_mapping(cbt, ctx, BS)
    ks, vs = b.extra["k_scale"], b.extra["v_scale"]
    kc, vc = of8.cache_write_fp8(kc, vc, _bf16_f64(b.key)[seqs], _bf16_f64(b.value)[seqs],
                                 slots, BS, ks, vs)
    return of8.paged_attention_decode_fp8(_bf16_f64(b.query)[seqs], kc, vc, cbt, ctx, b.scale,
                                          ks, vs)


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["tiny_fp8", "llama3_8b_fp8"])
def test_gpu_fp8_write_is_bitwise_and_touches_only_target_rows(name):
    import oracle
    from workloads import make_fp8_config
    pkv = _gpu()
    b = make_fp8_config(name, device="cuda")
    slots, kc, vc, _ = _step(pkv, b)
    want = oracle.slot_mapping(b.block_tables, b.context_lens, b.spec.block_size)
    assert (slots.cpu().numpy() == want).all()
    NB, BS, Hkv, D = kc.shape
    s = torch.as_tensor(want.astype(np.int64), device="cuda")
    for new, old, src, sc in ((kc, b.key_cache, b.key, b.extra["k_scale"]),
                              (vc, b.value_cache, b.value, b.extra["v_scale"])):
        n, o = new.reshape(NB * BS, -1), old.reshape(NB * BS, -1)
        changed = (n != o).any(dim=1).nonzero().flatten()
        assert set(changed.tolist()) <= set(want.tolist())
        got = n.index_select(0, s).cpu().numpy()
        ref = of8.quantize(_bf16_f64(src).reshape(len(want), -1), sc)
        assert (got == ref).all()


@pytest.mark.gpu
@pytest.mark.parametrize("in_dtype", [torch.float32, torch.bfloat16])
def test_gpu_fp8_write_edge_values(in_dtype):
    # ties between codes (after the fp32 quotient), subnormals, the saturation edge,
    # infinities, NaN, signed zeros
    pkv = _gpu()
    Hkv, D, BS, NB = 2, 64, 16, 8
    codes = np.arange(256, dtype=np.uint8)
    vals = of8.e4m3_decode_array(codes)
    fin = vals[np.isfinite(vals)]
    pos = np.sort(fin[fin >= 0])
    mids = (pos[:-1] + pos[1:]) / 2
    special = np.array([0.0, -0.0, 448.0, 449.0, 463.9, 464.0, 480.0, 1e9, np.inf, -np.inf,
                        np.nan, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, -(2.0 ** -10), 1e-30])
    x = np.concatenate([mids, -mids, fin, special])
    n_el = Hkv * D
    T = -(-x.size // n_el)
    x = np.concatenate([x, np.zeros(T * n_el - x.size)]).reshape(T, Hkv, D)
    for scale in (1.0, 0.3):
        xin = torch.as_tensor(x * scale, dtype=torch.float32).to(in_dtype).cuda()
        kc = torch.full((NB, BS, Hkv, D), 0x7F, dtype=torch.uint8, device="cuda")
        vc = kc.clone()
        slots = torch.arange(T, dtype=torch.int32, device="cuda") * 3
        pkv.kv_cache_write_fp8(xin, -xin, kc, vc, slots, scale, scale)
        torch.cuda.synchronize()
        src = xin.float().cpu().numpy().astype(np.float64)       # the values handed over
        for cache, sign in ((kc, 1), (vc, -1)):
            got = cache.reshape(NB * BS, -1)[slots.long()].cpu().numpy()
            ref = of8.quantize((sign * src).reshape(T, -1), scale)
            assert (got == ref).all(), np.argwhere(got != ref)[:5]


@pytest.mark.gpu
def test_gpu_every_code_decodes_as_the_format_says():
    # V: one-token contexts give out = decode(v) * v_scale exactly, for all 256 codes
    pkv = _gpu()
    Hkv, D, BS, NB = 2, 128, 16, 4
    kc = torch.zeros((NB, BS, Hkv, D), dtype=torch.uint8, device="cuda")
    vc = torch.arange(256, dtype=torch.uint8, device="cuda").reshape(1, 1, Hkv, D).repeat(
        NB, BS, 1, 1)
    q = torch.zeros((1, Hkv, D), dtype=torch.bfloat16, device="cuda")
    bt = torch.tensor([[2]], dtype=torch.int32, device="cuda")
    cl = torch.tensor([1], dtype=torch.int32, device="cuda")
    out = pkv.paged_attention_decode_fp8(q, kc, vc, bt, cl, 1.0, 1.0, 1.0)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1).astype(np.float64)
    ref = of8.e4m3_decode_array(np.arange(256, dtype=np.uint8))
    assert (np.isnan(got) == np.isnan(ref)).all()
    ok = ~np.isnan(ref)
    assert (got[ok] == ref[ok]).all()
    # K: token 0's key holds every finite code (the two NaN codes replaced by 0: a NaN
    # anywhere in a key row makes that row's score NaN, as 0 * NaN is NaN), token 1's
    # key is zero; one-hot queries pick one element, so p_0 = sigmoid(scale * k_scale *
    # decode(code)) with V rows 1 and 0
    krow = np.arange(256, dtype=np.uint8)
    krow[[0x7F, 0xFF]] = 0
    kc = torch.zeros((NB, BS, Hkv, D), dtype=torch.uint8, device="cuda")
    kc[2, 0] = torch.as_tensor(krow.reshape(Hkv, D), device="cuda")
    vc = torch.zeros((NB, BS, Hkv, D), dtype=torch.uint8, device="cuda")
    vc[2, 0] = 0x38                                   # 1.0
    B = D
    q = torch.zeros((B, Hkv, D), dtype=torch.bfloat16, device="cuda")
    q[torch.arange(B), :, torch.arange(B)] = 1.0
    bt = torch.full((B, 1), 2, dtype=torch.int32, device="cuda")
    cl = torch.full((B,), 2, dtype=torch.int32, device="cuda")
    scale = 10.0 / 448.0
    out = pkv.paged_attention_decode_fp8(q, kc, vc, bt, cl, scale, 1.0, 1.0)
    torch.cuda.synchronize()
    p0 = out.cpu().numpy()[:, :, 0].astype(np.float64)        # [element e, head]
    codes = krow.reshape(Hkv, D).T                             # [e, head]
    s = scale * of8.e4m3_decode_array(codes)
    ref = 1.0 / (1.0 + np.exp(-s))
    assert np.isfinite(p0).all()
    assert np.abs(p0 - ref).max() < 2e-6
    # a NaN code in a key row turns that head's output NaN, and only that head's
    for nan_code, head in ((0x7F, 0), (0xFF, 1)):
        kc2 = kc.clone()
        kc2[2, 0, head, 5] = nan_code
        out = pkv.paged_attention_decode_fp8(q[:1], kc2, vc, bt[:1], cl[:1], scale, 1.0, 1.0)
        torch.cuda.synchronize()
        o = out.cpu()
        assert torch.isnan(o[0, head]).all() and torch.isfinite(o[0, 1 - head]).all()


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["tiny_fp8", "llama3_8b_fp8", "long_ctx_fp8"])
def test_gpu_fp8_attention_matches_oracle(name):
    # every sequence of the workload
    from workloads import make_fp8_config
    pkv = _gpu()
    b = make_fp8_config(name, device="cuda")
    _, _, _, out = _step(pkv, b)
    ref = _oracle_step(b)
    g = out.cpu().numpy().astype(np.float64)
    assert ref.shape[0] == b.num_seqs
    err = float(np.abs(g - ref).max())
    print(f"{name}: max |gpu - oracle| = {err:.3e} over {b.num_seqs} sequences")
    assert np.isfinite(out.cpu().numpy()).all()
    assert err <= FP8_ATOL


FP8_BOUNDARY = [1, 15, 16, 17, 511, 512, 513, 1024, 8192]


@pytest.mark.gpu
@pytest.mark.parametrize("D,G,Hkv,BS", [(128, 4, 2, 16), (128, 8, 1, 32), (128, 1, 8, 16),
                                        (64, 2, 2, 16), (64, 8, 4, 32), (128, 2, 3, 16)])
def test_gpu_fp8_boundary_contexts(D, G, Hkv, BS):
    from workloads import build_fp8_batch
    pkv = _gpu()
    b = build_fp8_batch(_spec(D=D, G=G, Hkv=Hkv, BS=BS, NB=2048), FP8_BOUNDARY, device="cuda")
    _, _, _, out = _step(pkv, b)
    err = float(np.abs(out.cpu().numpy().astype(np.float64) - _oracle_step(b)).max())
    print(f"D={D} G={G} Hkv={Hkv} BS={BS}: max err {err:.3e}")
    assert err <= FP8_ATOL


@pytest.mark.gpu
@pytest.mark.parametrize("Hkv", [2, 8, 16])
def test_gpu_fp8_fused_prologue_fp32_inputs_equal_separate_write(Hkv):
    # fp32 new rows (bf16 values plus a small fp32 offset, so that the quotient's
    # rounding sees fp32 bits): the fused prologue's E4M3 codes equal the separate
    # write's bit for bit, for code rows of 256 B, 1 KiB and 2 KiB
    from workloads import build_fp8_batch
    pkv = _gpu()
    b = build_fp8_batch(_spec(D=128, G=4, Hkv=Hkv, BS=16, NB=2048), [1, 17, 600, 3000],
                        device="cuda")
    gen = torch.Generator(device="cpu").manual_seed(Hkv)
    k32 = b.key.float() + 1e-3 * torch.randn(b.key.shape, generator=gen).to("cuda")
    v32 = b.value.float() + 1e-3 * torch.randn(b.value.shape, generator=gen).to("cuda")
    bt, cl = _meta(b)
    ks, vs = b.extra["k_scale"], b.extra["v_scale"]
    NB, BS = b.key_cache.shape[:2]
    kc1, vc1 = b.key_cache.clone(), b.value_cache.clone()
    s1 = pkv.slot_mapping(bt, cl, BS, NB)
    pkv.kv_cache_write_fp8(k32, v32, kc1, vc1, s1, ks, vs)
    kc2, vc2 = b.key_cache.clone(), b.value_cache.clone()
    ws = pkv.alloc_workspace(b.query, bt, BS, pkv.PARTITION_BALANCED)
    s2 = pkv.decode_prologue_fp8(bt, cl, k32, v32, kc2, vc2, ws, ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2)
    # and the codes are the oracle's
    want_k = of8.quantize(k32.double().cpu().numpy(), ks)
    got_k = kc2.view(NB * BS, -1)[s1.long()].cpu().numpy().reshape(want_k.shape)
    assert (got_k == want_k).all()


@pytest.mark.gpu
def test_gpu_fp8_staged_and_fused_equal_decode_bitwise_and_bf16_output():
    from workloads import build_fp8_batch
    pkv = _gpu()
    b = build_fp8_batch(_spec(NB=2048), [3, 513, 2000, 5000, 1], device="cuda")
    s1, k1, v1, o1 = _step(pkv, b)
    s2, k2, v2, o2 = _step(pkv, b, fused=True)
    assert torch.equal(s1, s2) and torch.equal(k1, k2) and torch.equal(v1, v2)
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
    o3 = _step(pkv, b, out_dtype=torch.bfloat16)[3]
    assert torch.equal(o3.view(torch.int16), o1.to(torch.bfloat16).view(torch.int16))


@pytest.mark.gpu
def test_gpu_fp8_invalid_device_data_gives_nan_rows():
    from workloads import build_fp8_batch
    pkv = _gpu()
    b = build_fp8_batch(_spec(NB=1024), [20, 300, 40, 700], device="cuda")
    _, kc, vc, good = _step(pkv, b)
    bt, cl = _meta(b)
    bt[1, 3] = 5000
    cl[2] = 0
    out = pkv.paged_attention_decode_fp8(b.query, kc, vc, bt, cl, b.scale, b.extra["k_scale"],
                                         b.extra["v_scale"])
    torch.cuda.synchronize()
    o = out.cpu()
    assert torch.isnan(o[1]).all() and torch.isnan(o[2]).all()
    assert (o[[0, 3]] - good.cpu()[[0, 3]]).abs().max().item() <= 2e-5


@pytest.mark.gpu
def test_gpu_fp8_copy_blocks_is_a_bit_copy():
    pkv = _gpu()
    g = torch.Generator(device="cuda").manual_seed(3)
    kc = torch.randint(0, 256, (64, 16, 8, 128), generator=g, dtype=torch.int32,
                       device="cuda").to(torch.uint8)
    vc = torch.randint(0, 256, (64, 16, 8, 128), generator=g, dtype=torch.int32,
                       device="cuda").to(torch.uint8)
    k0, v0 = kc.clone(), vc.clone()
    pairs = torch.tensor([[3, 40], [7, 41], [63, 0]], dtype=torch.int32, device="cuda")
    pkv.copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    from oracle.block_pool import copy_blocks as ref_copy
    rk, rv = ref_copy(k0.cpu().numpy(), v0.cpu().numpy(), pairs.cpu().numpy())
    assert (kc.cpu().numpy() == rk).all() and (vc.cpu().numpy() == rv).all()


@pytest.mark.gpu
def test_gpu_fp8_prepared_step_equals_per_call_wrappers():
    from workloads import build_fp8_batch
    pkv = _gpu()
    b = build_fp8_batch(_spec(NB=2048), [3, 513, 2000, 5000, 2], device="cuda")
    s1, k1, v1, o1 = _step(pkv, b, fused=True)
    kc, vc = b.key_cache.clone(), b.value_cache.clone()
    bt, cl = _meta(b)
    ks, vs = b.extra["k_scale"], b.extra["v_scale"]
    ds = pkv.DecodeStep(b.query, b.key, b.value, kc, vc, bt, cl, b.scale, k_scale=ks, v_scale=vs)
    o2 = ds()
    torch.cuda.synchronize()
    assert torch.equal(s1, ds.slot_mapping) and torch.equal(k1, kc) and torch.equal(v1, vc)
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
    with pytest.raises(ValueError):
        pkv.DecodeStep(b.query, b.key, b.value, kc, vc, bt, cl, b.scale)
