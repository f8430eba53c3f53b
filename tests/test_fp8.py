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
