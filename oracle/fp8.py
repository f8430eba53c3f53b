"""CPU oracle of the FP8 KV cache: the E4M3 code, the quantised cache write and
attention over the dequantised cache.

TEST INFRASTRUCTURE.  Only the tests and the bench's CPU-baseline leg may import
this module.  It shares no code with the HIP path.

The pages name an FP8 KV cache only as a serving option (page "vLLM PagedAttention
原理与源码深度解析", section 8.4, `--kv-cache-dtype fp8`) and fix neither the format
nor the scaling.  Readings adopted:

  F1  Format: OCP 8-bit floating point E4M3 (sign, 4 exponent bits with bias 7, 3
      mantissa bits; no infinities; S.1111.111 is NaN; the largest finite magnitude is
      1.75 * 2^8 = 448; exponent field 0 holds the subnormals m * 2^-9).
  F2  Scaling: one fp32 scale per cache (k_scale, v_scale).  A value x is stored as
      E4M3(x / scale), the quotient taken in fp32 (correctly rounded), the precision
      the kernel divides in; the cache's real value is decode(code) * scale.
  F3  Encoding: round to nearest, ties to the even code; magnitudes past 448 saturate
      to +-448; NaN stays NaN (code 0x7F); the sign of zero is kept.
  F4  Attention reads decode(code) * scale exactly (in fp64 here) and is otherwise the
      attention of paged_decode (O3-O6).

Pins (tests/test_fp8.py): decode of all 256 codes and encode of finite values up to
464 against torch's float8_e4m3fn conversions (a library implementation of the same
format; past 464 torch returns NaN where F3 saturates); values the format fixes
(1 -> 0x38, 448 -> 0x7E, 2^-6 -> 0x08, 2^-9 -> 0x01, -2 -> 0xC0); every finite code's
value encodes back to the code; midpoints between neighbouring codes go to the even
one; saturation and NaN; the quantised write bit for bit; fp8 attention against
dense fp64 attention on the dequantised context.
"""

from __future__ import annotations

import math

import numpy as np

from .paged_decode import softmax_attention

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_decode(code: int) -> float:
    """F1: the real value of one code (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_DECODE = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_decode_array(codes: np.ndarray) -> np.ndarray:
    return _DECODE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: float) -> int:
    """F3: the code of the nearest representable value, ties to the even code;
    saturating at 448; NaN -> 0x7F."""
    x = float(x)
    if math.isnan(x):
        return E4M3_NAN
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    if a >= E4M3_MAX:
        return sign | 0x7E
    # the finite non-negative codes 0x00 .. 0x7E are in increasing value order
    lo, hi = 0, 0x7E
    while hi - lo > 1:                     # largest code with value <= a
        mid = (lo + hi) // 2
        if _DECODE[mid] <= a:
            lo = mid
        else:
            hi = mid
    if _DECODE[hi] <= a:
        lo = hi
    if lo == 0x7E:
        return sign | lo
    below, above = _DECODE[lo], _DECODE[lo + 1]
    if a - below < above - a:
        c = lo
    elif a - below > above - a:
        c = lo + 1
    else:
        c = lo if lo % 2 == 0 else lo + 1   # tie: the even code
    return sign | c


def e4m3_encode_array(x: np.ndarray) -> np.ndarray:
    flat = np.asarray(x, dtype=np.float64).reshape(-1)
    return np.array([e4m3_encode(v) for v in flat], dtype=np.uint8).reshape(np.shape(x))


def quantize(values: np.ndarray, scale: float) -> np.ndarray:
    """F2/F3: codes of values / scale; values and scale are fp32-representable (the
    cache write's inputs are bf16 or fp32), the quotient is rounded to fp32."""
    q = np.asarray(values, dtype=np.float32) / np.float32(scale)
    return e4m3_encode_array(q.astype(np.float64))


def cache_write_fp8(key_cache: np.ndarray, value_cache: np.ndarray, key: np.ndarray,
                    value: np.ndarray, slots: np.ndarray, block_size: int,
                    k_scale: float, v_scale: float):
    """O2 with F2/F3: copies of the uint8 caches with each token's quantised K/V rows at
    its slot (negative slots skipped).  ``key``/``value`` hold fp32-representable
    values (the widened bf16 or fp32 inputs)."""
    kc = key_cache.copy()
    vc = value_cache.copy()
    kq = quantize(key, k_scale)
    vq = quantize(value, v_scale)
    for t in range(slots.shape[0]):
        s = int(slots[t])
        if s < 0:
            continue
        kc[s // block_size, s % block_size] = kq[t]
        vc[s // block_size, s % block_size] = vq[t]
    return kc, vc


def paged_attention_decode_fp8(query: np.ndarray, key_cache: np.ndarray,
                               value_cache: np.ndarray, block_tables: np.ndarray,
                               context_lens: np.ndarray, scale: float, k_scale: float,
                               v_scale: float, seqs=None) -> np.ndarray:
    """F4: attention over decode(code) * scale.  ``query`` is real-valued [B, H, D]
    (fp64); caches are uint8 codes [NB, BS, Hkv, D].  Returns fp64 [len(seqs), H, D]."""
    B, H, D = query.shape
    Hkv = key_cache.shape[2]
    G = H // Hkv
    seqs = list(range(B)) if seqs is None else list(seqs)
    out = np.zeros((len(seqs), H, D))
    for r, i in enumerate(seqs):
        ctx = int(context_lens[i])
        for g in range(Hkv):
            K = e4m3_decode_array(_gather_codes(key_cache, block_tables[i], ctx, g)) * k_scale
            V = e4m3_decode_array(_gather_codes(value_cache, block_tables[i], ctx, g)) * v_scale
            for h in range(g * G, (g + 1) * G):
                out[r, h] = softmax_attention(np.asarray(query[i, h], np.float64), K, V, scale)
    return out


def _gather_codes(cache: np.ndarray, table_row: np.ndarray, ctx: int, kv_head: int) -> np.ndarray:
    """O3 on raw codes: the sequence's first ``ctx`` rows for one kv head."""
    block_size = cache.shape[1]
    nblk = -(-ctx // block_size)
    pieces = [cache[int(table_row[j]), :, kv_head, :] for j in range(nblk)]
    return np.concatenate(pieces, axis=0)[:ctx]
