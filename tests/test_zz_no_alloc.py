"""The decode entry point that allocates nothing (pkv_paged_attention_decode_noalloc),
called through the C ABI, against pkv_paged_attention_decode with a caller workspace:
the same bits, on two calls in a row, the second with a smaller batch (the fixed
device buffer keeps the first call's contents, which must not matter)."""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_441_amd as pkv
from paged_kv_cache_441_amd import _lib
from workloads import build_batch
from workloads.decode_batches import ConfigSpec

pytestmark = pytest.mark.gpu

BAL = _lib.PKV_PARTITION_BALANCED


def _spec(NB):
    return ConfigSpec("noalloc", 1, 32, 8, 128, 16, NB, "bf16", 1, ("fixed", (1,)), 31)


def _written_caches(b, bt, cl):
    """The batch's caches with every sequence's new token written (its row is poison
    until then)."""
    kc, vc = b.key_cache.clone(), b.value_cache.clone()
    slots = pkv.slot_mapping(bt, cl, kc.shape[1], kc.shape[0])
    pkv.kv_cache_write(b.key, b.value, kc, vc, slots)
    return kc, vc


def _call_noalloc(lib, b, kc, vc, bt, cl, P, out):
    st = lib.pkv_paged_attention_decode_noalloc(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(b.query.data_ptr()),
        ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(vc.data_ptr()),
        ctypes.c_void_p(bt.data_ptr()), ctypes.c_void_p(cl.data_ptr()), b.num_seqs,
        b.spec.num_heads, b.spec.num_kv_heads, b.spec.head_dim, b.spec.block_size,
        bt.shape[1], kc.shape[0], float(b.scale), P, _lib.PKV_BF16, _lib.PKV_F32,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def _call_with_workspace(lib, b, kc, vc, bt, cl, P, out):
    n = lib.pkv_paged_attention_workspace_bytes(b.num_seqs, b.spec.num_heads, b.spec.head_dim,
                                                b.spec.block_size, bt.shape[1], P)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    st = lib.pkv_paged_attention_decode(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(b.query.data_ptr()),
        ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(vc.data_ptr()),
        ctypes.c_void_p(bt.data_ptr()), ctypes.c_void_p(cl.data_ptr()), b.num_seqs,
        b.spec.num_heads, b.spec.num_kv_heads, b.spec.head_dim, b.spec.block_size,
        bt.shape[1], kc.shape[0], float(b.scale), P, _lib.PKV_BF16, _lib.PKV_F32,
        ctypes.c_void_p(ws.data_ptr()), n, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, ws


@pytest.mark.parametrize("P", [BAL, 0, 128])
def test_noalloc_equals_decode_on_two_calls(P):
    assert torch.cuda.is_available()
    lib = _lib.load_library()
    rng = np.random.default_rng(100 + P)
    big = rng.integers(1, 6000, size=48)
    big[:4] = [1, 16, 17, 8192]
    small = rng.integers(1, 900, size=7)
    for ctx in (big, small):                     # second call: a smaller batch
        b = build_batch(_spec(NB=int(np.ceil(ctx / 16).sum()) + 64), ctx, device="cuda")
        bt = torch.as_tensor(b.block_tables, device="cuda")
        cl = torch.as_tensor(b.context_lens, device="cuda")
        kc, vc = _written_caches(b, bt, cl)
        want = torch.empty_like(b.query, dtype=torch.float32)
        got = torch.full_like(want, float("nan"))
        st, ws = _call_with_workspace(lib, b, kc, vc, bt, cl, P, want)
        assert st == _lib.PKV_OK
        assert _call_noalloc(lib, b, kc, vc, bt, cl, P, got) == _lib.PKV_OK
        torch.cuda.synchronize()
        assert torch.isfinite(got).all()
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), \
            f"P={P} B={b.num_seqs}: max diff {(got - want).abs().max().item():.3e}"


def test_noalloc_binding_and_limit():
    lib = _lib.load_library()
    b = build_batch(_spec(NB=512), [5, 300, 1200], device="cuda")
    bt = torch.as_tensor(b.block_tables, device="cuda")
    cl = torch.as_tensor(b.context_lens, device="cuda")
    kc, vc = _written_caches(b, bt, cl)
    want = pkv.paged_attention_decode(b.query, kc, vc, bt, cl, b.scale, BAL)
    got = pkv.paged_attention_decode_noalloc(b.query, kc, vc, bt, cl, b.scale, BAL)
    torch.cuda.synchronize()
    assert torch.isfinite(got).all()
    assert torch.equal(got.view(torch.int32), want.view(torch.int32))
    # a batch whose workspace would exceed the fixed buffer is refused before any work
    assert lib.pkv_paged_attention_workspace_bytes(
        4096, 32, 128, 16, 512, BAL) > _lib.PKV_NOALLOC_SCRATCH_BYTES
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    st = lib.pkv_paged_attention_decode_noalloc(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(out.data_ptr()), 4096, 32, 8, 128, 16,
        512, 1024, 0.088, BAL, _lib.PKV_BF16, _lib.PKV_F32, ctypes.c_void_p(0))
    assert st == _lib.PKV_ERR_SCRATCH_LIMIT
