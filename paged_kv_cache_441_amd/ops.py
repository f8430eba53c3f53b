"""Torch-facing wrappers over the libpagedkv C ABI.

Argument marshalling only: each function checks dtype, device and contiguity,
passes raw device pointers, sizes and the current HIP stream of the tensors'
device, and raises ``PkvError`` on a non-OK status.  All computation happens in
the library's kernels; tensors must already live on the GPU.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from . import _lib

_KV_DTYPES = {torch.float32: _lib.PKV_F32, torch.bfloat16: _lib.PKV_BF16}
# partition_size: 0 = fixed partitions of 512 tokens; PARTITION_BALANCED = the balanced
# split (equal shares of the batch's tile list per workgroup)
PARTITION_DEFAULT = _lib.PKV_PARTITION_DEFAULT
PARTITION_BALANCED = _lib.PKV_PARTITION_BALANCED
# E4M3 caches hold raw codes: uint8, or torch's float8_e4m3fn (the same format)
_FP8_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def _dev(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _i32(t: torch.Tensor, name: str) -> None:
    _dev(t, name)
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32 (got {t.dtype})")


def _kv(t: torch.Tensor, name: str) -> int:
    _dev(t, name)
    if t.dtype not in _KV_DTYPES:
        raise TypeError(f"{name} must be float32 or bfloat16 (got {t.dtype})")
    return _KV_DTYPES[t.dtype]


def _fp8(t: torch.Tensor, name: str) -> None:
    _dev(t, name)
    if t.dtype not in _FP8_DTYPES:
        raise TypeError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn; got {t.dtype})")


def _storage(t: torch.Tensor, name: str) -> int:
    """Cache element type for bit copies: float32, bfloat16 or E4M3 codes."""
    if isinstance(t, torch.Tensor) and t.dtype in _FP8_DTYPES:
        _dev(t, name)
        return _lib.PKV_FP8_E4M3
    return _kv(t, name)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {devs}")


def slot_mapping(block_tables: torch.Tensor, context_lens: torch.Tensor, block_size: int,
                 num_blocks: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Slot of each sequence's new token (position context_len - 1); -1 if invalid."""
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    B = context_lens.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=context_lens.device)
    _i32(out, "out")
    _same_device(block_tables, context_lens, out)
    lib = _lib.load_library()
    st = lib.pkv_slot_mapping(_ptr(block_tables), _ptr(context_lens), _ptr(out), B,
                              block_tables.shape[1], int(block_size), int(num_blocks),
                              _stream(out))
    _lib.check(st, "pkv_slot_mapping")
    return out


def kv_cache_write(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                   value_cache: torch.Tensor, slot_mapping: torch.Tensor) -> None:
    """reshape_and_cache: copy each token's K/V row into its slot of the paged caches."""
    dt = _kv(key, "key")
    for t, n in ((value, "value"), (key_cache, "key_cache"), (value_cache, "value_cache")):
        if _kv(t, n) != dt:
            raise TypeError(f"{n} dtype differs from key")
    _i32(slot_mapping, "slot_mapping")
    _same_device(key, value, key_cache, value_cache, slot_mapping)
    if key_cache.dim() != 4 or value_cache.shape != key_cache.shape:
        raise ValueError("caches must both be [num_blocks, block_size, num_kv_heads, head_dim]")
    NB, BS, Hkv, D = key_cache.shape
    T = slot_mapping.shape[0]
    if key.shape != (T, Hkv, D) or value.shape != (T, Hkv, D):
        raise ValueError(f"key/value must be [{T}, {Hkv}, {D}]")
    lib = _lib.load_library()
    st = lib.pkv_kv_cache_write(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                _ptr(slot_mapping), T, Hkv, D, BS, NB, dt, _stream(key))
    _lib.check(st, "pkv_kv_cache_write")


def _call(name: str, args) -> None:
    _lib.check(getattr(_lib.load_library(), name)(*args), name)


def _prologue_args(block_tables, context_lens, key, value, key_cache, value_cache, workspace,
                   partition_size, slot_mapping, stream):
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    dt = _kv(key, "key")
    for t, n in ((value, "value"), (key_cache, "key_cache"), (value_cache, "value_cache")):
        if _kv(t, n) != dt:
            raise TypeError(f"{n} dtype differs from key")
    _dev(workspace, "workspace")
    B = context_lens.shape[0]
    if key_cache.dim() != 4 or value_cache.shape != key_cache.shape:
        raise ValueError("caches must both be [num_blocks, block_size, num_kv_heads, head_dim]")
    NB, BS, Hkv, D = key_cache.shape
    if key.shape != (B, Hkv, D) or value.shape != (B, Hkv, D):
        raise ValueError(f"key/value must be [{B}, {Hkv}, {D}]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    if slot_mapping is None:
        slot_mapping = torch.empty(B, dtype=torch.int32, device=key.device)
    _i32(slot_mapping, "slot_mapping")
    _same_device(block_tables, context_lens, key, value, key_cache, value_cache, workspace,
                 slot_mapping)
    args = (_ptr(block_tables), _ptr(context_lens), _ptr(key), _ptr(value), _ptr(key_cache),
            _ptr(value_cache), _ptr(slot_mapping), B, block_tables.shape[1], Hkv, D, BS, NB, dt,
            int(partition_size), _ptr(workspace), workspace.numel() * workspace.element_size(),
            stream if stream is not None else _stream(key))
    return "pkv_decode_prologue", args, slot_mapping


def decode_prologue(block_tables: torch.Tensor, context_lens: torch.Tensor, key: torch.Tensor,
                    value: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                    workspace: torch.Tensor, partition_size: int = 0,
                    slot_mapping: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Slot mapping + cache write + attention plan in one launch; returns the slots."""
    name, args, slot_mapping = _prologue_args(block_tables, context_lens, key, value, key_cache,
                                              value_cache, workspace, partition_size,
                                              slot_mapping, None)
    _call(name, args)
    return slot_mapping


def workspace_bytes(num_seqs: int, num_heads: int, head_dim: int, block_size: int,
                    max_blocks_per_seq: int, partition_size: int = 0) -> int:
    return int(_lib.load_library().pkv_paged_attention_workspace_bytes(
        num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq, partition_size))


def alloc_workspace(query: torch.Tensor, block_tables: torch.Tensor, block_size: int,
                    partition_size: int = 0) -> torch.Tensor:
    B, H, D = query.shape
    n = workspace_bytes(B, H, D, block_size, block_tables.shape[1], partition_size)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=query.device)


def _attention_args(query, key_cache, value_cache, block_tables, context_lens, out, out_dtype,
                    workspace, partition_size):
    dt = _kv(query, "query")
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache")):
        if _kv(t, n) != dt:
            raise TypeError(f"{n} dtype differs from query")
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    if query.dim() != 3 or key_cache.dim() != 4 or value_cache.shape != key_cache.shape:
        raise ValueError("query [B, H, D]; caches [NB, BS, Hkv, D]")
    B, H, D = query.shape
    NB, BS, Hkv, Dk = key_cache.shape
    if Dk != D or context_lens.shape != (B,) or block_tables.dim() != 2 or \
            block_tables.shape[0] != B:
        raise ValueError("inconsistent shapes")
    if out is None:
        out = torch.empty((B, H, D), dtype=out_dtype, device=query.device)
    if out.dtype not in _KV_DTYPES or out.shape != (B, H, D):
        raise ValueError("out must be float32/bfloat16 [B, H, D]")
    _dev(out, "out")
    if workspace is None:
        workspace = alloc_workspace(query, block_tables, BS, partition_size)
    _dev(workspace, "workspace")
    _same_device(query, key_cache, value_cache, block_tables, context_lens, out, workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    return (dt, out, workspace, ws_bytes, B, H, Hkv, D, BS, NB)


def paged_attention_decode(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                           partition_size: int = 0, out: Optional[torch.Tensor] = None,
                           out_dtype: torch.dtype = torch.float32,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode attention of one query per sequence over its paged context."""
    dt, out, ws, wsb, B, H, Hkv, D, BS, NB = _attention_args(
        query, key_cache, value_cache, block_tables, context_lens, out, out_dtype, workspace,
        partition_size)
    lib = _lib.load_library()
    st = lib.pkv_paged_attention_decode(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), B, H, Hkv, D, BS, block_tables.shape[1], NB, float(scale),
        int(partition_size), dt, _KV_DTYPES[out.dtype], _ptr(ws), wsb, _stream(query))
    _lib.check(st, "pkv_paged_attention_decode")
    return out


def paged_attention_decode_noalloc(query: torch.Tensor, key_cache: torch.Tensor,
                                   value_cache: torch.Tensor, block_tables: torch.Tensor,
                                   context_lens: torch.Tensor, scale: float,
                                   partition_size: int = 0,
                                   out: Optional[torch.Tensor] = None,
                                   out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """paged_attention_decode with its workspace in the library's fixed device buffer
    (pkv_paged_attention_decode_noalloc): the library allocates nothing.  Calls that
    overlap on one GPU race for that buffer."""
    dt = _kv(query, "query")
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache")):
        if _kv(t, n) != dt:
            raise TypeError(f"{n} dtype differs from query")
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    if query.dim() != 3 or key_cache.dim() != 4 or value_cache.shape != key_cache.shape:
        raise ValueError("query [B, H, D]; caches [NB, BS, Hkv, D]")
    B, H, D = query.shape
    NB, BS, Hkv, Dk = key_cache.shape
    if Dk != D or context_lens.shape != (B,) or block_tables.dim() != 2 or \
            block_tables.shape[0] != B:
        raise ValueError("inconsistent shapes")
    if out is None:
        out = torch.empty((B, H, D), dtype=out_dtype, device=query.device)
    if out.dtype not in _KV_DTYPES or out.shape != (B, H, D):
        raise ValueError("out must be float32/bfloat16 [B, H, D]")
    _dev(out, "out")
    _same_device(query, key_cache, value_cache, block_tables, context_lens, out)
    lib = _lib.load_library()
    st = lib.pkv_paged_attention_decode_noalloc(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), B, H, Hkv, D, BS, block_tables.shape[1], NB, float(scale),
        int(partition_size), dt, _KV_DTYPES[out.dtype], _stream(query))
    _lib.check(st, "pkv_paged_attention_decode_noalloc")
    return out


def paged_attention_decode_per_head(query: torch.Tensor, key_cache: torch.Tensor,
                                    value_cache: torch.Tensor, block_tables: torch.Tensor,
                                    context_lens: torch.Tensor, scale: float,
                                    partition_size: int = 0, out: Optional[torch.Tensor] = None,
                                    out_dtype: torch.dtype = torch.float32,
                                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """paged_attention_decode with fixed partitions in the per-head layout (for batches
    whose sequences share prefix blocks)."""
    dt, out, ws, wsb, B, H, Hkv, D, BS, NB = _attention_args(
        query, key_cache, value_cache, block_tables, context_lens, out, out_dtype, workspace,
        partition_size)
    lib = _lib.load_library()
    st = lib.pkv_paged_attention_decode_per_head(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), B, H, Hkv, D, BS, block_tables.shape[1], NB, float(scale),
        int(partition_size), dt, _KV_DTYPES[out.dtype], _ptr(ws), wsb, _stream(query))
    _lib.check(st, "pkv_paged_attention_decode_per_head")
    return out


def paged_attention_plan(context_lens: torch.Tensor, workspace: torch.Tensor, block_size: int,
                         max_blocks_per_seq: int, partition_size: int = 0) -> torch.Tensor:
    """Stage 1 of paged_attention_decode: the work list, written into ``workspace``."""
    _i32(context_lens, "context_lens")
    _dev(workspace, "workspace")
    _same_device(context_lens, workspace)
    lib = _lib.load_library()
    st = lib.pkv_paged_attention_plan(_ptr(context_lens), context_lens.shape[0], int(block_size),
                                      int(max_blocks_per_seq), int(partition_size),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(workspace))
    _lib.check(st, "pkv_paged_attention_plan")
    return workspace


def _partition_args(query, key_cache, value_cache, block_tables, context_lens, scale,
                    partition_size, out, out_dtype, workspace, stream, per_head=False):
    dt, out, ws, wsb, B, H, Hkv, D, BS, NB = _attention_args(
        query, key_cache, value_cache, block_tables, context_lens, out, out_dtype, workspace,
        partition_size)
    args = (_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
            _ptr(context_lens), B, H, Hkv, D, BS, block_tables.shape[1], NB, float(scale),
            int(partition_size), dt, _KV_DTYPES[out.dtype], _ptr(ws), wsb,
            stream if stream is not None else _stream(query))
    name = "pkv_paged_attention_partition" + ("_per_head" if per_head else "")
    return name, args, out, ws


def paged_attention_partition(query, key_cache, value_cache, block_tables, context_lens, scale,
                              partition_size=0, out=None, out_dtype=torch.float32, workspace=None):
    """Stage 2 of paged_attention_decode (needs a plan in ``workspace``); returns (out, workspace)."""
    name, args, out, ws = _partition_args(query, key_cache, value_cache, block_tables,
                                          context_lens, scale, partition_size, out, out_dtype,
                                          workspace, None)
    _call(name, args)
    return out, ws


def paged_attention_partition_per_head(query, key_cache, value_cache, block_tables, context_lens,
                                       scale, partition_size=0, out=None, out_dtype=torch.float32,
                                       workspace=None):
    """Stage 2 in the per-head layout of fixed partitions; returns (out, workspace)."""
    name, args, out, ws = _partition_args(query, key_cache, value_cache, block_tables,
                                          context_lens, scale, partition_size, out, out_dtype,
                                          workspace, None, per_head=True)
    _call(name, args)
    return out, ws


def _reduce_args(out, context_lens, workspace, block_size, max_blocks_per_seq, partition_size,
                 stream):
    _dev(out, "out")
    _i32(context_lens, "context_lens")
    _dev(workspace, "workspace")
    if out.dtype not in _KV_DTYPES:
        raise TypeError("out must be float32 or bfloat16")
    _same_device(out, context_lens, workspace)
    B, H, D = out.shape
    args = (_ptr(out), _ptr(context_lens), B, H, D, int(block_size), int(max_blocks_per_seq),
            int(partition_size), _KV_DTYPES[out.dtype], _ptr(workspace),
            workspace.numel() * workspace.element_size(),
            stream if stream is not None else _stream(out))
    return "pkv_paged_attention_reduce", args


def paged_attention_reduce(out: torch.Tensor, context_lens: torch.Tensor, workspace: torch.Tensor,
                           block_size: int, max_blocks_per_seq: int,
                           partition_size: int = 0) -> torch.Tensor:
    """Stage 3 of paged_attention_decode: merge the partition records into ``out``."""
    _call(*_reduce_args(out, context_lens, workspace, block_size, max_blocks_per_seq,
                        partition_size, None))
    return out


def decode_step(query, key, value, key_cache, value_cache, block_tables, context_lens, scale,
                partition_size=0, out=None, out_dtype=torch.float32, workspace=None,
                slots=None, per_head=False):
    """One decode step on the GPU: slot mapping, cache write, paged attention."""
    NB, BS = key_cache.shape[0], key_cache.shape[1]
    slots = slot_mapping(block_tables, context_lens, BS, NB, out=slots)
    kv_cache_write(key, value, key_cache, value_cache, slots)
    attend = paged_attention_decode_per_head if per_head else paged_attention_decode
    return attend(query, key_cache, value_cache, block_tables, context_lens, scale,
                  partition_size, out=out, out_dtype=out_dtype, workspace=workspace)


# ---- steps with several new tokens per sequence ---------------------------------------

def slot_mapping_multi_query(block_tables: torch.Tensor, context_lens: torch.Tensor,
                             query_start_loc: torch.Tensor, num_tokens: int, block_size: int,
                             num_blocks: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Slot of every new token of the flat batch (-1 where the sequence does not fit)."""
    for t, n in ((block_tables, "block_tables"), (context_lens, "context_lens"),
                 (query_start_loc, "query_start_loc")):
        _i32(t, n)
    B = context_lens.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != B or query_start_loc.shape != (B + 1,):
        raise ValueError("block_tables [B, MB], context_lens [B], query_start_loc [B + 1]")
    if out is None:
        out = torch.empty(int(num_tokens), dtype=torch.int32, device=context_lens.device)
    _i32(out, "out")
    _same_device(block_tables, context_lens, query_start_loc, out)
    lib = _lib.load_library()
    st = lib.pkv_slot_mapping_multi_query(_ptr(block_tables), _ptr(context_lens),
                                          _ptr(query_start_loc), _ptr(out), B, int(num_tokens),
                                          block_tables.shape[1], int(block_size), int(num_blocks),
                                          _stream(out))
    _lib.check(st, "pkv_slot_mapping_multi_query")
    return out


def multi_query_workspace_bytes(num_seqs: int, num_tokens: int, num_heads: int,
                                num_kv_heads: int, head_dim: int, block_size: int,
                                max_blocks_per_seq: int) -> int:
    return int(_lib.load_library().pkv_paged_attention_multi_query_workspace_bytes(
        num_seqs, num_tokens, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq))


def paged_attention_multi_query(query: torch.Tensor, key_cache: torch.Tensor,
                                value_cache: torch.Tensor, block_tables: torch.Tensor,
                                context_lens: torch.Tensor, query_start_loc: torch.Tensor,
                                scale: float, out: Optional[torch.Tensor] = None,
                                out_dtype: torch.dtype = torch.float32,
                                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal attention of every new token of the flat batch over its sequence's paged
    context (the new tokens' rows already written)."""
    dt = _kv(query, "query")
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache")):
        if _kv(t, n) != dt:
            raise TypeError(f"{n} dtype differs from query")
    for t, n in ((block_tables, "block_tables"), (context_lens, "context_lens"),
                 (query_start_loc, "query_start_loc")):
        _i32(t, n)
    if query.dim() != 3 or key_cache.dim() != 4 or value_cache.shape != key_cache.shape:
        raise ValueError("query [T, H, D]; caches [NB, BS, Hkv, D]")
    T, H, D = query.shape
    NB, BS, Hkv, Dk = key_cache.shape
    B = context_lens.shape[0]
    if Dk != D or block_tables.dim() != 2 or block_tables.shape[0] != B or \
            query_start_loc.shape != (B + 1,):
        raise ValueError("inconsistent shapes")
    if out is None:
        out = torch.empty((T, H, D), dtype=out_dtype, device=query.device)
    if out.dtype not in _KV_DTYPES or out.shape != (T, H, D):
        raise ValueError("out must be float32/bfloat16 [T, H, D]")
    _dev(out, "out")
    if workspace is None:
        n = multi_query_workspace_bytes(B, T, H, Hkv, D, BS, block_tables.shape[1])
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=query.device)
    _dev(workspace, "workspace")
    _same_device(query, key_cache, value_cache, block_tables, context_lens, query_start_loc, out,
                 workspace)
    lib = _lib.load_library()
    st = lib.pkv_paged_attention_multi_query(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(query_start_loc), B, T, H, Hkv, D, BS, block_tables.shape[1], NB,
        float(scale), dt, _KV_DTYPES[out.dtype], _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(query))
    _lib.check(st, "pkv_paged_attention_multi_query")
    return out


# ---- E4M3 (FP8) caches ---------------------------------------------------------------

def _fp8_caches(key_cache, value_cache):
    _fp8(key_cache, "key_cache")
    _fp8(value_cache, "value_cache")
    if key_cache.dim() != 4 or value_cache.shape != key_cache.shape:
        raise ValueError("caches must both be [num_blocks, block_size, num_kv_heads, head_dim]")
    return key_cache.shape


def kv_cache_write_fp8(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                       value_cache: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float,
                       v_scale: float) -> None:
    """reshape_and_cache into E4M3 caches: each token's rows divided by the cache's
    scale, rounded to E4M3 (ties to even, saturating at 448)."""
    dt = _kv(key, "key")
    if _kv(value, "value") != dt:
        raise TypeError("value dtype differs from key")
    NB, BS, Hkv, D = _fp8_caches(key_cache, value_cache)
    _i32(slot_mapping, "slot_mapping")
    _same_device(key, value, key_cache, value_cache, slot_mapping)
    T = slot_mapping.shape[0]
    if key.shape != (T, Hkv, D) or value.shape != (T, Hkv, D):
        raise ValueError(f"key/value must be [{T}, {Hkv}, {D}]")
    lib = _lib.load_library()
    st = lib.pkv_kv_cache_write_fp8(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                    _ptr(slot_mapping), T, Hkv, D, BS, NB, dt, float(k_scale),
                                    float(v_scale), _stream(key))
    _lib.check(st, "pkv_kv_cache_write_fp8")


def _prologue_fp8_args(block_tables, context_lens, key, value, key_cache, value_cache,
                       workspace, k_scale, v_scale, slot_mapping, stream):
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    dt = _kv(key, "key")
    if _kv(value, "value") != dt:
        raise TypeError("value dtype differs from key")
    NB, BS, Hkv, D = _fp8_caches(key_cache, value_cache)
    _dev(workspace, "workspace")
    B = context_lens.shape[0]
    if key.shape != (B, Hkv, D) or value.shape != (B, Hkv, D):
        raise ValueError(f"key/value must be [{B}, {Hkv}, {D}]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    if slot_mapping is None:
        slot_mapping = torch.empty(B, dtype=torch.int32, device=key.device)
    _i32(slot_mapping, "slot_mapping")
    _same_device(block_tables, context_lens, key, value, key_cache, value_cache, workspace,
                 slot_mapping)
    args = (_ptr(block_tables), _ptr(context_lens), _ptr(key), _ptr(value), _ptr(key_cache),
            _ptr(value_cache), _ptr(slot_mapping), B, block_tables.shape[1], Hkv, D, BS, NB, dt,
            float(k_scale), float(v_scale), _ptr(workspace),
            workspace.numel() * workspace.element_size(),
            stream if stream is not None else _stream(key))
    return "pkv_decode_prologue_fp8", args, slot_mapping


def decode_prologue_fp8(block_tables: torch.Tensor, context_lens: torch.Tensor,
                        key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                        value_cache: torch.Tensor, workspace: torch.Tensor, k_scale: float,
                        v_scale: float, slot_mapping: Optional[torch.Tensor] = None
                        ) -> torch.Tensor:
    """decode_prologue for E4M3 caches (balanced-split plan); returns the slots."""
    name, args, slot_mapping = _prologue_fp8_args(block_tables, context_lens, key, value,
                                                  key_cache, value_cache, workspace, k_scale,
                                                  v_scale, slot_mapping, None)
    _call(name, args)
    return slot_mapping


def _fp8_attention_args(query, key_cache, value_cache, block_tables, context_lens, out,
                        out_dtype, workspace):
    _dev(query, "query")
    if query.dtype != torch.bfloat16:
        raise TypeError("query must be bfloat16 beside E4M3 caches")
    NB, BS, Hkv, Dk = _fp8_caches(key_cache, value_cache)
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    if query.dim() != 3:
        raise ValueError("query [B, H, D]")
    B, H, D = query.shape
    if Dk != D or context_lens.shape != (B,) or block_tables.dim() != 2 or \
            block_tables.shape[0] != B:
        raise ValueError("inconsistent shapes")
    if out is None:
        out = torch.empty((B, H, D), dtype=out_dtype, device=query.device)
    if out.dtype not in _KV_DTYPES or out.shape != (B, H, D):
        raise ValueError("out must be float32/bfloat16 [B, H, D]")
    _dev(out, "out")
    if workspace is None:
        workspace = alloc_workspace(query, block_tables, BS, PARTITION_BALANCED)
    _dev(workspace, "workspace")
    _same_device(query, key_cache, value_cache, block_tables, context_lens, out, workspace)
    return out, workspace, workspace.numel() * workspace.element_size(), B, H, Hkv, D, BS, NB


def paged_attention_decode_fp8(query: torch.Tensor, key_cache: torch.Tensor,
                               value_cache: torch.Tensor, block_tables: torch.Tensor,
                               context_lens: torch.Tensor, scale: float, k_scale: float,
                               v_scale: float, out: Optional[torch.Tensor] = None,
                               out_dtype: torch.dtype = torch.float32,
                               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode attention over E4M3 caches (bf16 queries, balanced split)."""
    out, ws, wsb, B, H, Hkv, D, BS, NB = _fp8_attention_args(
        query, key_cache, value_cache, block_tables, context_lens, out, out_dtype, workspace)
    lib = _lib.load_library()
    st = lib.pkv_paged_attention_decode_fp8(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), B, H, Hkv, D, BS, block_tables.shape[1], NB, float(scale),
        float(k_scale), float(v_scale), _KV_DTYPES[out.dtype], _ptr(ws), wsb, _stream(query))
    _lib.check(st, "pkv_paged_attention_decode_fp8")
    return out


def _partition_fp8_args(query, key_cache, value_cache, block_tables, context_lens, scale,
                        k_scale, v_scale, out, out_dtype, workspace, stream):
    out, ws, wsb, B, H, Hkv, D, BS, NB = _fp8_attention_args(
        query, key_cache, value_cache, block_tables, context_lens, out, out_dtype, workspace)
    args = (_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
            _ptr(context_lens), B, H, Hkv, D, BS, block_tables.shape[1], NB, float(scale),
            float(k_scale), float(v_scale), _KV_DTYPES[out.dtype], _ptr(ws), wsb,
            stream if stream is not None else _stream(query))
    return "pkv_paged_attention_partition_fp8", args, out, ws


def paged_attention_partition_fp8(query, key_cache, value_cache, block_tables, context_lens,
                                  scale, k_scale, v_scale, out=None, out_dtype=torch.float32,
                                  workspace=None):
    """Stage 2 over E4M3 caches (needs a balanced plan in ``workspace``); returns
    (out, workspace)."""
    name, args, out, ws = _partition_fp8_args(query, key_cache, value_cache, block_tables,
                                              context_lens, scale, k_scale, v_scale, out,
                                              out_dtype, workspace, None)
    _call(name, args)
    return out, ws


class DecodeStep:
    """One decode step bound to fixed tensors: slot mapping, cache write and plan
    (``prologue``), the partition stage (``partition``) and the merge (``reduce``).

    The arguments are checked once, here, and each stage is then a single C call with
    the stored pointers and sizes, on the stream given (default: the current stream of
    the query's device at construction).  The tensors' contents may change between
    calls (new tokens, longer contexts, new block tables); their storage, shapes and
    dtypes must not.  ``partition_size`` None is the library default (512-token
    partitions); ``per_head`` selects the per-head layout of fixed partitions.  E4M3
    caches (uint8 or float8_e4m3fn) take ``k_scale`` and ``v_scale`` and always use the
    balanced split."""

    def __init__(self, query, key, value, key_cache, value_cache, block_tables, context_lens,
                 scale, partition_size=None, out=None, out_dtype=torch.float32, workspace=None,
                 slot_mapping=None, k_scale=None, v_scale=None, stream=None, per_head=False):
        _dev(query, "query")
        fp8 = isinstance(key_cache, torch.Tensor) and key_cache.dtype in _FP8_DTYPES
        if fp8 and (k_scale is None or v_scale is None):
            raise ValueError("E4M3 caches need k_scale and v_scale")
        if partition_size is None:
            partition_size = PARTITION_BALANCED if fp8 else PARTITION_DEFAULT
        if fp8 and (partition_size != PARTITION_BALANCED or per_head):
            raise ValueError("E4M3 caches use the balanced split (PARTITION_BALANCED)")
        if per_head and partition_size == PARTITION_BALANCED:
            raise ValueError("the per-head layout runs fixed partitions only")
        if stream is None:
            stream = torch.cuda.current_stream(query.device)
        st = ctypes.c_void_p(stream.cuda_stream)
        BS = key_cache.shape[1]
        if workspace is None:
            workspace = alloc_workspace(query, block_tables, BS, partition_size)
        if fp8:
            self._prologue = _prologue_fp8_args(block_tables, context_lens, key, value,
                                                key_cache, value_cache, workspace, k_scale,
                                                v_scale, slot_mapping, st)
            self._partition = _partition_fp8_args(query, key_cache, value_cache, block_tables,
                                                  context_lens, scale, k_scale, v_scale, out,
                                                  out_dtype, workspace, st)
        else:
            self._prologue = _prologue_args(block_tables, context_lens, key, value, key_cache,
                                            value_cache, workspace, partition_size,
                                            slot_mapping, st)
            self._partition = _partition_args(query, key_cache, value_cache, block_tables,
                                              context_lens, scale, partition_size, out,
                                              out_dtype, workspace, st, per_head=per_head)
        self.slot_mapping = self._prologue[2]
        self.out, self.workspace = self._partition[2], self._partition[3]
        self._reduce = _reduce_args(self.out, context_lens, workspace, BS, block_tables.shape[1],
                                    partition_size, st)
        lib = _lib.load_library()
        self._fns = [(getattr(lib, c[0]), c[0], c[1])
                     for c in (self._prologue, self._partition, self._reduce)]
        # the tensors whose pointers the calls hold
        self._keep = (query, key, value, key_cache, value_cache, block_tables, context_lens)

    def _run(self, i: int) -> None:
        fn, name, args = self._fns[i]
        st = fn(*args)
        if st:
            _lib.check(st, name)

    def prologue(self) -> None:
        self._run(0)

    def partition(self) -> None:
        self._run(1)

    def reduce(self) -> None:
        self._run(2)

    def __call__(self) -> torch.Tensor:
        self._run(0)
        self._run(1)
        self._run(2)
        return self.out


def copy_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor,
                pairs: torch.Tensor) -> None:
    """Copy-on-write copies: block dst of both caches becomes block src, for every
    (src, dst) row of ``pairs`` (int32 [n, 2] on the caches' device)."""
    dt = _storage(key_cache, "key_cache")
    if _storage(value_cache, "value_cache") != dt:
        raise TypeError("value_cache dtype differs from key_cache")
    _i32(pairs, "pairs")
    _same_device(key_cache, value_cache, pairs)
    if key_cache.dim() != 4 or value_cache.shape != key_cache.shape:
        raise ValueError("caches must both be [num_blocks, block_size, num_kv_heads, head_dim]")
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n, 2]")
    NB, BS, Hkv, D = key_cache.shape
    lib = _lib.load_library()
    st = lib.pkv_copy_blocks(_ptr(key_cache), _ptr(value_cache), _ptr(pairs), pairs.shape[0], Hkv,
                             D, BS, NB, dt, _stream(key_cache))
    _lib.check(st, "pkv_copy_blocks")


def prefix_block_hashes(tokens, block_size: int) -> np.ndarray:
    """Chained hashes (uint64) of the full blocks of a token sequence."""
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
    out = np.zeros(t.shape[0] // int(block_size), np.uint64)
    _lib.check(_lib.load_library().pkv_prefix_block_hashes(
        t.ctypes.data_as(ctypes.c_void_p), t.shape[0], int(block_size),
        out.ctypes.data_as(ctypes.c_void_p)), "pkv_prefix_block_hashes")
    return out


class BlockPool:
    """The library's host block pool (free list and reference counts of the physical
    blocks).  Block tables are numpy int32 arrays [num_seqs, capacity] with their
    lengths in a separate int32 array; both are updated in place."""

    def __init__(self, num_blocks: int):
        self._lib = _lib.load_library()
        h = ctypes.c_void_p()
        _lib.check(self._lib.pkv_block_pool_create(int(num_blocks), ctypes.byref(h)),
                   "pkv_block_pool_create")
        self._h = h
        self.num_blocks = int(num_blocks)

    def close(self) -> None:
        if self._h:
            self._lib.pkv_block_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_free(self) -> int:
        return self._lib.pkv_block_pool_num_free(self._h)

    def ref_count(self, block: int) -> int:
        return self._lib.pkv_block_pool_ref_count(self._h, int(block))

    def allocate(self) -> int:
        b = ctypes.c_int32()
        _lib.check(self._lib.pkv_block_pool_allocate(self._h, ctypes.byref(b)),
                   "pkv_block_pool_allocate")
        return b.value

    @staticmethod
    def _ids(blocks):
        a = np.ascontiguousarray(np.asarray(blocks, dtype=np.int32).reshape(-1))
        return a, a.ctypes.data_as(ctypes.c_void_p)

    def release(self, blocks) -> None:
        a, p = self._ids(blocks)
        _lib.check(self._lib.pkv_block_pool_release(self._h, p, a.shape[0]),
                   "pkv_block_pool_release")

    def fork(self, blocks) -> None:
        a, p = self._ids(blocks)
        _lib.check(self._lib.pkv_block_pool_fork(self._h, p, a.shape[0]), "pkv_block_pool_fork")

    # ---- prefix caching ----
    @property
    def num_cached(self) -> int:
        return self._lib.pkv_block_pool_num_cached(self._h)

    def match_prefix(self, tokens, block_size: int) -> list:
        """Reused leading full blocks of ``tokens`` (their counts raised)."""
        t, p = self._ids(tokens)
        out = np.empty(max(1, t.shape[0] // int(block_size)), np.int32)
        n = ctypes.c_int32()
        _lib.check(self._lib.pkv_block_pool_match_prefix(
            self._h, p, t.shape[0], int(block_size), out.ctypes.data_as(ctypes.c_void_p),
            t.shape[0] // int(block_size), ctypes.byref(n)), "pkv_block_pool_match_prefix")
        return out[:n.value].tolist()

    def register_prefix(self, tokens, table, block_size: int) -> int:
        """Enter the full blocks of a sequence (K/V stored in ``table``) into the map;
        returns how many entered."""
        t, p = self._ids(tokens)
        tb, tp = self._ids(table)
        n = ctypes.c_int32()
        _lib.check(self._lib.pkv_block_pool_register_prefix(
            self._h, p, t.shape[0], int(block_size), tp, tb.shape[0], ctypes.byref(n)),
            "pkv_block_pool_register_prefix")
        return n.value

    def append_slots(self, tables: np.ndarray, table_lens: np.ndarray, num_tokens,
                     block_size: int):
        """Slots of every sequence's next token; returns (slots int32 [B], copies
        int32 [n, 2]).  Raises PkvError (status PKV_ERR_NO_BLOCKS when the pool runs
        dry); the sequences handled before the failure stay updated."""
        for a, n in ((tables, "tables"), (table_lens, "table_lens")):
            if not (isinstance(a, np.ndarray) and a.dtype == np.int32 and a.flags.c_contiguous):
                raise TypeError(f"{n} must be a C-contiguous numpy int32 array")
        B = table_lens.shape[0]
        if tables.ndim != 2 or tables.shape[0] != B:
            raise ValueError("tables must be [num_seqs, capacity]")
        ntok = np.ascontiguousarray(np.asarray(num_tokens, dtype=np.int32))
        if ntok.shape != (B,):
            raise ValueError("num_tokens must have one entry per sequence")
        slots = np.empty(B, np.int32)
        copies = np.empty((max(B, 1), 2), np.int32)
        ncp, done = ctypes.c_int32(), ctypes.c_int32()
        vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        st = self._lib.pkv_block_pool_append_slots(self._h, vp(tables), vp(table_lens),
                                                   tables.shape[1], vp(ntok), B, int(block_size),
                                                   vp(slots), vp(copies), ctypes.byref(ncp),
                                                   ctypes.byref(done))
        _lib.check(st, f"pkv_block_pool_append_slots (done {done.value} of {B})")
        return slots, copies[:ncp.value].copy()
