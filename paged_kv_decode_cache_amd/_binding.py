"""ctypes binding of libpkv.so.

Argument marshalling only: shapes, dtypes and devices of torch tensors are
checked, raw device pointers and the current HIP stream are handed to the C
ABI, and its status codes become exceptions.  Every step of the computation
runs in the library's HIP kernels; there is no other implementation to fall
back to, so a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "pkv.h")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_LAUNCH = -3
PKV_ERR_NO_SPACE = -4
PKV_ERR_SCRATCH = -5


class NoSpaceError(RuntimeError):
    """The block allocator has too few free blocks (or a table is full)."""

_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float

_SIGNATURES = {
    "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_version": (ctypes.c_int, []),
    "kv_cache_append": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "paged_attention_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                              _I, _F, _P]),
    "paged_attention_decode_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                                 _I, _I, _F, _P, _P]),
    "paged_attention_decode_split": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I,
                                                    _I, _I, _I, _I, _I, _I, _F, _P]),
    "paged_attention_decode_split_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I,
                                                       _I, _I, _I, _I, _I, _I, _F, _P, _P]),
    "split_reduce": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "paged_decode_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                         _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "paged_decode_step_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                            _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P]),
    "paged_decode_step_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I,
                                                 _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "paged_decode_step_q8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                            _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                                            _P]),
    "paged_attention_prefill": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                               _I, _I, _I, _F, _P]),
    "paged_attention_prefill_split": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I,
                                                     _I, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "kv_cache_append_q8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "paged_attention_decode_q8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                                 _I, _I, _I, _F, _P]),
    "paged_attention_decode_split_q8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I,
                                                       _I, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "pkv_allocator_create": (_P, [_I, _I, _I, _I]),
    "pkv_allocator_destroy": (None, [_P]),
    "pkv_allocator_num_free": (_I, [_P]),
    "pkv_allocator_context_len": (_I, [_P, _I]),
    "pkv_allocator_append_slots": (ctypes.c_int, [_P, _I, _I, _P]),
    "pkv_allocator_free_seq": (ctypes.c_int, [_P, _I]),
    "pkv_allocator_block_table": (ctypes.c_int, [_P, _I, _P, _I]),
    "pkv_allocator_build_decode_batch": (ctypes.c_int, [_P, _P, _I, _I, _P, _P, _P]),
    "pkv_allocator_build_prefill_batch": (ctypes.c_int, [_P, _P, _P, _I, _I, _P, _P, _P, _P]),
}

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpkv.so (built in-tree) and declare its C signatures."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m paged_kv_decode_cache_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def declared_functions(header: str = HEADER_PATH):
    """Names of the functions include/pkv.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, flags=re.M)))


def status_string(code: int) -> str:
    return load_library().pkv_status_string(code).decode()


def _raise(code: int, what: str):
    if code == PKV_OK:
        return
    msg = f"{what}: {status_string(code)} (status {code})"
    if code == PKV_ERR_INVALID_ARG:
        raise ValueError(msg)
    if code == PKV_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    if code == PKV_ERR_NO_SPACE:
        raise NoSpaceError(msg)
    raise RuntimeError(msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class LaunchConfig(ctypes.Structure):
    """pkv_launch_config: an explicit launch shape for one call (0 = default).
    grid: 0 auto, 1 direct, 2 compact."""
    _fields_ = [("waves_per_group", ctypes.c_int32), ("subtiles_per_tile", ctypes.c_int32),
                ("tiles_in_flight", ctypes.c_int32), ("grid", ctypes.c_int32)]


_GRID = {"auto": 0, "direct": 1, "compact": 2}


def _launch(launch):
    """None, or a LaunchConfig from a dict with keys waves, subtiles, depth,
    grid ('auto' / 'direct' / 'compact')."""
    if launch is None:
        return None
    if isinstance(launch, LaunchConfig):
        return launch
    unknown = set(launch) - {"waves", "subtiles", "depth", "grid"}
    if unknown:
        raise ValueError(f"unknown launch keys {sorted(unknown)}")
    grid = launch.get("grid", 0)
    return LaunchConfig(int(launch.get("waves", 0)), int(launch.get("subtiles", 0)),
                        int(launch.get("depth", 0)), _GRID[grid] if isinstance(grid, str)
                        else int(grid))


def kv_cache_append(k_pool, v_pool, k_new, v_new, slot_mapping, stream=None):
    """Write k_new/v_new [N, Hkv, D] into the pools at slot_mapping [N]."""
    _need(k_pool, "k_pool", torch.float16, 4)
    dev = k_pool.device
    _need(v_pool, "v_pool", torch.float16, 4, dev)
    _need(k_new, "k_new", torch.float16, 3, dev)
    _need(v_new, "v_new", torch.float16, 3, dev)
    _need(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    NB, bs, Hkv, D = k_pool.shape
    N = k_new.shape[0]
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")
    if k_new.shape != (N, Hkv, D) or v_new.shape != (N, Hkv, D) or slot_mapping.shape != (N,):
        raise ValueError("k_new/v_new must be [N, Hkv, D] and slot_mapping [N]")
    rc = load_library().kv_cache_append(_ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new),
                                        _ptr(slot_mapping), N, NB, bs, Hkv, D,
                                        _stream(dev, stream))
    _raise(rc, "kv_cache_append")


def _attn_shapes(q, k_pool, v_pool, block_tables, context_lens):
    _need(q, "q", torch.float16, 3)
    dev = q.device
    _need(k_pool, "k_pool", torch.float16, 4, dev)
    _need(v_pool, "v_pool", torch.float16, 4, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, Hq, D = q.shape
    NB, bs, Hkv, D2 = k_pool.shape
    if v_pool.shape != k_pool.shape or D2 != D:
        raise ValueError("pools must be [num_blocks, block_size, Hkv, D] with q's D")
    if block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, max_blocks] and context_lens [B]")
    return dev, B, Hq, Hkv, D, bs, NB, block_tables.shape[1]


def paged_attention_decode(q, k_pool, v_pool, block_tables, context_lens, scale,
                           out=None, stream=None, launch=None):
    """out [B, Hq, D] fp16 = paged decode attention (one launch).  launch: an
    explicit launch shape (dict: waves, subtiles, depth), else defaults."""
    dev, B, Hq, Hkv, D, bs, NB, maxb = _attn_shapes(q, k_pool, v_pool, block_tables,
                                                    context_lens)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    _need(out, "out", torch.float16, 3, dev)
    if out.shape != (B, Hq, D):
        raise ValueError("out must be [B, Hq, D]")
    args = (_ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
            _ptr(context_lens), B, Hq, Hkv, D, bs, NB, maxb, float(scale))
    cfg = _launch(launch)
    if cfg is None:
        rc = load_library().paged_attention_decode(*args, _stream(dev, stream))
    else:
        rc = load_library().paged_attention_decode_ex(*args, ctypes.byref(cfg),
                                                      _stream(dev, stream))
    _raise(rc, "paged_attention_decode")
    return out


def paged_attention_prefill(q, k_pool, v_pool, block_tables, context_lens, query_start, scale,
                            max_query_len, out=None, stream=None):
    """Chunked-prefill attention: q and out are [total_q, Hq, D]; sequence b's
    chunk is rows query_start[b] .. query_start[b+1]-1 (int32 [B + 1] on the
    GPU), the last rows of its context_lens[b] positions, attended causally.
    max_query_len bounds every chunk length (it sizes the launch; the binding
    does not read device data to find it)."""
    _need(q, "q", torch.float16, 3)
    dev = q.device
    _need(k_pool, "k_pool", torch.float16, 4, dev)
    _need(v_pool, "v_pool", torch.float16, 4, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    _need(query_start, "query_start", torch.int32, 1, dev)
    T, Hq, D = q.shape
    NB, bs, Hkv, D2 = k_pool.shape
    B = context_lens.shape[0]
    if v_pool.shape != k_pool.shape or D2 != D:
        raise ValueError("pools must be [num_blocks, block_size, Hkv, D] with q's D")
    if block_tables.shape[0] != B or query_start.shape != (B + 1,):
        raise ValueError("block_tables must be [B, max_blocks] and query_start [B + 1]")
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float16, device=dev)
    _need(out, "out", torch.float16, 3, dev)
    if out.shape != (T, Hq, D):
        raise ValueError("out must have q's shape")
    rc = load_library().paged_attention_prefill(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), _ptr(context_lens),
        _ptr(query_start), B, int(max_query_len), Hq, Hkv, D, bs, NB, block_tables.shape[1],
        float(scale), _stream(dev, stream))
    _raise(rc, "paged_attention_prefill")
    return out


def paged_attention_prefill_split(q, k_pool, v_pool, block_tables, context_lens, query_start,
                                  scale, max_query_len, partition_size, max_partitions=None,
                                  partial_out=None, partial_lse=None, row_context_lens=None,
                                  stream=None):
    """Split pass of chunked-prefill attention over context partitions.
    Returns (partial_out [total_q, Hq, Pm, D] fp32, partial_lse [total_q, Hq,
    Pm] fp32, row_context_lens [total_q] int32); merge with
    split_reduce(partial_out, partial_lse, row_context_lens, partition_size).
    row_context_lens starts as zeros when allocated here, so rows no sequence
    owns merge to zeros."""
    _need(q, "q", torch.float16, 3)
    dev = q.device
    _need(k_pool, "k_pool", torch.float16, 4, dev)
    _need(v_pool, "v_pool", torch.float16, 4, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    _need(query_start, "query_start", torch.int32, 1, dev)
    T, Hq, D = q.shape
    NB, bs, Hkv, D2 = k_pool.shape
    B = context_lens.shape[0]
    if v_pool.shape != k_pool.shape or D2 != D:
        raise ValueError("pools must be [num_blocks, block_size, Hkv, D] with q's D")
    if block_tables.shape[0] != B or query_start.shape != (B + 1,):
        raise ValueError("block_tables must be [B, max_blocks] and query_start [B + 1]")
    maxb = block_tables.shape[1]
    if max_partitions is None:
        max_partitions = max_partitions_for(maxb, bs, partition_size)
    Pm = int(max_partitions)
    if partial_out is None:
        partial_out = torch.empty((T, Hq, Pm, D), dtype=torch.float32, device=dev)
    if partial_lse is None:
        partial_lse = torch.empty((T, Hq, Pm), dtype=torch.float32, device=dev)
    if row_context_lens is None:
        row_context_lens = torch.zeros((T,), dtype=torch.int32, device=dev)
    _need(partial_out, "partial_out", torch.float32, 4, dev)
    _need(partial_lse, "partial_lse", torch.float32, 3, dev)
    _need(row_context_lens, "row_context_lens", torch.int32, 1, dev)
    if partial_out.shape != (T, Hq, Pm, D) or partial_lse.shape != (T, Hq, Pm) or \
            row_context_lens.shape != (T,):
        raise ValueError("partials must be [total_q, Hq, Pm, D] / [total_q, Hq, Pm] and "
                         "row_context_lens [total_q]")
    rc = load_library().paged_attention_prefill_split(
        _ptr(partial_out), _ptr(partial_lse), _ptr(row_context_lens), _ptr(q), _ptr(k_pool),
        _ptr(v_pool), _ptr(block_tables), _ptr(context_lens), _ptr(query_start), B,
        int(max_query_len), Hq, Hkv, D, bs, NB, maxb, int(partition_size), Pm, float(scale),
        _stream(dev, stream))
    _raise(rc, "paged_attention_prefill_split")
    return partial_out, partial_lse, row_context_lens


def _q8_shapes(k_codes, v_codes, k_scales, v_scales, dev):
    _need(k_codes, "k_codes", torch.int8, 4, dev)
    _need(v_codes, "v_codes", torch.int8, 4, dev)
    _need(k_scales, "k_scales", torch.float32, 3, dev)
    _need(v_scales, "v_scales", torch.float32, 3, dev)
    NB, Hkv, bs, D = k_codes.shape
    if v_codes.shape != k_codes.shape or k_scales.shape != (NB, Hkv, bs) or \
            v_scales.shape != (NB, Hkv, bs):
        raise ValueError("8-bit pools: codes [num_blocks, Hkv, block_size, D] int8 and scales "
                         "[num_blocks, Hkv, block_size] fp32")
    return NB, bs, Hkv, D


def kv_cache_append_q8(k_codes, v_codes, k_scales, v_scales, k_new, v_new, slot_mapping,
                       stream=None):
    """Quantise and write each new token's K/V rows into the 8-bit cache."""
    _need(k_new, "k_new", torch.float16, 3)
    dev = k_new.device
    NB, bs, Hkv, D = _q8_shapes(k_codes, v_codes, k_scales, v_scales, dev)
    _need(v_new, "v_new", torch.float16, 3, dev)
    _need(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    N = k_new.shape[0]
    if k_new.shape != (N, Hkv, D) or v_new.shape != (N, Hkv, D) or slot_mapping.shape != (N,):
        raise ValueError("k_new/v_new must be [N, Hkv, D] and slot_mapping [N]")
    rc = load_library().kv_cache_append_q8(
        _ptr(k_codes), _ptr(v_codes), _ptr(k_scales), _ptr(v_scales), _ptr(k_new), _ptr(v_new),
        _ptr(slot_mapping), N, NB, bs, Hkv, D, _stream(dev, stream))
    _raise(rc, "kv_cache_append_q8")


def paged_attention_decode_q8(q, k_codes, v_codes, k_scales, v_scales, block_tables,
                              context_lens, scale, out=None, stream=None):
    """Paged decode over the 8-bit cache (one launch): out [B, Hq, D] fp16."""
    _need(q, "q", torch.float16, 3)
    dev = q.device
    NB, bs, Hkv, D = _q8_shapes(k_codes, v_codes, k_scales, v_scales, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, Hq, Dq = q.shape
    if Dq != D or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("q must be [B, Hq, D], block_tables [B, max_blocks], context_lens [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    _need(out, "out", torch.float16, 3, dev)
    rc = load_library().paged_attention_decode_q8(
        _ptr(out), _ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_scales), _ptr(v_scales),
        _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, D, bs, NB, block_tables.shape[1],
        float(scale), _stream(dev, stream))
    _raise(rc, "paged_attention_decode_q8")
    return out


def paged_attention_decode_split_q8(q, k_codes, v_codes, k_scales, v_scales, block_tables,
                                    context_lens, scale, partition_size, max_partitions=None,
                                    partial_out=None, partial_lse=None, stream=None):
    """Split pass over the 8-bit cache; merge with split_reduce."""
    _need(q, "q", torch.float16, 3)
    dev = q.device
    NB, bs, Hkv, D = _q8_shapes(k_codes, v_codes, k_scales, v_scales, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, Hq, _ = q.shape
    Pm = max_partitions or max_partitions_for(block_tables.shape[1], bs, partition_size)
    if partial_out is None:
        partial_out = torch.empty((B, Hq, Pm, D), dtype=torch.float32, device=dev)
    if partial_lse is None:
        partial_lse = torch.empty((B, Hq, Pm), dtype=torch.float32, device=dev)
    _need(partial_out, "partial_out", torch.float32, 4, dev)
    _need(partial_lse, "partial_lse", torch.float32, 3, dev)
    rc = load_library().paged_attention_decode_split_q8(
        _ptr(partial_out), _ptr(partial_lse), _ptr(q), _ptr(k_codes), _ptr(v_codes),
        _ptr(k_scales), _ptr(v_scales), _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, D,
        bs, NB, block_tables.shape[1], partition_size, Pm, float(scale), _stream(dev, stream))
    _raise(rc, "paged_attention_decode_split_q8")
    return partial_out, partial_lse


def max_partitions_for(max_blocks_per_seq: int, block_size: int, partition_size: int) -> int:
    return -(-max_blocks_per_seq * block_size // partition_size)


def paged_attention_decode_split(q, k_pool, v_pool, block_tables, context_lens, scale,
                                 partition_size, max_partitions=None, partial_out=None,
                                 partial_lse=None, stream=None, launch=None):
    """Split pass; returns (partial_out [B,Hq,P,D] fp32, partial_lse [B,Hq,P] fp32).
    launch: an explicit launch shape (dict: waves, subtiles, depth, grid)."""
    dev, B, Hq, Hkv, D, bs, NB, maxb = _attn_shapes(q, k_pool, v_pool, block_tables,
                                                    context_lens)
    if max_partitions is None:
        max_partitions = max_partitions_for(maxb, bs, partition_size)
    if partial_out is None:
        partial_out = torch.empty((B, Hq, max_partitions, D), dtype=torch.float32, device=dev)
    if partial_lse is None:
        partial_lse = torch.empty((B, Hq, max_partitions), dtype=torch.float32, device=dev)
    _need(partial_out, "partial_out", torch.float32, 4, dev)
    _need(partial_lse, "partial_lse", torch.float32, 3, dev)
    if partial_out.shape != (B, Hq, max_partitions, D) or \
            partial_lse.shape != (B, Hq, max_partitions):
        raise ValueError("partial_out must be [B, Hq, P, D] and partial_lse [B, Hq, P]")
    args = (_ptr(partial_out), _ptr(partial_lse), _ptr(q), _ptr(k_pool), _ptr(v_pool),
            _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, D, bs, NB, maxb,
            int(partition_size), int(max_partitions), float(scale))
    cfg = _launch(launch)
    if cfg is None:
        rc = load_library().paged_attention_decode_split(*args, _stream(dev, stream))
    else:
        rc = load_library().paged_attention_decode_split_ex(*args, ctypes.byref(cfg),
                                                            _stream(dev, stream))
    _raise(rc, "paged_attention_decode_split")
    return partial_out, partial_lse


def split_reduce(partial_out, partial_lse, context_lens, partition_size, out=None,
                 lse_out=None, want_lse=False, stream=None):
    """Merge partitions; returns out [B, Hq, D] fp16 (and lse [B, Hq] fp32)."""
    _need(partial_out, "partial_out", torch.float32, 4)
    dev = partial_out.device
    _need(partial_lse, "partial_lse", torch.float32, 3, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, Hq, P, D = partial_out.shape
    if partial_lse.shape != (B, Hq, P) or context_lens.shape != (B,):
        raise ValueError("partial_lse must be [B, Hq, P] and context_lens [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    _need(out, "out", torch.float16, 3, dev)
    if want_lse and lse_out is None:
        lse_out = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, 2, dev)
        if lse_out.shape != (B, Hq):
            raise ValueError("lse_out must be [B, Hq]")
    rc = load_library().split_reduce(_ptr(out), _ptr(lse_out), _ptr(partial_out),
                                     _ptr(partial_lse), _ptr(context_lens), B, Hq, D,
                                     int(partition_size), P, _stream(dev, stream))
    _raise(rc, "split_reduce")
    return (out, lse_out) if lse_out is not None else out


COUNTER_STRIDE = 32  # int32 words per ticket counter (one 128-byte line)


class StepWorkspace:
    """Device workspace of paged_decode_step: split partials and the
    per-(sequence, KV head) ticket counters, all zero ("not written").  Set up
    here once; every call leaves it in that state.  Allocated with torch by
    the caller's code, never by the library.  reset() restores the state
    (after an aborted call)."""

    def __init__(self, B, num_q_heads, num_kv_heads, head_dim, max_partitions, device):
        self.partial_out = torch.empty((B, num_q_heads, max_partitions, head_dim),
                                       dtype=torch.float32, device=device)
        self.partial_lse = torch.empty((B, num_q_heads, max_partitions), dtype=torch.float32,
                                       device=device)
        # one 128-byte line of ticket counter per (sequence, KV head)
        self.counters = torch.empty((B, num_kv_heads, COUNTER_STRIDE), dtype=torch.int32,
                                    device=device)
        self.max_partitions = max_partitions
        self.reset()

    def reset(self):
        self.partial_out.zero_()
        self.partial_lse.zero_()
        self.counters.zero_()


def paged_decode_step(q, k_pool, v_pool, block_tables, context_lens, scale, partition_size,
                      k_new=None, v_new=None, slot_mapping=None, workspace=None, out=None,
                      lse_out=None, want_lse=False, stream=None, launch=None):
    """Fused decode step: append (if slot_mapping is given) + split pass +
    merge in one launch.  Returns out [B, Hq, D] fp16 (and lse [B, Hq]).
    launch: an explicit launch shape (dict: waves, subtiles, depth, grid)."""
    dev, B, Hq, Hkv, D, bs, NB, maxb = _attn_shapes(q, k_pool, v_pool, block_tables,
                                                    context_lens)
    Pm = max_partitions_for(maxb, bs, partition_size)
    if workspace is None:
        workspace = StepWorkspace(B, Hq, Hkv, D, Pm, dev)
    ws = workspace
    _need(ws.partial_out, "partial_out", torch.float32, 4, dev)
    _need(ws.partial_lse, "partial_lse", torch.float32, 3, dev)
    _need(ws.counters, "counters", torch.int32, 3, dev)
    Pm = ws.max_partitions
    if ws.partial_out.shape != (B, Hq, Pm, D) or ws.partial_lse.shape != (B, Hq, Pm) or \
            ws.counters.shape != (B, Hkv, COUNTER_STRIDE):
        raise ValueError("workspace shapes do not match the call")
    if slot_mapping is not None:
        _need(k_new, "k_new", torch.float16, 3, dev)
        _need(v_new, "v_new", torch.float16, 3, dev)
        _need(slot_mapping, "slot_mapping", torch.int64, 1, dev)
        if k_new.shape != (B, Hkv, D) or v_new.shape != (B, Hkv, D) or \
                slot_mapping.shape != (B,):
            raise ValueError("k_new/v_new must be [B, Hkv, D] and slot_mapping [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    _need(out, "out", torch.float16, 3, dev)
    if want_lse and lse_out is None:
        lse_out = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, 2, dev)
    args = (_ptr(out), _ptr(lse_out), _ptr(k_pool), _ptr(v_pool), _ptr(q),
            _ptr(k_new) if slot_mapping is not None else None,
            _ptr(v_new) if slot_mapping is not None else None, _ptr(slot_mapping),
            _ptr(block_tables), _ptr(context_lens), _ptr(ws.partial_out), _ptr(ws.partial_lse),
            _ptr(ws.counters), B, Hq, Hkv, D, bs, NB, maxb, int(partition_size), Pm,
            float(scale))
    cfg = _launch(launch)
    if cfg is None:
        rc = load_library().paged_decode_step(*args, _stream(dev, stream))
    else:
        rc = load_library().paged_decode_step_ex(*args, ctypes.byref(cfg), _stream(dev, stream))
    _raise(rc, "paged_decode_step")
    return (out, lse_out) if lse_out is not None else out


def paged_decode_step_noalloc(q, k_pool, v_pool, block_tables, context_lens, scale,
                              partition_size, k_new=None, v_new=None, slot_mapping=None,
                              out=None, lse_out=None, want_lse=False, stream=None):
    """paged_decode_step on the library's static scratch (no workspace; the C
    call allocates nothing).  Returns out [B, Hq, D] fp16 (and lse [B, Hq]).
    Raises ValueError when the call needs more scratch than the library holds
    (PKV_ERR_SCRATCH)."""
    dev, B, Hq, Hkv, D, bs, NB, maxb = _attn_shapes(q, k_pool, v_pool, block_tables,
                                                    context_lens)
    Pm = max_partitions_for(maxb, bs, partition_size)
    if slot_mapping is not None:
        _need(k_new, "k_new", torch.float16, 3, dev)
        _need(v_new, "v_new", torch.float16, 3, dev)
        _need(slot_mapping, "slot_mapping", torch.int64, 1, dev)
        if k_new.shape != (B, Hkv, D) or v_new.shape != (B, Hkv, D) or \
                slot_mapping.shape != (B,):
            raise ValueError("k_new/v_new must be [B, Hkv, D] and slot_mapping [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    _need(out, "out", torch.float16, 3, dev)
    if want_lse and lse_out is None:
        lse_out = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, 2, dev)
    rc = load_library().paged_decode_step_noalloc(
        _ptr(out), _ptr(lse_out), _ptr(k_pool), _ptr(v_pool), _ptr(q),
        _ptr(k_new) if slot_mapping is not None else None,
        _ptr(v_new) if slot_mapping is not None else None, _ptr(slot_mapping),
        _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, D, bs, NB, maxb,
        int(partition_size), Pm, float(scale), _stream(dev, stream))
    if rc == PKV_ERR_SCRATCH:
        raise ValueError(f"paged_decode_step_noalloc: {status_string(rc)} (status {rc})")
    _raise(rc, "paged_decode_step_noalloc")
    return (out, lse_out) if lse_out is not None else out


def paged_decode_step_q8(q, k_codes, v_codes, k_scales, v_scales, block_tables, context_lens,
                         scale, partition_size, k_new=None, v_new=None, slot_mapping=None,
                         workspace=None, out=None, lse_out=None, want_lse=False, stream=None):
    """Fused decode step over the 8-bit cache: quantising append (if
    slot_mapping is given) + split pass + merge in one launch.  Returns out
    [B, Hq, D] fp16 (and lse [B, Hq])."""
    _need(q, "q", torch.float16, 3)
    dev = q.device
    NB, bs, Hkv, D = _q8_shapes(k_codes, v_codes, k_scales, v_scales, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, Hq, Dq = q.shape
    if Dq != D or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("q must be [B, Hq, D], block_tables [B, max_blocks], context_lens [B]")
    maxb = block_tables.shape[1]
    Pm = max_partitions_for(maxb, bs, partition_size)
    if workspace is None:
        workspace = StepWorkspace(B, Hq, Hkv, D, Pm, dev)
    ws = workspace
    _need(ws.partial_out, "partial_out", torch.float32, 4, dev)
    _need(ws.partial_lse, "partial_lse", torch.float32, 3, dev)
    _need(ws.counters, "counters", torch.int32, 3, dev)
    Pm = ws.max_partitions
    if ws.partial_out.shape != (B, Hq, Pm, D) or ws.partial_lse.shape != (B, Hq, Pm) or \
            ws.counters.shape != (B, Hkv, COUNTER_STRIDE):
        raise ValueError("workspace shapes do not match the call")
    if slot_mapping is not None:
        _need(k_new, "k_new", torch.float16, 3, dev)
        _need(v_new, "v_new", torch.float16, 3, dev)
        _need(slot_mapping, "slot_mapping", torch.int64, 1, dev)
        if k_new.shape != (B, Hkv, D) or v_new.shape != (B, Hkv, D) or \
                slot_mapping.shape != (B,):
            raise ValueError("k_new/v_new must be [B, Hkv, D] and slot_mapping [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    _need(out, "out", torch.float16, 3, dev)
    if want_lse and lse_out is None:
        lse_out = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, 2, dev)
    rc = load_library().paged_decode_step_q8(
        _ptr(out), _ptr(lse_out), _ptr(k_codes), _ptr(v_codes), _ptr(k_scales), _ptr(v_scales),
        _ptr(q), _ptr(k_new) if slot_mapping is not None else None,
        _ptr(v_new) if slot_mapping is not None else None, _ptr(slot_mapping),
        _ptr(block_tables), _ptr(context_lens), _ptr(ws.partial_out), _ptr(ws.partial_lse),
        _ptr(ws.counters), B, Hq, Hkv, D, bs, NB, maxb, int(partition_size), Pm, float(scale),
        _stream(dev, stream))
    _raise(rc, "paged_decode_step_q8")
    return (out, lse_out) if lse_out is not None else out


def _np_ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


class BlockAllocator:
    """Host block allocator of the paged cache (the library's pkv_allocator_*
    calls on host memory): a FIFO free-block queue, one block table per
    sequence id, slot mappings and batch metadata as numpy arrays."""

    def __init__(self, num_blocks, block_size, max_seqs, max_blocks_per_seq):
        import numpy as np
        self._np = np
        self._lib = load_library()
        self._h = self._lib.pkv_allocator_create(num_blocks, block_size, max_seqs,
                                                 max_blocks_per_seq)
        if not self._h:
            raise ValueError("pkv_allocator_create failed (bad sizes or out of memory)")
        self.num_blocks, self.block_size = num_blocks, block_size
        self.max_seqs, self.max_blocks_per_seq = max_seqs, max_blocks_per_seq

    def close(self):
        if self._h:
            self._lib.pkv_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_free(self) -> int:
        return int(self._lib.pkv_allocator_num_free(self._h))

    def context_len(self, seq) -> int:
        n = int(self._lib.pkv_allocator_context_len(self._h, seq))
        if n < 0:
            _raise(n, "pkv_allocator_context_len")
        return n

    def append_slots(self, seq, num_tokens):
        out = self._np.empty(max(num_tokens, 0), dtype=self._np.int64)
        _raise(self._lib.pkv_allocator_append_slots(self._h, seq, num_tokens, _np_ptr(out)),
               "pkv_allocator_append_slots")
        return out

    def free(self, seq):
        _raise(self._lib.pkv_allocator_free_seq(self._h, seq), "pkv_allocator_free_seq")

    def block_table(self, seq, width):
        row = self._np.empty(width, dtype=self._np.int32)
        _raise(self._lib.pkv_allocator_block_table(self._h, seq, _np_ptr(row), width),
               "pkv_allocator_block_table")
        return row

    def decode_batch(self, seqs, width):
        """One new token per sequence: (slot_mapping [B] int64, block_tables
        [B, width] int32, context_lens [B] int32)."""
        np = self._np
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        B = seqs.size
        slots = np.empty(B, dtype=np.int64)
        tables = np.empty((B, width), dtype=np.int32)
        lens = np.empty(B, dtype=np.int32)
        _raise(self._lib.pkv_allocator_build_decode_batch(
            self._h, _np_ptr(seqs), B, width, _np_ptr(slots), _np_ptr(tables), _np_ptr(lens)),
            "pkv_allocator_build_decode_batch")
        return slots, tables, lens

    def prefill_batch(self, seqs, chunk_lens, width):
        """One chunk per sequence: (query_start [B + 1], slot_mapping
        [total] int64, block_tables [B, width], context_lens [B])."""
        np = self._np
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        chunk_lens = np.ascontiguousarray(chunk_lens, dtype=np.int32)
        B = seqs.size
        if chunk_lens.size != B:
            raise ValueError("one chunk length per sequence")
        qs = np.empty(B + 1, dtype=np.int32)
        slots = np.empty(int(chunk_lens.astype(np.int64).sum()) if B else 0, dtype=np.int64)
        tables = np.empty((B, width), dtype=np.int32)
        lens = np.empty(B, dtype=np.int32)
        _raise(self._lib.pkv_allocator_build_prefill_batch(
            self._h, _np_ptr(seqs), _np_ptr(chunk_lens), B, width, _np_ptr(qs), _np_ptr(slots),
            _np_ptr(tables), _np_ptr(lens)), "pkv_allocator_build_prefill_batch")
        return qs, slots, tables, lens
