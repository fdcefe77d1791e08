"""paged_kv_cache_390_amd -- the paged-KV-cache hot path on AMD MI355X.

A thin binding over the C ABI of ``libpa.so`` (declared in ``include/pa.h``):
argument checks and marshalling only.  Every step of the path runs in the
library: the HIP kernels for the slot-mapped cache write, paged decode
attention and block copy, and the C++ block manager that builds tables,
slots and copy-on-write pairs.  PyTorch only provides device memory and the
current HIP stream.  There is no fallback: if the library is not built, every
call raises.

Functions carry the C names: ``pa_reshape_and_cache``, ``pa_decode``, ``pa_decode_append``,
``pa_decode_order``, ``pa_decode_workspace_size``, ``pa_prefill``, ``pa_prefill_workspace_size``, ``pa_copy_blocks``, ``pa_swap_blocks``;
``BlockManager`` wraps the ``pa_bm_*`` calls.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK = 0
PA_COW = 1
PA_ERR_INVALID = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_HIP = -3
PA_ERR_OOM = -4
PA_ERR_STATE = -5
PA_DTYPE_F16 = 0
PA_SWAP_OUT = 0
PA_SWAP_IN = 1

_lib = None


class PAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class OutOfBlocks(PAError):
    pass


class BadState(PAError):
    pass


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m paged_kv_cache_390_amd.build` "
                           "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "pa_last_error": ([], ctypes.c_char_p),
        "pa_reshape_and_cache": ([P, P, i64, P, i32, P, P, i32, i32, i32, i32, i32, P], ctypes.c_int),
        "pa_decode": ([P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, f32, i32, i32, P, sz, P, i32, P],
                      ctypes.c_int),
        "pa_decode_append": ([P, P, P, P, i64, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, f32, i32, i32, P,
                              sz, P, i32, P], ctypes.c_int),
        "pa_prefill": ([P, P, i32, P, P, P, i32, P, P, i32, i32, i32, i32, i32, i32, f32, i32, P, sz, P, i32, P],
                       ctypes.c_int),
        "pa_decode_order": ([P, P, i32, i32, P], ctypes.c_int),
        "pa_decode_noalloc": ([P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, f32, i32, i32, P, i32, P],
                              ctypes.c_int),
        "pa_prefill_append": ([P, P, i32, P, P, i64, P, P, P, i32, P, P, i32, i32, i32, i32, i32, i32, f32, i32, P, sz,
                               P, i32, P], ctypes.c_int),
        "pa_prefill_workspace_size": ([i32, i32, i32, i32, i32, i32, i32, i32], sz),
        "pa_decode_workspace_size": ([i32, i32, i32, i32, i32, i32, i32], sz),
        "pa_decode_default_partition": ([i32, i32, i32, i32, i32, i32], i32),
        "pa_copy_blocks": ([P, P, i32, P, i32, i32, i64, i32, P], ctypes.c_int),
        "pa_swap_blocks": ([P, P, i32, P, i32, i32, i32, i64, i32, i32, P], ctypes.c_int),
        "pa_bench_stream_read_groups": ([sz], i64),
        "pa_bench_stream_read": ([P, sz, P, P], ctypes.c_int),
        "pa_bench_block_read": ([P, P, P, i32, P, i32, i32, i32, i32, i32, P, P], ctypes.c_int),
        "pa_bm_create": ([i32, i32], P),
        "pa_bm_create_with_host": ([i32, i32, i32], P),
        "pa_bm_swap_out": ([P, P, i32, P, i32, P], ctypes.c_int),
        "pa_bm_swap_in": ([P, P, i32, P, i32, P], ctypes.c_int),
        "pa_bm_is_swapped": ([P, i64], i32),
        "pa_bm_host_refcount": ([P, i32], i32),
        "pa_bm_host_free_list": ([P, P, i32], i32),
        "pa_bm_seq_table": ([P, i64, P, i32], i32),
        "pa_bm_add_sequence_cached": ([P, i64, P, i32, P, P], ctypes.c_int),
        "pa_bm_num_cached_blocks": ([P], i32),
        "pa_bm_destroy": ([P], None),
        "pa_bm_add_sequence": ([P, i64, i32, P], ctypes.c_int),
        "pa_bm_set_table": ([P, i64, P, i32, i32], ctypes.c_int),
        "pa_bm_fork": ([P, i64, i64], ctypes.c_int),
        "pa_bm_append_token": ([P, i64, P, P, P], ctypes.c_int),
        "pa_bm_append_tokens": ([P, P, i32, P, P, P, P], ctypes.c_int),
        "pa_bm_free_sequence": ([P, i64], ctypes.c_int),
        "pa_bm_get_tables": ([P, P, i32, P, i32, P], ctypes.c_int),
        "pa_bm_get_slots": ([P, i64, i32, i32, P], ctypes.c_int),
        "pa_bm_refcount": ([P, i32], i32),
        "pa_bm_num_free": ([P], i32),
        "pa_bm_free_list": ([P, P, i32], i32),
        "pa_bm_seq_len": ([P, i64], i32),
        "pa_bm_seq_blocks": ([P, i64], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def last_error() -> str:
    return lib().pa_last_error().decode()


def _check(rc: int, what: str) -> int:
    if rc >= 0:
        return rc
    msg = last_error()
    if rc == PA_ERR_OOM:
        raise OutOfBlocks(rc, msg or what)
    if rc == PA_ERR_STATE:
        raise BadState(rc, msg or what)
    raise PAError(rc, msg or what)


# ---------------------------------------------------------------------------
# device calls
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dev_tensor(t, name, dtype, ndim=None, contiguous=True):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device (HIP) tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got shape {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def pa_reshape_and_cache(key, value, slot_mapping, k_cache, v_cache) -> None:
    """Write key/value [T, Hkv, D] (fp16, head_dim contiguous, any token
    stride) into k_cache/v_cache [NB, Hkv, B, D] at slot_mapping[T] (int64)."""
    torch = _torch()
    _dev_tensor(k_cache, "k_cache", torch.float16, 4)
    _dev_tensor(v_cache, "v_cache", torch.float16, 4)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    NB, Hkv, B, D = k_cache.shape
    _dev_tensor(key, "key", torch.float16, 3, contiguous=False)
    _dev_tensor(value, "value", torch.float16, 3, contiguous=False)
    _dev_tensor(slot_mapping, "slot_mapping", torch.int64, 1)
    T = key.shape[0]
    if tuple(key.shape) != (T, Hkv, D) or tuple(value.shape) != (T, Hkv, D):
        raise ValueError(f"key/value must be [T, {Hkv}, {D}]")
    if key.stride() != value.stride() or key.stride(2) != 1 or key.stride(1) != D:
        raise ValueError("key and value need equal strides with contiguous [Hkv, D] rows")
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping length != number of tokens")
    _check(lib().pa_reshape_and_cache(key.data_ptr(), value.data_ptr(), key.stride(0),
                                      slot_mapping.data_ptr(), T, k_cache.data_ptr(),
                                      v_cache.data_ptr(), NB, Hkv, B, D, PA_DTYPE_F16,
                                      _stream(k_cache.device)), "pa_reshape_and_cache")


def pa_decode_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                             block_size: int, max_context_len: int, partition_size: int = 0) -> int:
    n = lib().pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                       max_context_len, partition_size)
    if n == ctypes.c_size_t(-1).value:
        raise PAError(PA_ERR_INVALID, "pa_decode_workspace_size: invalid arguments")
    return n


def pa_decode_default_partition(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                                block_size: int, max_context_len: int) -> int:
    p = lib().pa_decode_default_partition(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                          max_context_len)
    if p < 0:
        raise PAError(PA_ERR_INVALID, "pa_decode_default_partition: invalid arguments")
    return p


def _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, block_size, max_context_len,
                 partition_size, workspace, seq_order):
    """Checks shared by pa_decode and pa_decode_append; returns the sizes
    and the workspace / order pointers."""
    torch = _torch()
    _dev_tensor(k_cache, "k_cache", torch.float16, 4)
    _dev_tensor(v_cache, "v_cache", torch.float16, 4)
    NB, Hkv, B, D = k_cache.shape
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if block_size is not None and block_size != B:
        raise ValueError(f"block_size {block_size} != cache block dimension {B}")
    _dev_tensor(q, "q", torch.float16, 3)
    _dev_tensor(out, "out", torch.float16, 3)
    S, H, Dq = q.shape
    if Dq != D or tuple(out.shape) != (S, H, D):
        raise ValueError("q/out must be [S, H, head_dim]")
    _dev_tensor(block_tables, "block_tables", torch.int32, 2)
    _dev_tensor(context_lens, "context_lens", torch.int32, 1)
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables/context_lens must have one row per sequence")
    W = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = W * B
    need = pa_decode_workspace_size(S, H, Hkv, D, B, max_context_len, partition_size)
    ws_ptr, ws_bytes = 0, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _dev_tensor(workspace, "workspace", torch.uint8, 1)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    order_ptr = None
    if seq_order is not None:
        _dev_tensor(seq_order, "seq_order", torch.int32, 1)
        if seq_order.shape[0] != S:
            raise ValueError("seq_order must have one entry per sequence")
        order_ptr = seq_order.data_ptr()
    return S, H, Hkv, D, B, NB, W, int(max_context_len), ws_ptr, ws_bytes, order_ptr


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
              block_size: Optional[int] = None, max_context_len: Optional[int] = None,
              partition_size: int = 0, workspace=None, seq_order=None) -> None:
    """out[S, H, D] = softmax(scale * K q) V for each sequence over its first
    context_lens[s] cached tokens, found through block_tables[S, W].

    max_context_len defaults to W * block_size (a bound known without reading
    context_lens back).  workspace (a uint8 device tensor) is allocated from
    torch's caching allocator when needed and not given.  seq_order (int32
    device tensor [S], from pa_decode_order) is the dispatch order shared by
    the layers of a step; without it pa_decode computes one per call."""
    S, H, Hkv, D, B, NB, W, mcl, ws_ptr, ws_bytes, order_ptr = _decode_args(
        out, q, k_cache, v_cache, block_tables, context_lens, block_size, max_context_len, partition_size,
        workspace, seq_order)
    _check(lib().pa_decode(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                           block_tables.data_ptr(), W, context_lens.data_ptr(), S, H, Hkv, D, B, NB,
                           float(scale), mcl, int(partition_size), ws_ptr, ws_bytes,
                           order_ptr, PA_DTYPE_F16, _stream(q.device)), "pa_decode")


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                      block_size: Optional[int] = None, max_context_len: Optional[int] = None,
                      partition_size: int = 0, seq_order=None) -> None:
    """pa_decode with the workspace held by the library (one fixed-size
    device array per GPU): allocates nothing, for callers that cannot.
    Raises PAError (PA_ERR_INVALID) when the sizes need more workspace than
    that array holds.  Calls that may overlap on one GPU share the array and
    must be serialised by the caller."""
    torch = _torch()
    _dev_tensor(k_cache, "k_cache", torch.float16, 4)
    _dev_tensor(v_cache, "v_cache", torch.float16, 4)
    NB, Hkv, B, D = k_cache.shape
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if block_size is not None and block_size != B:
        raise ValueError(f"block_size {block_size} != cache block dimension {B}")
    _dev_tensor(q, "q", torch.float16, 3)
    _dev_tensor(out, "out", torch.float16, 3)
    S, H, Dq = q.shape
    if Dq != D or tuple(out.shape) != (S, H, D):
        raise ValueError("q/out must be [S, H, head_dim]")
    _dev_tensor(block_tables, "block_tables", torch.int32, 2)
    _dev_tensor(context_lens, "context_lens", torch.int32, 1)
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables/context_lens must have one row per sequence")
    W = block_tables.shape[1]
    mcl = W * B if max_context_len is None else int(max_context_len)
    order_ptr = None
    if seq_order is not None:
        _dev_tensor(seq_order, "seq_order", torch.int32, 1)
        if seq_order.shape[0] != S:
            raise ValueError("seq_order must have one entry per sequence")
        order_ptr = seq_order.data_ptr()
    _check(lib().pa_decode_noalloc(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                   block_tables.data_ptr(), W, context_lens.data_ptr(), S, H, Hkv, D, B, NB,
                                   float(scale), mcl, int(partition_size), order_ptr, PA_DTYPE_F16,
                                   _stream(q.device)), "pa_decode_noalloc")


def pa_decode_append(out, q, key, value, k_cache, v_cache, block_tables, context_lens, scale: float,
                     block_size: Optional[int] = None, max_context_len: Optional[int] = None,
                     partition_size: int = 0, workspace=None, seq_order=None) -> None:
    """pa_reshape_and_cache of one new token per sequence followed by
    pa_decode, in one call: key/value [S, Hkv, D] (fp16, head_dim
    contiguous, any 16-byte-aligned token stride) hold sequence s's token at
    position context_lens[s] - 1; it is written into the cache at that
    position's slot of block_tables and attended to with the cached ones."""
    torch = _torch()
    S, H, Hkv, D, B, NB, W, mcl, ws_ptr, ws_bytes, order_ptr = _decode_args(
        out, q, k_cache, v_cache, block_tables, context_lens, block_size, max_context_len, partition_size,
        workspace, seq_order)
    _dev_tensor(key, "key", torch.float16, 3, contiguous=False)
    _dev_tensor(value, "value", torch.float16, 3, contiguous=False)
    if tuple(key.shape) != (S, Hkv, D) or tuple(value.shape) != (S, Hkv, D):
        raise ValueError(f"key/value must be [{S}, {Hkv}, {D}]")
    if key.stride() != value.stride() or key.stride(2) != 1 or key.stride(1) != D:
        raise ValueError("key and value need equal strides with contiguous [Hkv, D] rows")
    _check(lib().pa_decode_append(out.data_ptr(), q.data_ptr(), key.data_ptr(), value.data_ptr(), key.stride(0),
                                  k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), W,
                                  context_lens.data_ptr(), S, H, Hkv, D, B, NB, float(scale), mcl,
                                  int(partition_size), ws_ptr, ws_bytes, order_ptr, PA_DTYPE_F16,
                                  _stream(q.device)), "pa_decode_append")


def pa_decode_order(context_lens, max_context_len: int, out=None):
    """Longest-first dispatch order of the sequences (int32 device tensor
    [S]) for the seq_order of pa_decode and pa_prefill; compute it once per
    step, after context_lens is final, and pass it to every layer."""
    torch = _torch()
    _dev_tensor(context_lens, "context_lens", torch.int32, 1)
    S = context_lens.shape[0]
    if out is None:
        out = torch.empty(S, dtype=torch.int32, device=context_lens.device)
    _dev_tensor(out, "out", torch.int32, 1)
    if out.shape[0] != S:
        raise ValueError("out must have one entry per sequence")
    _check(lib().pa_decode_order(out.data_ptr(), context_lens.data_ptr(), S, int(max_context_len),
                                 _stream(context_lens.device)), "pa_decode_order")
    return out


def pa_prefill_workspace_size(num_tokens: int, num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                              block_size: int, max_blocks_per_seq: int, max_query_len: int) -> int:
    n = lib().pa_prefill_workspace_size(num_tokens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                        max_blocks_per_seq, max_query_len)
    if n == ctypes.c_size_t(-1).value:
        raise PAError(PA_ERR_INVALID, "pa_prefill_workspace_size: invalid arguments")
    return n


def _prefill_args(out, q, k_cache, v_cache, block_tables, context_lens, query_start, max_query_len, workspace,
                  split, seq_order):
    torch = _torch()
    _dev_tensor(k_cache, "k_cache", torch.float16, 4)
    _dev_tensor(v_cache, "v_cache", torch.float16, 4)
    NB, Hkv, B, D = k_cache.shape
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    _dev_tensor(q, "q", torch.float16, 3)
    _dev_tensor(out, "out", torch.float16, 3)
    T, H, Dq = q.shape
    if Dq != D or tuple(out.shape) != (T, H, D):
        raise ValueError("q/out must be [T, H, head_dim]")
    _dev_tensor(block_tables, "block_tables", torch.int32, 2)
    _dev_tensor(context_lens, "context_lens", torch.int32, 1)
    _dev_tensor(query_start, "query_start", torch.int32, 1)
    S = context_lens.shape[0]
    if block_tables.shape[0] != S or query_start.shape[0] != S + 1:
        raise ValueError("block_tables / context_lens / query_start disagree on the number of sequences")
    if max_query_len is None:
        max_query_len = T
    ws_ptr, ws_bytes = None, 0
    if split:
        need = pa_prefill_workspace_size(T, S, H, Hkv, D, B, block_tables.shape[1], int(max_query_len))
        if need:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            _dev_tensor(workspace, "workspace", torch.uint8, 1)
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    order_ptr = None
    if seq_order is not None:
        _dev_tensor(seq_order, "seq_order", torch.int32, 1)
        if seq_order.shape[0] != S:
            raise ValueError("seq_order must have one entry per sequence")
        order_ptr = seq_order.data_ptr()
    return T, S, H, Hkv, D, B, NB, int(max_query_len), ws_ptr, ws_bytes, order_ptr


def pa_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float,
               max_query_len: Optional[int] = None, workspace=None, split: bool = True, seq_order=None) -> None:
    """Causal attention of the packed new tokens q[T, H, D] over the paged
    cache: sequence s's rows query_start[s] .. query_start[s+1]-1 are its
    last m tokens (K/V already cached), row i at position context_lens[s] -
    m + i.  max_query_len defaults to T.  workspace (uint8 device tensor)
    is allocated when the batch is small enough for the context to be split
    and none is given; split=False passes none (no split).  seq_order (int32
    device [S], from pa_decode_order over context_lens, once per step)
    dispatches the sequences longest first; the result is the same."""
    T, S, H, Hkv, D, B, NB, mq, ws_ptr, ws_bytes, order_ptr = _prefill_args(
        out, q, k_cache, v_cache, block_tables, context_lens, query_start, max_query_len, workspace, split,
        seq_order)
    _check(lib().pa_prefill(out.data_ptr(), q.data_ptr(), T, k_cache.data_ptr(), v_cache.data_ptr(),
                            block_tables.data_ptr(), block_tables.shape[1], context_lens.data_ptr(),
                            query_start.data_ptr(), S, H, Hkv, D, B, NB, float(scale), mq,
                            ws_ptr, ws_bytes, order_ptr, PA_DTYPE_F16, _stream(q.device)), "pa_prefill")


def pa_prefill_append(out, q, key, value, k_cache, v_cache, block_tables, context_lens, query_start, scale: float,
                      max_query_len: Optional[int] = None, workspace=None, split: bool = True,
                      seq_order=None) -> None:
    """pa_reshape_and_cache of the new tokens followed by pa_prefill, in one
    call: key/value [T, Hkv, D] (fp16, head_dim contiguous, any 16-byte
    aligned token stride) hold the K/V of the token in the same row of q; each
    is written into the cache at its position's slot of block_tables and
    attended to with the cached ones."""
    torch = _torch()
    T, S, H, Hkv, D, B, NB, mq, ws_ptr, ws_bytes, order_ptr = _prefill_args(
        out, q, k_cache, v_cache, block_tables, context_lens, query_start, max_query_len, workspace, split,
        seq_order)
    _dev_tensor(key, "key", torch.float16, 3, contiguous=False)
    _dev_tensor(value, "value", torch.float16, 3, contiguous=False)
    if tuple(key.shape) != (T, Hkv, D) or tuple(value.shape) != (T, Hkv, D):
        raise ValueError(f"key/value must be [{T}, {Hkv}, {D}]")
    if key.stride() != value.stride() or key.stride(2) != 1 or key.stride(1) != D:
        raise ValueError("key and value need equal strides with contiguous [Hkv, D] rows")
    _check(lib().pa_prefill_append(out.data_ptr(), q.data_ptr(), T, key.data_ptr(), value.data_ptr(), key.stride(0),
                                   k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                                   block_tables.shape[1], context_lens.data_ptr(), query_start.data_ptr(), S, H, Hkv,
                                   D, B, NB, float(scale), mq, ws_ptr, ws_bytes, order_ptr, PA_DTYPE_F16,
                                   _stream(q.device)),
           "pa_prefill_append")


def pa_copy_blocks(k_caches: Sequence, v_caches: Sequence, src_dst_pairs) -> None:
    """For every layer, copy block pairs[i, 0] onto block pairs[i, 1] (K and
    V).  src_dst_pairs: int64 device tensor [N, 2]."""
    torch = _torch()
    if len(k_caches) != len(v_caches):
        raise ValueError("k_caches and v_caches differ in length")
    _dev_tensor(src_dst_pairs, "src_dst_pairs", torch.int64, 2)
    if src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be [N, 2]")
    N = src_dst_pairs.shape[0]
    L = len(k_caches)
    if N == 0 or L == 0:
        return
    shape = k_caches[0].shape
    for i, t in enumerate(list(k_caches) + list(v_caches)):
        _dev_tensor(t, f"cache[{i}]", torch.float16, 4)
        if t.shape != shape:
            raise ValueError("all caches must share one shape")
    NB = shape[0]
    block_elems = int(shape[1] * shape[2] * shape[3])
    kp = (ctypes.c_void_p * L)(*[t.data_ptr() for t in k_caches])
    vp = (ctypes.c_void_p * L)(*[t.data_ptr() for t in v_caches])
    _check(lib().pa_copy_blocks(ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(vp, ctypes.c_void_p), L,
                                src_dst_pairs.data_ptr(), N, NB, block_elems, PA_DTYPE_F16,
                                _stream(src_dst_pairs.device)), "pa_copy_blocks")


def pa_swap_blocks(dev_caches: Sequence, host_caches: Sequence, pairs, direction: int) -> None:
    """Copy whole blocks between device caches and pinned host caches:
    direction PA_SWAP_OUT copies device block pairs[i, 0] to host block
    pairs[i, 1] in every cache, PA_SWAP_IN host pairs[i, 0] to device
    pairs[i, 1].  dev_caches[i] / host_caches[i]: fp16 tensors of one block
    shape (list K and V of every layer); pairs: int64 device tensor [N, 2]."""
    torch = _torch()
    if len(dev_caches) != len(host_caches):
        raise ValueError("dev_caches and host_caches differ in length")
    _dev_tensor(pairs, "pairs", torch.int64, 2)
    if pairs.shape[1] != 2:
        raise ValueError("pairs must be [N, 2]")
    N = pairs.shape[0]
    C = len(dev_caches)
    if N == 0 or C == 0:
        return
    bshape = tuple(dev_caches[0].shape[1:])
    for i, t in enumerate(dev_caches):
        _dev_tensor(t, f"dev_caches[{i}]", torch.float16)
        if tuple(t.shape[1:]) != bshape or t.shape[0] != dev_caches[0].shape[0]:
            raise ValueError("all device caches must share one shape")
    for i, t in enumerate(host_caches):
        if not isinstance(t, torch.Tensor) or t.device.type != "cpu" or not t.is_pinned():
            raise ValueError(f"host_caches[{i}]: must be a pinned CPU tensor")
        if t.dtype != torch.float16 or not t.is_contiguous():
            raise TypeError(f"host_caches[{i}]: must be contiguous float16")
        if tuple(t.shape[1:]) != bshape or t.shape[0] != host_caches[0].shape[0]:
            raise ValueError("all host caches must share one shape, with the device block shape")
    block_elems = int(np.prod(bshape))
    dp = (ctypes.c_void_p * C)(*[t.data_ptr() for t in dev_caches])
    hp = (ctypes.c_void_p * C)(*[t.data_ptr() for t in host_caches])
    _check(lib().pa_swap_blocks(ctypes.cast(dp, ctypes.c_void_p), ctypes.cast(hp, ctypes.c_void_p), C,
                                pairs.data_ptr(), N, dev_caches[0].shape[0], host_caches[0].shape[0],
                                block_elems, int(direction), PA_DTYPE_F16, _stream(pairs.device)),
           "pa_swap_blocks")


# ---------------------------------------------------------------------------
# host block manager
# ---------------------------------------------------------------------------
def pa_bench_stream_read(buf, sink=None):
    """Measurement aid (include/pa_bench.h): read every byte of the
    contiguous device tensor `buf` once; returns the sink tensor (one uint32
    word per MiB, as int32)."""
    torch = _torch()
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    groups = lib().pa_bench_stream_read_groups(nbytes)
    if sink is None:
        sink = torch.empty(max(groups, 1), dtype=torch.int32, device=buf.device)
    _dev_tensor(sink, "sink", torch.int32, 1)
    if sink.numel() < groups:
        raise ValueError(f"sink needs {groups} words")
    _check(lib().pa_bench_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), _stream(buf.device)),
           "pa_bench_stream_read")
    return sink


def pa_bench_block_read(k_cache, v_cache, block_tables, context_lens, sink=None):
    """Measurement aid (include/pa_bench.h): the decode access pattern --
    the K and V slabs of every block of every (sequence, KV head) -- with
    no arithmetic; returns the sink tensor (one word per pair)."""
    torch = _torch()
    _dev_tensor(k_cache, "k_cache", torch.float16, 4)
    _dev_tensor(v_cache, "v_cache", torch.float16, 4)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    NB, Hkv, B, D = k_cache.shape
    _dev_tensor(block_tables, "block_tables", torch.int32, 2)
    _dev_tensor(context_lens, "context_lens", torch.int32, 1)
    S, W = block_tables.shape
    if context_lens.shape[0] != S:
        raise ValueError("context_lens must have one entry per sequence")
    if sink is None:
        sink = torch.empty(max(S * Hkv, 1), dtype=torch.int32, device=k_cache.device)
    _dev_tensor(sink, "sink", torch.int32, 1)
    if sink.numel() < S * Hkv:
        raise ValueError(f"sink needs {S * Hkv} words")
    _check(lib().pa_bench_block_read(k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), W,
                                     context_lens.data_ptr(), S, Hkv, D, B, NB, sink.data_ptr(),
                                     _stream(k_cache.device)), "pa_bench_block_read")
    return sink


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class BlockManager:
    """Owner of a ``pa_bm`` handle (host memory only)."""

    def __init__(self, num_blocks: int, block_size: int, num_host_blocks: int = 0):
        self._L = lib()
        h = self._L.pa_bm_create_with_host(num_blocks, block_size, num_host_blocks)
        if not h:
            raise PAError(PA_ERR_INVALID, last_error())
        self._h = ctypes.c_void_p(h)
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.num_host_blocks = num_host_blocks

    def close(self):
        if getattr(self, "_h", None):
            self._L.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_sequence(self, seq: int, n_tokens: int) -> np.ndarray:
        slots = np.empty(max(n_tokens, 0), dtype=np.int64)
        _check(self._L.pa_bm_add_sequence(self._h, seq, n_tokens, slots.ctypes.data if n_tokens else None),
               "add_sequence")
        return slots

    def add_sequence_cached(self, seq: int, token_ids) -> Tuple[np.ndarray, int]:
        """New sequence from its prompt's token ids, sharing the blocks of a
        cached common prefix; returns (slots of every position, number of
        leading positions whose K/V are already cached)."""
        t = _i32(token_ids)
        slots = np.empty(max(t.size, 0), dtype=np.int64)
        nc = ctypes.c_int32()
        _check(self._L.pa_bm_add_sequence_cached(self._h, seq, t.ctypes.data if t.size else None, t.size,
                                                 slots.ctypes.data if t.size else None, ctypes.byref(nc)),
               "add_sequence_cached")
        return slots, nc.value

    def num_cached_blocks(self) -> int:
        return self._L.pa_bm_num_cached_blocks(self._h)

    def set_table(self, seq: int, blocks, n_tokens: int) -> None:
        b = _i32(blocks)
        _check(self._L.pa_bm_set_table(self._h, seq, b.ctypes.data if b.size else None, b.size, n_tokens),
               "set_table")

    def fork(self, parent: int, child: int) -> None:
        _check(self._L.pa_bm_fork(self._h, parent, child), "fork")

    def append_token(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        slot, src, dst = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        rc = _check(self._L.pa_bm_append_token(self._h, seq, ctypes.byref(slot), ctypes.byref(src),
                                               ctypes.byref(dst)), "append_token")
        return slot.value, ((src.value, dst.value) if rc == PA_COW else None)

    def append_tokens(self, seqs) -> Tuple[np.ndarray, np.ndarray]:
        """Batched append: returns (slots[n], cow_pairs[k, 2])."""
        s = _i64(seqs)
        n = s.size
        slots = np.empty(n, dtype=np.int64)
        pairs = np.empty((max(n, 1), 2), dtype=np.int64)
        ncow, ndone = ctypes.c_int32(), ctypes.c_int32()
        _check(self._L.pa_bm_append_tokens(self._h, s.ctypes.data, n, slots.ctypes.data, pairs.ctypes.data,
                                           ctypes.byref(ncow), ctypes.byref(ndone)), "append_tokens")
        return slots, pairs[:ncow.value]

    def free_sequence(self, seq: int) -> None:
        _check(self._L.pa_bm_free_sequence(self._h, seq), "free_sequence")

    def get_tables(self, seqs, max_blocks: int, out: Optional[np.ndarray] = None,
                   lens_out: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
        s = _i64(seqs)
        n = s.size
        tables = out if out is not None else np.empty((n, max_blocks), dtype=np.int32)
        lens = lens_out if lens_out is not None else np.empty(n, dtype=np.int32)
        if tables.dtype != np.int32 or tables.shape != (n, max_blocks) or not tables.flags.c_contiguous:
            raise ValueError("tables buffer must be int32 [n, max_blocks], C-contiguous")
        if lens.dtype != np.int32 or lens.shape != (n,):
            raise ValueError("lens buffer must be int32 [n]")
        _check(self._L.pa_bm_get_tables(self._h, s.ctypes.data, n, tables.ctypes.data, max_blocks,
                                        lens.ctypes.data), "get_tables")
        return tables, lens

    def get_slots(self, seq: int, pos_begin: int, count: int) -> np.ndarray:
        out = np.empty(count, dtype=np.int64)
        _check(self._L.pa_bm_get_slots(self._h, seq, pos_begin, count, out.ctypes.data if count else None),
               "get_slots")
        return out

    def refcount(self, blk: int) -> int:
        return self._L.pa_bm_refcount(self._h, blk)

    def num_free(self) -> int:
        return self._L.pa_bm_num_free(self._h)

    def free_list(self) -> List[int]:
        n = self._L.pa_bm_free_list(self._h, None, 0)
        out = np.empty(max(n, 1), dtype=np.int32)
        self._L.pa_bm_free_list(self._h, out.ctypes.data, n)
        return out[:n].tolist()

    def _move(self, fn, seqs) -> np.ndarray:
        s = _i64(seqs)
        cap = 0
        for q in s.tolist():
            cap += max(self._L.pa_bm_seq_table(self._h, q, None, 0), 0)
        pairs = np.empty((max(cap, 1), 2), dtype=np.int64)
        n = ctypes.c_int32()
        _check(fn(self._h, s.ctypes.data if s.size else None, s.size, pairs.ctypes.data, cap, ctypes.byref(n)),
               "swap")
        return pairs[:n.value]

    def swap_out(self, seqs) -> np.ndarray:
        """Move a group to the host pool; returns (device id, host id) rows."""
        return self._move(self._L.pa_bm_swap_out, seqs)

    def swap_in(self, seqs) -> np.ndarray:
        """Move a swapped-out group back; returns (host id, device id) rows."""
        return self._move(self._L.pa_bm_swap_in, seqs)

    def is_swapped(self, seq: int) -> bool:
        r = self._L.pa_bm_is_swapped(self._h, seq)
        if r < 0:
            raise BadState(PA_ERR_STATE, f"unknown sequence {seq}")
        return bool(r)

    def host_refcount(self, hblk: int) -> int:
        return self._L.pa_bm_host_refcount(self._h, hblk)

    def host_free_list(self) -> List[int]:
        n = self._L.pa_bm_host_free_list(self._h, None, 0)
        out = np.empty(max(n, 1), dtype=np.int32)
        self._L.pa_bm_host_free_list(self._h, out.ctypes.data, n)
        return out[:n].tolist()

    def raw_table(self, seq: int) -> List[int]:
        """The table as stored: device ids, or host ids while swapped out."""
        n = self._L.pa_bm_seq_table(self._h, seq, None, 0)
        if n < 0:
            raise BadState(PA_ERR_STATE, f"unknown sequence {seq}")
        out = np.empty(max(n, 1), dtype=np.int32)
        self._L.pa_bm_seq_table(self._h, seq, out.ctypes.data, n)
        return out[:n].tolist()

    def seq_len(self, seq: int) -> int:
        return self._L.pa_bm_seq_len(self._h, seq)

    def table(self, seq: int) -> List[int]:
        nb = self._L.pa_bm_seq_blocks(self._h, seq)
        if nb < 0:
            raise BadState(PA_ERR_STATE, f"unknown sequence {seq}")
        t, _ = self.get_tables([seq], nb)
        return t[0].tolist()
