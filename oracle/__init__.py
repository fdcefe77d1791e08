"""Oracle for the paged-KV-cache hot path — TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the cpu_baseline leg of
``bench.py`` may import, call, link or execute anything in this package.  The
product (``paged_kv_cache_390_amd``) never imports it, and the two share no
code: the oracle is a plain fp64 C implementation (``pa_oracle.c``) plus a
Python model of the block manager (``block_manager.py``) and the pages'
closed forms (``closed_forms.py``).

Functions here marshal numpy arrays into the C oracle.  fp16 data is passed as
numpy float16 arrays and read bit for bit; attention results come back as
float64.

Parity status: every function here is pinned by a CPU test in
``tests/test_oracle_*.py`` (closed forms, the pages' worked examples, a
library attention routine, brute force and invariances).
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib() -> ctypes.CDLL:
    """Load oracle/liboracle.so, compiling it with gcc if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
        _build.build()
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    L.oracle_half_to_double.restype = f64
    L.oracle_decode.argtypes = [P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i64, f64, i32]
    L.oracle_decode.restype = ctypes.c_int
    L.oracle_prefill.argtypes = [P, P, P, P, P, i32, P, P, i32, i32, i32, i32, i32, i64, f64, i32]
    L.oracle_prefill.restype = ctypes.c_int
    L.oracle_attention_contig.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, f64, i32]
    L.oracle_attention_contig.restype = ctypes.c_int
    L.oracle_reshape_and_cache.argtypes = [P, P, i64, P, i32, P, P, i64, i32, i32, i32]
    L.oracle_reshape_and_cache.restype = ctypes.c_int
    L.oracle_copy_blocks.argtypes = [P, P, i32, P, i32, i64, i64]
    L.oracle_copy_blocks.restype = ctypes.c_int
    _lib = L
    return L


def default_threads() -> int:
    """Threads the oracle uses: the CPUs this process may run on, capped by
    OMP_NUM_THREADS when it is set (the machine's CPU share for one job),
    else by 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "") or 16)
    except ValueError:
        cap = 16
    return max(1, min(n, cap))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _need(a: np.ndarray, dtype, name: str) -> np.ndarray:
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"{name}: expected {np.dtype(dtype)}, got {a.dtype}")
    if not a.flags.c_contiguous:
        raise ValueError(f"{name}: must be C-contiguous")
    return a


def half_to_double(bits: int) -> float:
    return lib().oracle_half_to_double(int(bits) & 0xFFFF)


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
           block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
           nthreads: int | None = None) -> np.ndarray:
    """fp64 attention of q[S, H, D] over the paged caches [NB, Hkv, B, D]."""
    _need(q, np.float16, "q")
    _need(k_cache, np.float16, "k_cache")
    _need(v_cache, np.float16, "v_cache")
    _need(block_tables, np.int32, "block_tables")
    _need(context_lens, np.int32, "context_lens")
    S, H, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if block_tables.ndim != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("table / length shape mismatch")
    out = np.zeros((S, H, D), dtype=np.float64)
    rc = lib().oracle_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                             _ptr(block_tables), block_tables.shape[1],
                             _ptr(context_lens), S, H, Hkv, D, B, NB,
                             float(scale), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_decode failed: {rc}")
    return out


def prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
            block_tables: np.ndarray, context_lens: np.ndarray, query_start: np.ndarray,
            scale: float, nthreads: int | None = None) -> np.ndarray:
    """fp64 causal attention of the packed new tokens q[T, H, D] over the
    paged caches: sequence s's rows query_start[s] .. query_start[s+1]-1 are
    its last m tokens, row i at position context_lens[s] - m + i, attending
    to positions 0 .. that position."""
    _need(q, np.float16, "q")
    _need(k_cache, np.float16, "k_cache")
    _need(v_cache, np.float16, "v_cache")
    _need(block_tables, np.int32, "block_tables")
    _need(context_lens, np.int32, "context_lens")
    _need(query_start, np.int32, "query_start")
    T, H, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    S = context_lens.shape[0]
    if D2 != D or v_cache.shape != k_cache.shape or block_tables.shape[0] != S or \
       query_start.shape != (S + 1,) or query_start[-1] != T or query_start[0] != 0:
        raise ValueError("shape mismatch")
    out = np.zeros((T, H, D), dtype=np.float64)
    rc = lib().oracle_prefill(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                              block_tables.shape[1], _ptr(context_lens), _ptr(query_start), S, H, Hkv, D,
                              B, NB, float(scale), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_prefill failed: {rc}")
    return out


def attention_contig(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     seq_start: np.ndarray, lens: np.ndarray, scale: float,
                     nthreads: int | None = None) -> np.ndarray:
    """fp64 attention of q[S, H, D] over contiguous k/v [tokens, Hkv, D];
    sequence s owns rows seq_start[s] .. seq_start[s] + lens[s] - 1."""
    _need(q, np.float16, "q")
    _need(k, np.float16, "k")
    _need(v, np.float16, "v")
    _need(seq_start, np.int64, "seq_start")
    _need(lens, np.int32, "lens")
    S, H, D = q.shape
    T, Hkv, D2 = k.shape
    if D2 != D or v.shape != k.shape or seq_start.shape != (S,) or lens.shape != (S,):
        raise ValueError("shape mismatch")
    if S and (np.any(seq_start < 0) or np.any(seq_start + lens > T)):
        raise ValueError("sequence range outside k/v")
    out = np.zeros((S, H, D), dtype=np.float64)
    rc = lib().oracle_attention_contig(_ptr(out), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(seq_start), _ptr(lens), S, H, Hkv, D,
                                       float(scale), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_attention_contig failed: {rc}")
    return out


def reshape_and_cache(key: np.ndarray, value: np.ndarray, slot_mapping: np.ndarray,
                      k_cache: np.ndarray, v_cache: np.ndarray) -> None:
    """In place: write key/value [T, Hkv, D] into the caches at their slots."""
    _need(key, np.float16, "key")
    _need(value, np.float16, "value")
    _need(slot_mapping, np.int64, "slot_mapping")
    _need(k_cache, np.float16, "k_cache")
    _need(v_cache, np.float16, "v_cache")
    T, Hkv, D = key.shape
    NB, Hkv2, B, D2 = k_cache.shape
    if value.shape != key.shape or v_cache.shape != k_cache.shape or (Hkv2, D2) != (Hkv, D):
        raise ValueError("shape mismatch")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping shape")
    rc = lib().oracle_reshape_and_cache(_ptr(key), _ptr(value), Hkv * D,
                                        _ptr(slot_mapping), T, _ptr(k_cache),
                                        _ptr(v_cache), NB, Hkv, B, D)
    if rc != 0:
        raise RuntimeError(f"oracle_reshape_and_cache failed: {rc}")


def copy_blocks(k_caches: Sequence[np.ndarray], v_caches: Sequence[np.ndarray],
                pairs: np.ndarray) -> None:
    """In place, for every layer: block pairs[i, 1] := block pairs[i, 0]."""
    if len(k_caches) != len(v_caches):
        raise ValueError("layer count mismatch")
    _need(pairs, np.int64, "pairs")
    if pairs.size == 0 or len(k_caches) == 0:
        return
    if pairs.ndim != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [N, 2]")
    shape = k_caches[0].shape
    for a in list(k_caches) + list(v_caches):
        _need(a, np.float16, "cache")
        if a.shape != shape:
            raise ValueError("all caches must share one shape")
    NB = shape[0]
    block_elems = int(np.prod(shape[1:]))
    kp = (ctypes.c_void_p * len(k_caches))(*[_ptr(a) for a in k_caches])
    vp = (ctypes.c_void_p * len(v_caches))(*[_ptr(a) for a in v_caches])
    rc = lib().oracle_copy_blocks(ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(vp, ctypes.c_void_p),
                                  len(k_caches), _ptr(pairs), pairs.shape[0],
                                  block_elems, NB)
    if rc != 0:
        raise RuntimeError(f"oracle_copy_blocks failed: {rc}")


def move_blocks(dst_pools: Sequence[np.ndarray], src_pools: Sequence[np.ndarray], pairs: np.ndarray) -> None:
    """In place, for every pool i and pair row (s, d): dst_pools[i][d] :=
    src_pools[i][s] -- whole blocks, bit for bit.  This is the data movement
    of a swap between the device pool and the host pool ([lpnh-1824136] 4.2:
    KV blocks can be moved out to host memory and back).  Destinations must
    be distinct; the source and destination pools are different arrays, so
    the order of the rows does not matter."""
    if len(dst_pools) != len(src_pools):
        raise ValueError("pool count mismatch")
    _need(pairs, np.int64, "pairs")
    if pairs.size == 0:
        return
    if pairs.ndim != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [N, 2]")
    if len(set(pairs[:, 1].tolist())) != pairs.shape[0]:
        raise ValueError("destinations must be distinct")
    for dst, src in zip(dst_pools, src_pools):
        if dst.dtype != src.dtype or dst.shape[1:] != src.shape[1:]:
            raise ValueError("pools must share the block shape")
        if np.any(pairs[:, 0] < 0) or np.any(pairs[:, 0] >= src.shape[0]) or \
           np.any(pairs[:, 1] < 0) or np.any(pairs[:, 1] >= dst.shape[0]):
            raise ValueError("block id outside its pool")
        for sblk, dblk in pairs.tolist():
            dst[dblk] = src[sblk]
