"""Seeded synthetic inputs for the paged-KV-cache hot path.

This module serves both the GPU path and the oracle, so it holds none of the
method's arithmetic: no slot mapping, no block accounting, no attention.  It
only draws numbers -- context lengths, physical-id permutations and fp16
values -- from fixed seeds.  Integer structure comes from numpy's PCG64 (the
same on every machine); bulk fp16 values come from a seeded torch generator
on the requested device (the oracle receives a host copy of exactly those
values, taken before any kernel runs).

Workload shapes follow the pages' examples: the 12-token, block-size-4 table
[7, 3, 1] of the 5688vip.com "4、PagedAttention" page (section 分页机制);
Llama-2-7B heads (32 x 128, fp16) and 2048-token contexts from the sizing
snippet on the explore.n1n.ai page (section "什么是 KV 缓存"); the prompt
mean of 500 tokens and outputs up to 1024 of the block-size experiment on the
5688vip.com page (section 案例); the 7B / 4096-token / 16-request sizing of
lpnh.cn/news/2758356 section 1.1; and parallel sampling over a shared prompt
from the same page, section 4.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np


def _rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([seed, *stream]))


def _torch_normal_f16(shape, seed: int, device, stream: int = 0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream)) & 0x7FFFFFFFFFFFFFFF)
    return torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float16)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


# ---------------------------------------------------------------------------
# Tiny case: 4 sequences, block_size 4, two heads of dim 16
# ---------------------------------------------------------------------------
@dataclass
class Tiny:
    block_size: int
    num_blocks: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    lens: List[int]
    tables: List[List[int]]          # physical ids per sequence, ceil(n/B) each
    k_tokens: np.ndarray             # [sum n, Hkv, D] fp16, sequence-major
    v_tokens: np.ndarray
    seq_start: np.ndarray            # int64 [S]
    q: np.ndarray                    # [S, H, D] fp16
    scale: float


def tiny(seed: int = 0, lens=(1, 5, 12, 50), block_size: int = 4,
         num_heads: int = 2, num_kv_heads: int = 2, head_dim: int = 16,
         num_blocks: int = 64, fixed_seq: int = 2, fixed_table=(7, 3, 1)) -> Tiny:
    """Values drawn fp32 N(0, 1) and rounded to fp16.  Sequence `fixed_seq`
    gets the table printed on the page; the others get distinct ids drawn by
    a random permutation of the remaining pool."""
    rng = _rng(seed, 1)
    lens = [int(n) for n in lens]
    S = len(lens)
    fixed = [int(b) for b in fixed_table]
    rest = np.array([b for b in range(num_blocks) if b not in set(fixed)], dtype=np.int64)
    rest = rest[rng.permutation(len(rest))]
    tables, used = [], 0
    for s, n in enumerate(lens):
        nb = ceil_div(n, block_size)
        if s == fixed_seq and fixed:
            if nb != len(fixed):
                raise ValueError("fixed table does not fit the sequence length")
            tables.append(list(fixed))
        else:
            tables.append([int(b) for b in rest[used:used + nb]])
            used += nb
    total = sum(lens)
    k = rng.standard_normal((total, num_kv_heads, head_dim), dtype=np.float32).astype(np.float16)
    v = rng.standard_normal((total, num_kv_heads, head_dim), dtype=np.float32).astype(np.float16)
    q = rng.standard_normal((S, num_heads, head_dim), dtype=np.float32).astype(np.float16)
    seq_start = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    return Tiny(block_size, num_blocks, num_heads, num_kv_heads, head_dim, lens,
                tables, k, v, seq_start, q, 1.0 / math.sqrt(head_dim))


# ---------------------------------------------------------------------------
# Llama-2-7B-shaped decode over a pre-filled pool
# ---------------------------------------------------------------------------
@dataclass
class PoolDecode:
    block_size: int
    num_blocks: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    lens: np.ndarray                 # int32 [S]: context length INCLUDING the new token
    perm_tables: np.ndarray          # int32 [S, width]: a random permutation of the pool
    scale: float
    seed: int
    layers: int = 1

    def pool(self, layer: int, device):
        """(k_cache, v_cache) fp16 [NB, Hkv, B, D], every slot N(0, 1)."""
        shape = (self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim)
        return (_torch_normal_f16(shape, self.seed, device, 100 + 2 * layer),
                _torch_normal_f16(shape, self.seed, device, 101 + 2 * layer))

    def new_tokens(self, step: int, device):
        """(q [S, H, D], key [S, Hkv, D], value [S, Hkv, D]) for one step."""
        S = len(self.lens)
        return (_torch_normal_f16((S, self.num_heads, self.head_dim), self.seed, device, 10_000 + 3 * step),
                _torch_normal_f16((S, self.num_kv_heads, self.head_dim), self.seed, device, 10_001 + 3 * step),
                _torch_normal_f16((S, self.num_kv_heads, self.head_dim), self.seed, device, 10_002 + 3 * step))


def llama7b_decode(seed: int = 0, num_seqs: int = 64, max_len: int = 2048,
                   block_size: int = 16, num_heads: int = 32,
                   num_kv_heads: int = 32, head_dim: int = 128,
                   layers: int = 1, min_len: int = 1) -> PoolDecode:
    """Context lengths uniform on [min_len, max_len]; pool of
    num_seqs * ceil(max_len / B) blocks; sequence i's table row is slice i of
    one random permutation of the pool."""
    rng = _rng(seed, 2)
    lens = rng.integers(min_len, max_len + 1, size=num_seqs).astype(np.int32)
    width = ceil_div(max_len, block_size)
    nb = num_seqs * width
    perm = rng.permutation(nb).astype(np.int32)
    return PoolDecode(block_size, nb, num_heads, num_kv_heads, head_dim, lens,
                      perm.reshape(num_seqs, width), 1.0 / math.sqrt(head_dim), seed, layers)


def gqa_decode(seed: int = 0, num_seqs: int = 256, max_len: int = 2048, block_size: int = 16,
               num_heads: int = 64, num_kv_heads: int = 8, head_dim: int = 128,
               layers: int = 1, min_len: int = 1) -> PoolDecode:
    """Grouped-query decode: 8 query heads share each of 8 KV heads (the
    attention shape of the 70B-class model the lpnh.cn/news/1824136 page
    sizes in section 1.1), otherwise drawn like llama7b_decode.  256
    sequences put about 1 GB of K/V behind one layer's decode, as in the
    Llama-2-7B batch."""
    w = llama7b_decode(seed=seed, num_seqs=num_seqs, max_len=max_len, block_size=block_size,
                       num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                       layers=layers, min_len=min_len)
    return w


def long_context(seed: int = 0, num_seqs: int = 16, ctx: int = 4096,
                 block_size: int = 16, num_heads: int = 32, num_kv_heads: int = 32,
                 head_dim: int = 128, layers: int = 32, spare_blocks: int = 0) -> PoolDecode:
    """Every sequence at the same length; one permutation table for all
    layers.  spare_blocks extra ids (the highest) stay out of the tables, for
    tokens appended later."""
    rng = _rng(seed, 4)
    lens = np.full(num_seqs, ctx, dtype=np.int32)
    width = ceil_div(ctx, block_size)
    nb = num_seqs * width
    perm = rng.permutation(nb).astype(np.int32)
    return PoolDecode(block_size, nb + spare_blocks, num_heads, num_kv_heads, head_dim, lens,
                      perm.reshape(num_seqs, width), 1.0 / math.sqrt(head_dim), seed, layers)


# ---------------------------------------------------------------------------
# Block-size sweep: one set of token values shared by every block size
# ---------------------------------------------------------------------------
@dataclass
class Sweep:
    num_heads: int
    num_kv_heads: int
    head_dim: int
    lens: np.ndarray                 # int32 [S]
    seq_start: np.ndarray            # int64 [S]
    seed: int
    scale: float

    def tokens(self, device):
        """(k, v) fp16 [sum n, Hkv, D], sequence-major, the same for every B."""
        T = int(self.lens.sum())
        shape = (T, self.num_kv_heads, self.head_dim)
        return (_torch_normal_f16(shape, self.seed, device, 300),
                _torch_normal_f16(shape, self.seed, device, 301))

    def query(self, device):
        return _torch_normal_f16((len(self.lens), self.num_heads, self.head_dim), self.seed, device, 302)

    def perm_tables(self, block_size: int) -> List[np.ndarray]:
        """Pool of exactly sum ceil(n / B) blocks, dealt out by a random
        permutation (same seed for every block size)."""
        nbs = [ceil_div(int(n), block_size) for n in self.lens]
        perm = _rng(self.seed, 3, block_size).permutation(sum(nbs)).astype(np.int32)
        out, at = [], 0
        for nb in nbs:
            out.append(perm[at:at + nb])
            at += nb
        return out


def block_size_sweep(seed: int = 0, num_seqs: int = 256, prompt_mean: float = 500.0,
                     prompt_std: float = 150.0, prompt_min: int = 16,
                     prompt_max: int = 2048, gen_max: int = 1024,
                     num_heads: int = 32, num_kv_heads: int = 32,
                     head_dim: int = 128) -> Sweep:
    """Context = prompt (normal, rounded, clipped) + generated (uniform on
    [1, gen_max])."""
    rng = _rng(seed, 5)
    prompt = np.clip(np.rint(rng.normal(prompt_mean, prompt_std, size=num_seqs)),
                     prompt_min, prompt_max).astype(np.int64)
    gen = rng.integers(1, gen_max + 1, size=num_seqs)
    lens = (prompt + gen).astype(np.int32)
    seq_start = np.concatenate([[0], np.cumsum(lens.astype(np.int64))[:-1]]).astype(np.int64)
    return Sweep(num_heads, num_kv_heads, head_dim, lens, seq_start, seed,
                 1.0 / math.sqrt(head_dim))


# ---------------------------------------------------------------------------
# Parallel sampling over one shared prompt
# ---------------------------------------------------------------------------
@dataclass
class Sampling:
    num_blocks: int
    block_size: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    prompt_len: int
    num_samples: int
    steps: int
    seed: int
    scale: float

    def prompt_tokens(self, device):
        shape = (self.prompt_len, self.num_kv_heads, self.head_dim)
        return (_torch_normal_f16(shape, self.seed, device, 500),
                _torch_normal_f16(shape, self.seed, device, 501))

    def step_tokens(self, step: int, device):
        """(q [N, H, D], key [N, Hkv, D], value [N, Hkv, D]); one row per sample."""
        N = self.num_samples
        return (_torch_normal_f16((N, self.num_heads, self.head_dim), self.seed, device, 20_000 + 3 * step),
                _torch_normal_f16((N, self.num_kv_heads, self.head_dim), self.seed, device, 20_001 + 3 * step),
                _torch_normal_f16((N, self.num_kv_heads, self.head_dim), self.seed, device, 20_002 + 3 * step))


def parallel_sampling(seed: int = 0, num_blocks: int = 1024, block_size: int = 16,
                      prompt_len: int = 1000, num_samples: int = 32, steps: int = 256,
                      num_heads: int = 32, num_kv_heads: int = 32,
                      head_dim: int = 128) -> Sampling:
    return Sampling(num_blocks, block_size, num_heads, num_kv_heads, head_dim,
                    prompt_len, num_samples, steps, seed, 1.0 / math.sqrt(head_dim))


# ---------------------------------------------------------------------------
# Random operation streams for the block manager (differential testing)
# ---------------------------------------------------------------------------
def block_manager_ops(seed: int, n_ops: int, max_seqs: int = 6,
                      max_prompt: int = 40, swap: bool = False, cached: bool = False) -> List[tuple]:
    """A stream of ('add', seq, n) / ('fork', parent, child) / ('append', seq)
    / ('free', seq) operations, plus ('swap_out', [seqs]) / ('swap_in',
    [seqs]) groups when swap is set and ('add_cached', seq, [token ids])
    prompts drawn from a few shared prefixes when cached is set.  Ids may be
    stale or unknown on purpose, so error paths are exercised too."""
    rng = _rng(seed, 6)
    ops = []
    next_id = 0
    swapped_groups: List[List[int]] = []      # groups sent out, to bring back later
    prefixes = [rng.integers(0, 50, size=max_prompt).tolist() for _ in range(3)] if cached else []
    for _ in range(n_ops):
        if cached and rng.random() < 0.2:
            base = prefixes[int(rng.integers(0, 3))]
            keep = int(rng.integers(0, max_prompt + 1))
            tail = rng.integers(0, 50, size=int(rng.integers(0, max_prompt // 2 + 1))).tolist()
            ops.append(("add_cached", next_id, [int(t) for t in base[:keep] + tail][:max_prompt]))
            next_id += 1
            continue
        if swap and rng.random() < 0.15:
            if swapped_groups and rng.random() < 0.5:
                group = swapped_groups.pop(int(rng.integers(0, len(swapped_groups))))
                ops.append(("swap_in", group))
            else:
                k = int(rng.integers(1, 4))
                group = sorted({int(x) for x in rng.integers(max(next_id - 6, 0), max(next_id, 1), size=k)})
                ops.append(("swap_out", group))
                swapped_groups.append(group)
            continue
        r = rng.random()
        if r < 0.15:
            ops.append(("add", next_id, int(rng.integers(0, max_prompt + 1))))
            next_id += 1
        elif r < 0.25:
            ops.append(("fork", int(rng.integers(0, max(next_id, 1))), next_id))
            next_id += 1
        elif r < 0.85:
            ops.append(("append", int(rng.integers(0, max(next_id, 1)))))
        else:
            ops.append(("free", int(rng.integers(0, max(next_id, 1)))))
    return ops


def random_case(seed: int, lens, num_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, spare_blocks: int = 3) -> Tiny:
    """Arbitrary lengths: contiguous fp16 N(0, 1) K/V per sequence, q, and
    tables dealt from one random permutation of a pool with `spare_blocks`
    ids left over."""
    rng = _rng(seed, 7)
    lens = [int(n) for n in lens]
    nbs = [ceil_div(n, block_size) for n in lens]
    nb = sum(nbs) + spare_blocks
    perm = rng.permutation(nb)
    tables, at = [], 0
    for k in nbs:
        tables.append([int(b) for b in perm[at:at + k]])
        at += k
    total = sum(lens)
    k = rng.standard_normal((total, num_kv_heads, head_dim), dtype=np.float32).astype(np.float16)
    v = rng.standard_normal((total, num_kv_heads, head_dim), dtype=np.float32).astype(np.float16)
    q = rng.standard_normal((len(lens), num_heads, head_dim), dtype=np.float32).astype(np.float16)
    seq_start = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64) if lens else np.zeros(0, np.int64)
    return Tiny(block_size, nb, num_heads, num_kv_heads, head_dim, lens, tables, k, v,
                seq_start, q, 1.0 / math.sqrt(head_dim))
