"""Block-manager model: the oracle for block tables, refcounts, the free list,
slot mapping and copy-on-write pairs.

Test infrastructure only (see oracle/__init__.py).  A plain Python model of
what the pages describe; the product's C++ block manager is checked against it
operation by operation, bit for bit.

Sources (named by address, sections as the pages number them):
  [5688vip]       5688vip.com, "4、PagedAttention：显存管理、分页机制、块大小选择"
  [n1n]           explore.n1n.ai, "PagedAttention 对比传统 KV 缓存：vLLM 如何重塑
                  LLM 推理的 GPU 显存管理"
  [lpnh-2758356]  lpnh.cn/news/2758356, sections 1-5
  [lpnh-1824136]  lpnh.cn/news/1824136, sections 1-4

Rules modelled:
  * The pool starts as every physical id 0..N-1 on a free list; allocation
    takes the id at the END of that list and fails (returns None) when the
    list is empty ([n1n] code example under "实现逻辑代码示例").
  * A sequence is given blocks for its current tokens only; a new block is
    appended to its table when its last block is full or it has none
    ([5688vip] 分页机制; [n1n] 工作原理; [lpnh-2758356] 3.1).
  * Each allocated block carries a reference count set to 1; releasing a
    sequence walks its table, decrements each count and returns blocks that
    reach 0 to the free list ([lpnh-2758356] 3.2).
  * Forking shares the parent's blocks: the child's table points at the same
    ids and each count grows by one ([lpnh-2758356] 4.2, first step).
  * Writing into a shared block that still has free slots copies it first:
    allocate, copy the whole block, decrement the old count, repoint the
    table entry ([lpnh-2758356] 4.2, second and third steps).  A shared block
    that is already full is never copied: the next token simply gets a fresh
    block ([lpnh-2758356] 4.2, the closing remark on when COW fires).
  * Slot of logical position p: table[p // B] * B + p % B ([5688vip]
    分页机制 figure; [lpnh-2758356] 2.2).

  * Requests whose prompts start with the same tokens (the page's example:
    100 requests with one long system prompt) share the physical blocks of
    that common prefix; copying happens only where their tokens diverge
    ([n1n] 前缀缓存; [lpnh-1824136] 3.2, second step: a prompt equal to a
    running sequence's may share its blocks).
  * Under memory pressure a sequence's KV blocks can be moved to host memory
    and back ("swap": [lpnh-1824136] 4.2 names it as a supported, slow
    option for serving very long contexts when latency can be traded).

Readings where the pages leave a step open:
  * Fill level is tracked per sequence (its length) rather than per block;
    for an unshared block the two agree, and for a shared block the
    per-sequence length is what decides whether the writer's next slot is
    free.
  * Any operation that runs out of blocks changes nothing and reports OOM.
  * A batch of appends is processed in the order given; samples that share a
    block therefore copy one after another until the last holder finds a
    count of 1 and writes in place.
  * Swap works on a group of sequences at once (so blocks shared by forks
    stay shared): every distinct block of the group, in order of first
    appearance (sequence order, then table order), gets one block of a host
    pool -- a second pool with its own free list and counts, allocated like
    the device pool -- whose count is the number of group members holding
    it; the device count drops by that number and a block reaching 0 goes
    back to the device free list in the same order.  Swapping in is the
    mirror image.  A swapped-out sequence can only be swapped in or freed.
    A group short of free blocks on the receiving side changes nothing.
  * Prefix sharing is decided per FULL block and exactly: a full block is
    found again by (the id of the block before it in the sequence, or -1 for
    the first block; the block's own token ids).  Since a block's KV depends
    on every earlier token, chaining through the previous block's id makes
    the key stand for the whole prefix without storing it.  Only full prompt
    blocks of sequences added with their token ids are indexed; a partial
    last block is never shared this way (its next token would have to copy
    it), and a block leaves the index when its count drops to 0.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple


class OOM(Exception):
    """No free block was available; the model state is unchanged."""


class StateError(Exception):
    """Unknown sequence, duplicate id, or a block that is not free."""


@dataclass
class _Seq:
    table: List[int] = field(default_factory=list)
    length: int = 0
    swapped: bool = False            # table holds host-pool ids


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, num_host_blocks: int = 0):
        if num_blocks < 0 or block_size <= 0 or num_host_blocks < 0:
            raise ValueError("num_blocks >= 0, num_host_blocks >= 0 and block_size > 0 required")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: List[int] = list(range(num_blocks))
        self.refcount: List[int] = [0] * num_blocks
        self.seqs: Dict[int, _Seq] = {}
        self.num_host_blocks = num_host_blocks
        self.host_free: List[int] = list(range(num_host_blocks))
        self.host_refcount: List[int] = [0] * num_host_blocks
        self.prefix_index: Dict[tuple, int] = {}     # (previous block or -1, token ids) -> block
        self.block_key: Dict[int, tuple] = {}

    def _release(self, b: int) -> None:
        """A device block whose count reached 0 goes back on the free list
        and out of the prefix index."""
        self.free.append(b)
        key = self.block_key.pop(b, None)
        if key is not None:
            del self.prefix_index[key]

    def _resident(self, seq: int) -> _Seq:
        if seq not in self.seqs:
            raise StateError(f"unknown sequence {seq}")
        s = self.seqs[seq]
        if s.swapped:
            raise StateError(f"sequence {seq} is swapped out")
        return s

    # -- allocation ---------------------------------------------------------
    def _alloc(self) -> Optional[int]:
        if not self.free:
            return None
        b = self.free.pop()
        self.refcount[b] = 1
        return b

    def blocks_for(self, n_tokens: int) -> int:
        return -(-n_tokens // self.block_size)

    # -- sequence operations ------------------------------------------------
    def add_sequence(self, seq: int, n_tokens: int) -> List[int]:
        """Allocate blocks for a new sequence of n_tokens; return its slots."""
        if seq in self.seqs:
            raise StateError(f"sequence {seq} exists")
        if n_tokens < 0:
            raise ValueError("n_tokens must be >= 0")
        need = self.blocks_for(n_tokens)
        if need > len(self.free):
            raise OOM()
        s = _Seq()
        for _ in range(need):
            s.table.append(self._alloc())
        s.length = n_tokens
        self.seqs[seq] = s
        return [self.slot(seq, p) for p in range(n_tokens)]

    def add_sequence_cached(self, seq: int, tokens: Sequence[int]) -> Tuple[List[int], int]:
        """Add a sequence given its prompt's token ids, sharing every leading
        full block whose prefix is already cached.  Returns (slots of all
        positions, number of leading positions whose KV is already there)."""
        if seq in self.seqs:
            raise StateError(f"sequence {seq} exists")
        tokens = [int(t) for t in tokens]
        B = self.block_size
        n = len(tokens)
        hits: List[int] = []
        parent = -1
        for i in range(n // B):
            b = self.prefix_index.get((parent, tuple(tokens[i * B:(i + 1) * B])))
            if b is None:
                break
            hits.append(b)
            parent = b
        need = self.blocks_for(n) - len(hits)
        if need > len(self.free):
            raise OOM()
        for b in hits:
            self.refcount[b] += 1
        s = _Seq(table=list(hits), length=n)
        for i in range(len(hits), self.blocks_for(n)):
            b = self._alloc()
            s.table.append(b)
            if (i + 1) * B <= n:                       # a full prompt block: index it
                key = (s.table[i - 1] if i > 0 else -1, tuple(tokens[i * B:(i + 1) * B]))
                self.prefix_index[key] = b
                self.block_key[b] = key
        self.seqs[seq] = s
        return [self.slot(seq, p) for p in range(n)], len(hits) * B

    def set_table(self, seq: int, blocks: Sequence[int], n_tokens: int) -> None:
        """Give a new sequence an explicit table (ids must be free)."""
        if seq in self.seqs:
            raise StateError(f"sequence {seq} exists")
        blocks = [int(b) for b in blocks]
        if len(blocks) != self.blocks_for(n_tokens):
            raise ValueError("table length must be ceil(n_tokens / block_size)")
        if len(set(blocks)) != len(blocks):
            raise StateError("duplicate block id in table")
        free_set = set(self.free)
        for b in blocks:
            if not (0 <= b < self.num_blocks) or b not in free_set:
                raise StateError(f"block {b} is not free")
        taken = set(blocks)
        self.free = [b for b in self.free if b not in taken]
        for b in blocks:
            self.refcount[b] = 1
        self.seqs[seq] = _Seq(table=list(blocks), length=n_tokens)

    def fork(self, parent: int, child: int) -> None:
        p = self._resident(parent)
        if child in self.seqs:
            raise StateError(f"sequence {child} exists")
        for b in p.table:
            self.refcount[b] += 1
        self.seqs[child] = _Seq(table=list(p.table), length=p.length)

    def append_token(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot for the sequence's next token.

        Returns (slot, cow) where cow is (src, dst) when the shared last
        block had to be copied, else None.  Raises OOM with no change."""
        s = self._resident(seq)
        B = self.block_size
        n = s.length
        cow = None
        if n % B == 0:
            # no block yet, or the last one is full: take a fresh block
            b = self._alloc()
            if b is None:
                raise OOM()
            s.table.append(b)
        else:
            last = s.table[-1]
            if self.refcount[last] > 1:
                b = self._alloc()
                if b is None:
                    raise OOM()
                cow = (last, b)
                self.refcount[last] -= 1
                s.table[-1] = b
        s.length = n + 1
        return self.slot(seq, n), cow

    def free_sequence(self, seq: int) -> None:
        if seq not in self.seqs:
            raise StateError(f"unknown sequence {seq}")
        s = self.seqs.pop(seq)
        for b in s.table:
            if s.swapped:
                self.host_refcount[b] -= 1
                if self.host_refcount[b] == 0:
                    self.host_free.append(b)
            else:
                self.refcount[b] -= 1
                if self.refcount[b] == 0:
                    self._release(b)

    # -- swap to / from the host pool ---------------------------------------
    def _move(self, seqs: Sequence[int], out: bool) -> List[Tuple[int, int]]:
        seqs = [int(q) for q in seqs]
        if len(set(seqs)) != len(seqs):
            raise StateError("a sequence appears twice in the group")
        for q in seqs:
            if q not in self.seqs:
                raise StateError(f"unknown sequence {q}")
            if self.seqs[q].swapped == out:
                raise StateError(f"sequence {q} is already {'swapped out' if out else 'resident'}")
        src_count, src_free = (self.refcount, self.free) if out else (self.host_refcount, self.host_free)
        dst_count, dst_free = (self.host_refcount, self.host_free) if out else (self.refcount, self.free)
        order: List[int] = []
        holders: Dict[int, int] = {}
        for q in seqs:
            for b in self.seqs[q].table:
                if b not in holders:
                    order.append(b)
                    holders[b] = 0
                holders[b] += 1
        if len(order) > len(dst_free):
            raise OOM()
        new_id: Dict[int, int] = {}
        pairs = []
        for b in order:
            d = dst_free.pop()
            dst_count[d] = holders[b]
            new_id[b] = d
            pairs.append((b, d))
            src_count[b] -= holders[b]
            if src_count[b] == 0:
                if out:
                    self._release(b)
                else:
                    src_free.append(b)
        for q in seqs:
            s = self.seqs[q]
            s.table = [new_id[b] for b in s.table]
            s.swapped = out
        return pairs

    def swap_out(self, seqs: Sequence[int]) -> List[Tuple[int, int]]:
        """Move a group's blocks to the host pool; returns (device id, host
        id) pairs in order of first appearance.  Raises OOM with no change."""
        return self._move(seqs, True)

    def swap_in(self, seqs: Sequence[int]) -> List[Tuple[int, int]]:
        """Move a swapped-out group back; returns (host id, device id) pairs."""
        return self._move(seqs, False)

    # -- queries ------------------------------------------------------------
    def slot(self, seq: int, pos: int) -> int:
        s = self._resident(seq)
        B = self.block_size
        if not 0 <= pos < len(s.table) * B:
            raise IndexError(pos)
        return s.table[pos // B] * B + pos % B

    def table(self, seq: int) -> List[int]:
        return list(self.seqs[seq].table)

    def length(self, seq: int) -> int:
        return self.seqs[seq].length

    def tables(self, seqs: Sequence[int], max_blocks: int) -> Tuple[List[List[int]], List[int]]:
        rows, lens = [], []
        for q in seqs:
            t = self._resident(q).table
            if len(t) > max_blocks:
                raise ValueError("max_blocks too small")
            rows.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.seqs[q].length)
        return rows, lens

    def num_free(self) -> int:
        return len(self.free)

    def check_invariants(self) -> None:
        """In each pool (device, host): counts equal the number of tables
        holding each block; free ids have count 0; every id is either free
        or held."""
        for swapped, n, count, free in ((False, self.num_blocks, self.refcount, self.free),
                                        (True, self.num_host_blocks, self.host_refcount, self.host_free)):
            held: Dict[int, int] = {}
            for s in self.seqs.values():
                if len(set(s.table)) != len(s.table):
                    raise AssertionError("duplicate id within a table")
                if len(s.table) != self.blocks_for(s.length):
                    raise AssertionError("table length != ceil(len / B)")
                if s.swapped != swapped:
                    continue
                for b in s.table:
                    held[b] = held.get(b, 0) + 1
            for b in range(n):
                if count[b] != held.get(b, 0):
                    raise AssertionError(f"count[{b}]={count[b]} held={held.get(b, 0)} (host={swapped})")
            if len(set(free)) != len(free):
                raise AssertionError("duplicate id on a free list")
            if set(free) & set(held):
                raise AssertionError("a held block is on a free list")
            if len(free) + len(held) != n:
                raise AssertionError("free + held != pool size")
        for key, b in self.prefix_index.items():
            if self.block_key.get(b) != key or self.refcount[b] == 0:
                raise AssertionError(f"prefix index entry for block {b} is stale")
        if len(self.block_key) != len(self.prefix_index):
            raise AssertionError("prefix index and its reverse map differ")
