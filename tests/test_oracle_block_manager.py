"""Pins for the block-manager model (oracle O1) against the pages' worked
examples, the COW rules and invariants that hold for every operation."""
import pytest

import workloads
from oracle.block_manager import OOM, BlockManagerModel, StateError


def _page_example(g):
    """Rebuild the figure's pool: blocks 1-9 drawn, block 0 not drawn (taken
    here as held elsewhere), 5 and 8 held by another request."""
    m = BlockManagerModel(10, g["block_size"])
    m.set_table(100, [0], 1)                       # not in the figure
    m.set_table(101, g["other_request_blocks"], 2 * g["block_size"])
    m.set_table(1, g["table"], g["n_tokens"])
    return m


def test_page_figure_mapping(load_golden):
    g = load_golden("page_table_12_tokens.json")
    m = _page_example(g)
    B = g["block_size"]
    assert sorted(m.free) == g["free_blocks"]
    for lb, (lo, hi) in enumerate(g["logical_token_ranges"]):
        for off, p in enumerate(range(lo, hi + 1)):
            slot = m.slot(1, p)
            assert slot // B == g["table"][lb]            # the figure's physical block
            assert slot % B == off                        # tokens keep their order inside it
    # logical block 3 is unmapped until token 12 arrives
    with pytest.raises(IndexError):
        m.slot(1, 12)
    slot, cow = m.append_token(1)
    assert cow is None
    new = m.table(1)[3]
    assert new in g["next_block_one_of"]
    assert new == 9                                    # LIFO over the free list [2, 4, 6, 9]
    assert slot == new * B
    m.check_invariants()


def test_lpnh_60_token_table(load_golden):
    g = load_golden("lpnh_60_token_table.json")
    B = g["block_size"]
    n = sum(g["tokens_per_block"])
    m = BlockManagerModel(64, B)
    m.set_table(0, g["table"], n)
    fills = [0] * len(g["table"])
    for p in range(n):
        fills[g["table"].index(m.slot(0, p) // B)] += 1
    assert fills == g["tokens_per_block"]
    assert m.slot(0, n - 1) == 47 * 16 + 11


def test_allocation_is_lifo_and_oom_changes_nothing():
    # the pages' allocator pops from the end of list(range(N)) and reports
    # failure when the list is empty
    m = BlockManagerModel(3, 4)
    m.add_sequence(0, 4)
    assert m.table(0) == [2]
    m.add_sequence(1, 5)
    assert m.table(1) == [1, 0]
    snapshot = (list(m.free), list(m.refcount), m.table(0), m.table(1), m.length(0))
    with pytest.raises(OOM):
        m.append_token(0)                          # block 2 is full, pool empty
    assert (list(m.free), list(m.refcount), m.table(0), m.table(1), m.length(0)) == snapshot
    slot, cow = m.append_token(1)                  # block 0 has room
    assert (slot, cow) == (0 * 4 + 1, None)
    with pytest.raises(OOM):
        m.add_sequence(2, 1)
    assert 2 not in m.seqs


def test_fork_refcount_and_cow(load_golden):
    g = load_golden("lpnh_cow.json")
    B = 16
    m = BlockManagerModel(32, B)
    m.add_sequence(0, 20)                          # 2 blocks, last holds 4
    for c in range(1, g["fork_ways"]):
        m.fork(0, c)
    for b in m.table(0):
        assert m.refcount[b] == g["refcount_after_fork"]
    shared_last = m.table(0)[-1]
    # first writer into the shared, partly filled block copies it
    slot, cow = m.append_token(1)
    assert cow is not None and cow[0] == shared_last
    assert m.table(1)[-1] == cow[1] != shared_last
    assert m.refcount[shared_last] == 2 and m.refcount[cow[1]] == 1
    assert slot == cow[1] * B + 4
    assert m.table(1)[0] == m.table(0)[0]          # the full block stays shared
    # the second writer copies too; the last holder then writes in place
    _, cow2 = m.append_token(2)
    assert cow2 is not None and cow2[0] == shared_last
    slot0, cow0 = m.append_token(0)
    assert cow0 is None and m.refcount[shared_last] == 1
    assert slot0 == shared_last * B + 4
    m.check_invariants()


def test_full_shared_block_gets_fresh_block_without_copy(load_golden):
    g = load_golden("lpnh_cow.json")
    assert g["full_shared_block_gets_fresh_block_without_copy"]
    m = BlockManagerModel(16, 4)
    m.add_sequence(0, 8)                           # two full blocks
    m.fork(0, 1)
    m.fork(0, 2)
    before = m.table(0)
    for s in (0, 1, 2):
        slot, cow = m.append_token(s)
        assert cow is None
        assert m.table(s)[:2] == before            # shared prefix untouched
        assert len(m.table(s)) == 3 and m.refcount[m.table(s)[2]] == 1
        assert slot == m.table(s)[2] * 4
    assert len({m.table(s)[2] for s in (0, 1, 2)}) == 3
    m.check_invariants()


def test_release_returns_zero_count_blocks(load_golden):
    assert load_golden("lpnh_cow.json")["release_returns_zero_count_blocks"]
    m = BlockManagerModel(8, 4)
    m.add_sequence(0, 6)
    m.fork(0, 1)
    m.append_token(1)                              # COW of the tail block
    shared = m.table(0)[0]
    n0 = m.num_free()
    m.free_sequence(0)
    # block 0's private tail returns; the shared first block waits for seq 1
    assert m.num_free() == n0 + 1 and m.refcount[shared] == 1
    m.free_sequence(1)
    assert m.num_free() == 8 and all(r == 0 for r in m.refcount)
    with pytest.raises(StateError):
        m.free_sequence(1)
    m.check_invariants()


def test_parallel_sampling_shape():
    """The prompt-sharing workload: 1000 tokens at B=16 is 63 blocks with an
    8-token tail; 31 forks give count 32; the first round of appends copies
    31 times from the one tail block and the last sample writes in place."""
    w = workloads.parallel_sampling()
    m = BlockManagerModel(w.num_blocks, w.block_size)
    m.add_sequence(0, w.prompt_len)
    assert len(m.table(0)) == 63 and w.prompt_len - 62 * 16 == 8
    for c in range(1, w.num_samples):
        m.fork(0, c)
    assert all(m.refcount[b] == 32 for b in m.table(0))
    tail = m.table(0)[-1]
    pairs = []
    for s in range(w.num_samples):
        _, cow = m.append_token(s)
        if cow:
            pairs.append(cow)
    assert len(pairs) == 31 and all(src == tail for src, _ in pairs)
    assert m.table(31)[-1] == tail and m.refcount[tail] == 1
    for _ in range(w.steps - 1):
        for s in range(w.num_samples):
            assert m.append_token(s)[1] is None
    assert all(len(m.table(s)) == 79 for s in range(w.num_samples))   # 1256 tokens
    m.check_invariants()
    for s in range(w.num_samples):
        m.free_sequence(s)
    assert m.num_free() == w.num_blocks


@pytest.mark.parametrize("seed", range(8))
def test_invariants_under_random_ops(seed):
    m = BlockManagerModel(12, 4)
    for op in workloads.block_manager_ops(seed, 400):
        try:
            if op[0] == "add":
                m.add_sequence(op[1], op[2])
            elif op[0] == "fork":
                m.fork(op[1], op[2])
            elif op[0] == "append":
                m.append_token(op[1])
            else:
                m.free_sequence(op[1])
        except (OOM, StateError):
            pass
        m.check_invariants()


def test_set_table_rejects_bad_tables():
    m = BlockManagerModel(8, 4)
    with pytest.raises(ValueError):
        m.set_table(0, [1, 2], 9)                  # needs 3 blocks
    with pytest.raises(StateError):
        m.set_table(0, [1, 1], 8)
    m.set_table(0, [1, 2], 8)
    with pytest.raises(StateError):
        m.set_table(1, [2], 3)                     # not free
    with pytest.raises(StateError):
        m.set_table(1, [9], 3)                     # outside the pool


# ---------------------------------------------------------------------------
# swap to / from the host pool ([lpnh-1824136] 4.2 names the operation; the
# group semantics are a reading of that passage, pinned here by counting)
# ---------------------------------------------------------------------------
def _forked_group(nb=16, nh=16, B=4, prompt=10, samples=3):
    """A prompt of 10 tokens (2 full blocks + a 2-token tail) forked into
    `samples` sequences, each of which then appends one token: samples - 1
    copy the shared tail, the last writes in place."""
    m = BlockManagerModel(nb, B, nh)
    m.add_sequence(0, prompt)
    for c in range(1, samples):
        m.fork(0, c)
    for c in range(samples):
        m.append_token(c)
    return m


def test_swap_out_of_a_fork_group_keeps_sharing():
    m = _forked_group()
    shared = m.table(0)[:2]
    assert all(m.refcount[b] == 3 for b in shared)
    distinct = {b for q in range(3) for b in m.table(q)}
    assert len(distinct) == 2 + 3                    # two shared full blocks, three private tails
    pairs = m.swap_out([0, 1, 2])
    assert len(pairs) == 5 and len({h for _, h in pairs}) == 5
    assert m.num_free() == 16                        # every device block came back
    for q in range(3):
        assert m.seqs[q].swapped
    hs = m.seqs[0].table[:2]
    assert all(m.seqs[q].table[:2] == hs for q in range(3))   # still shared, on the host
    assert all(m.host_refcount[h] == 3 for h in hs)
    assert all(m.host_refcount[m.seqs[q].table[2]] == 1 for q in range(3))
    m.check_invariants()
    back = m.swap_in([2, 0, 1])
    assert len(back) == 5
    ds = m.table(2)[:2]
    assert all(m.table(q)[:2] == ds for q in range(3)) and all(m.refcount[b] == 3 for b in ds)
    assert len(m.host_free) == 16
    m.check_invariants()


def test_swap_pairs_follow_first_appearance_and_lifo():
    """Pairs list each distinct block once, in sequence order then table
    order; host ids are taken from the end of the host free list."""
    m = BlockManagerModel(8, 2, 5)
    m.add_sequence(0, 3)            # blocks 7, 6
    m.add_sequence(1, 2)            # block 5
    m.fork(0, 2)
    pairs = m.swap_out([1, 2])
    assert pairs == [(5, 4), (7, 3), (6, 2)]
    assert m.refcount[7] == 1 and m.refcount[6] == 1 and m.refcount[5] == 0
    assert m.free == [0, 1, 2, 3, 4, 5]
    assert m.seqs[1].table == [4] and m.seqs[2].table == [3, 2]
    m.check_invariants()


def test_swapping_one_member_out_splits_the_sharing():
    m = _forked_group()
    before = {b: m.refcount[b] for b in m.table(0)[:2]}
    pairs = m.swap_out([1])
    assert len(pairs) == 3
    for b, c in before.items():
        assert m.refcount[b] == c - 1                 # still held by samples 0 and 2
    assert all(m.host_refcount[h] == 1 for _, h in pairs)
    m.swap_in([1])
    assert m.table(1)[:2] != m.table(0)[:2]           # its own copies now
    m.check_invariants()


def test_swap_oom_changes_nothing():
    m = BlockManagerModel(8, 4, 2)
    m.add_sequence(0, 12)                             # 3 blocks > 2 host blocks
    snap = (list(m.free), list(m.refcount), list(m.host_free), list(m.host_refcount), m.table(0))
    with pytest.raises(OOM):
        m.swap_out([0])
    assert snap == (list(m.free), list(m.refcount), list(m.host_free), list(m.host_refcount), m.table(0))
    m2 = BlockManagerModel(3, 4, 8)
    m2.add_sequence(0, 12)
    m2.swap_out([0])
    m2.add_sequence(1, 4)                             # device now has 2 free blocks < 3
    with pytest.raises(OOM):
        m2.swap_in([0])
    assert m2.seqs[0].swapped and m2.num_free() == 2
    m2.check_invariants()


def test_swapped_sequence_only_swaps_in_or_frees():
    m = BlockManagerModel(8, 4, 8)
    m.add_sequence(0, 5)
    m.swap_out([0])
    for op in (lambda: m.append_token(0), lambda: m.fork(0, 1), lambda: m.slot(0, 0),
               lambda: m.tables([0], 4), lambda: m.swap_out([0])):
        with pytest.raises(StateError):
            op()
    with pytest.raises(StateError):
        m.swap_in([0, 0])
    m.free_sequence(0)
    assert len(m.host_free) == 8 and m.num_free() == 8
    m.check_invariants()


@pytest.mark.parametrize("seed", range(6))
def test_swap_round_trip_preserves_structure(seed):
    """After any reachable state, swapping a group out and back in gives
    tables that differ only by a relabelling of blocks: same lengths, same
    pattern of shared blocks, same counts."""
    m = BlockManagerModel(40, 4, 40)
    for op in workloads.block_manager_ops(seed, 120, max_prompt=12):
        try:
            getattr(m, {"add": "add_sequence", "fork": "fork", "append": "append_token",
                        "free": "free_sequence"}[op[0]])(*op[1:])
        except (OOM, StateError):
            pass
    group = sorted(m.seqs)[:3]
    if not group:
        pytest.skip("empty state")
    before = {q: (m.table(q), m.length(q)) for q in group}
    counts = {b: m.refcount[b] for q in group for b in m.table(q)}
    out = m.swap_out(group)
    assert len(out) == len({b for q in group for b in before[q][0]})
    snap = (list(m.free), list(m.refcount), list(m.host_free), list(m.host_refcount))
    try:
        m.swap_in(group)
    except OOM:
        # blocks shared with sequences outside the group stayed on the device,
        # so the pool can be short: nothing changed; make room and retry
        assert snap == (list(m.free), list(m.refcount), list(m.host_free), list(m.host_refcount))
        for q in [q for q in m.seqs if q not in group]:
            m.free_sequence(q)
        m.swap_in(group)
    relabel = {}
    for q in group:
        t0, n0 = before[q]
        t1 = m.table(q)
        assert len(t1) == len(t0) and m.length(q) == n0
        for a, b in zip(t0, t1):
            assert relabel.setdefault(a, b) == b
    assert len(set(relabel.values())) == len(relabel)
    holders = {b: sum(b in before[q][0] for q in group) for b in relabel}
    for a, b in relabel.items():
        assert m.refcount[b] == holders[a]            # the group's share of the old count
        assert holders[a] <= counts[a]
    m.check_invariants()


# ---------------------------------------------------------------------------
# prefix sharing across requests ([n1n] 前缀缓存: 100 requests with one long
# system prompt share its physical blocks; [lpnh-1824136] 3.2 second step)
# ---------------------------------------------------------------------------
def test_hundred_requests_share_one_system_prompt():
    """The page's example, counted: a 1000-token system prompt (62 full
    blocks of 16 + an 8-token tail) followed by each request's own text.
    The 62 full blocks exist once with count 100; every request owns only
    the blocks holding its tail and its own tokens."""
    import numpy as np
    rng = np.random.default_rng(0)
    B, P, R = 16, 1000, 100
    system = rng.integers(0, 32000, size=P).tolist()
    suffix_lens = rng.integers(1, 200, size=R).tolist()
    m = BlockManagerModel(20000, B)
    cached = []
    for r in range(R):
        toks = system + rng.integers(0, 32000, size=suffix_lens[r]).tolist()
        _, nc = m.add_sequence_cached(r, toks)
        cached.append(nc)
    full = P // B
    assert cached == [0] + [full * B] * (R - 1)
    shared = m.table(0)[:full]
    assert all(m.table(r)[:full] == shared for r in range(R))
    assert all(m.refcount[b] == R for b in shared)
    used = 20000 - m.num_free()
    want = full + sum(-(-(P + s) // B) - full for s in suffix_lens)
    assert used == want
    unshared = sum(-(-(P + s) // B) for s in suffix_lens)
    assert unshared - used == (R - 1) * full        # the prefix is stored once, not 100 times
    m.check_invariants()


def test_divergence_inside_a_block_shares_the_blocks_before_it():
    m = BlockManagerModel(32, 4)
    a = list(range(100, 114))                      # 3 full blocks + 2 tokens
    m.add_sequence_cached(0, a)
    b = a[:9] + [7, 7, 7, 7, 7]                    # differs at position 9, inside block 2
    _, nc = m.add_sequence_cached(1, b)
    assert nc == 8 and m.table(1)[:2] == m.table(0)[:2] and m.table(1)[2] != m.table(0)[2]
    _, nc = m.add_sequence_cached(2, a[:3])         # shorter than one block: nothing shared
    assert nc == 0 and not set(m.table(2)) & set(m.table(0))
    c = [9] * 4 + a[4:8]                           # same tokens as block 1 of `a`, another block 0
    _, nc = m.add_sequence_cached(3, c)
    assert nc == 0 and m.table(3)[1] != m.table(0)[1]   # the key chains through the block before
    m.check_invariants()


def test_fully_shared_prompt_appends_without_copy_and_index_forgets_freed_blocks():
    m = BlockManagerModel(16, 4)
    p = [1, 2, 3, 4, 5, 6, 7, 8]
    m.add_sequence_cached(0, p)
    _, nc = m.add_sequence_cached(1, p)
    assert nc == 8 and m.table(1) == m.table(0)
    slot, cow = m.append_token(1)                  # the shared last block is full: fresh block
    assert cow is None and m.table(1)[:2] == m.table(0)[:2] and len(m.table(1)) == 3
    assert len(m.prefix_index) == 2
    m.free_sequence(0)
    assert len(m.prefix_index) == 2                # sequence 1 still holds both blocks
    m.free_sequence(1)
    assert m.prefix_index == {} and m.num_free() == 16
    _, nc = m.add_sequence_cached(2, p)
    assert nc == 0
    m.check_invariants()


def test_cached_add_oom_changes_nothing():
    m = BlockManagerModel(3, 4)
    m.add_sequence_cached(0, list(range(8)))       # 2 blocks, both indexed
    snap = (list(m.free), list(m.refcount), dict(m.prefix_index))
    import pytest as _pytest
    with _pytest.raises(OOM):
        m.add_sequence_cached(1, list(range(8)) + list(range(50, 59)))   # 2 shared + 3 new > 1 free
    assert snap == (list(m.free), list(m.refcount), dict(m.prefix_index))
    m.check_invariants()
