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
