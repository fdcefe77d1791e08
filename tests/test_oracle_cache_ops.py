"""Pins for the oracle's scatter and block copy: round trips against the
layout's definition, untouched bytes, skipped slots and simultaneous copies."""
import numpy as np
import pytest

import oracle
from oracle.block_manager import BlockManagerModel


def _poisoned(NB, Hkv, B, D, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 16, size=(NB, Hkv, B, D), dtype=np.uint16)
    return bits.view(np.float16)


def test_scatter_round_trip_and_untouched_bytes():
    NB, Hkv, B, D = 20, 3, 4, 16
    kc, vc = _poisoned(NB, Hkv, B, D, 1), _poisoned(NB, Hkv, B, D, 2)
    k0, v0 = kc.copy(), vc.copy()
    m = BlockManagerModel(NB, B)
    slots = np.array(m.add_sequence(0, 11) + m.add_sequence(1, 6), dtype=np.int64)
    rng = np.random.default_rng(3)
    key = rng.standard_normal((17, Hkv, D)).astype(np.float16)
    val = rng.standard_normal((17, Hkv, D)).astype(np.float16)
    oracle.reshape_and_cache(key, val, slots, kc, vc)
    touched = np.zeros((NB, B), dtype=bool)
    for t, s in enumerate(slots):
        assert np.array_equal(kc[s // B, :, s % B, :].view(np.uint16), key[t].view(np.uint16))
        assert np.array_equal(vc[s // B, :, s % B, :].view(np.uint16), val[t].view(np.uint16))
        touched[s // B, s % B] = True
    mask = ~touched
    assert np.array_equal(kc.view(np.uint16).transpose(0, 2, 1, 3)[mask],
                          k0.view(np.uint16).transpose(0, 2, 1, 3)[mask])
    assert np.array_equal(vc.view(np.uint16).transpose(0, 2, 1, 3)[mask],
                          v0.view(np.uint16).transpose(0, 2, 1, 3)[mask])


def test_scatter_skips_negative_slots():
    NB, Hkv, B, D = 4, 1, 4, 16
    kc, vc = _poisoned(NB, Hkv, B, D, 4), _poisoned(NB, Hkv, B, D, 5)
    k0 = kc.copy()
    key = np.ones((2, Hkv, D), dtype=np.float16)
    oracle.reshape_and_cache(key, key, np.array([-1, 5], dtype=np.int64), kc, vc)
    assert np.all(kc[1, 0, 1] == 1)
    changed = np.argwhere(kc.view(np.uint16) != k0.view(np.uint16))
    assert set(map(tuple, changed[:, :3])) <= {(1, 0, 1)}


def test_scatter_rejects_slot_outside_pool():
    kc, vc = _poisoned(2, 1, 4, 16, 6), _poisoned(2, 1, 4, 16, 7)
    key = np.ones((1, 1, 16), dtype=np.float16)
    with pytest.raises(RuntimeError):
        oracle.reshape_and_cache(key, key, np.array([8], dtype=np.int64), kc, vc)


def test_copy_blocks_all_layers_simultaneous():
    NB, Hkv, B, D, L = 12, 2, 4, 16, 3
    ks = [_poisoned(NB, Hkv, B, D, 10 + i) for i in range(L)]
    vs = [_poisoned(NB, Hkv, B, D, 20 + i) for i in range(L)]
    k0 = [a.copy() for a in ks]
    v0 = [a.copy() for a in vs]
    pairs = np.array([[3, 7], [3, 8], [5, 1]], dtype=np.int64)   # a source may repeat
    oracle.copy_blocks(ks, vs, pairs)
    for l in range(L):
        for a, a0 in ((ks[l], k0[l]), (vs[l], v0[l])):
            for src, dst in pairs:
                assert np.array_equal(a[dst].view(np.uint16), a0[src].view(np.uint16))
            others = [b for b in range(NB) if b not in set(pairs[:, 1])]
            assert np.array_equal(a[others].view(np.uint16), a0[others].view(np.uint16))


def test_copy_blocks_rejects_ids_outside_pool():
    ks = [_poisoned(4, 1, 4, 16, 30)]
    with pytest.raises(RuntimeError):
        oracle.copy_blocks(ks, [ks[0].copy()], np.array([[0, 4]], dtype=np.int64))


def test_copy_then_write_matches_cow_semantics():
    """COW on the CPU: after the copy, writing the forked sample's next token
    leaves the parent's view of the shared block unchanged."""
    NB, Hkv, B, D = 8, 1, 4, 16
    m = BlockManagerModel(NB, B)
    rng = np.random.default_rng(31)
    kc = np.zeros((NB, Hkv, B, D), dtype=np.float16)
    vc = kc.copy()
    slots = np.array(m.add_sequence(0, 6), dtype=np.int64)
    kv = rng.standard_normal((6, Hkv, D)).astype(np.float16)
    oracle.reshape_and_cache(kv, kv, slots, kc, vc)
    m.fork(0, 1)
    slot, cow = m.append_token(1)
    assert cow is not None
    parent_tail = kc[cow[0]].copy()
    oracle.copy_blocks([kc], [vc], np.array([cow], dtype=np.int64))
    new = rng.standard_normal((1, Hkv, D)).astype(np.float16)
    oracle.reshape_and_cache(new, new, np.array([slot], dtype=np.int64), kc, vc)
    assert np.array_equal(kc[cow[0]].view(np.uint16), parent_tail.view(np.uint16))
    assert np.array_equal(kc[cow[1], :, :2].view(np.uint16), parent_tail[:, :2].view(np.uint16))
    assert np.array_equal(kc[cow[1], :, 2].view(np.uint16), new[0].view(np.uint16))


def test_move_blocks_matches_elementwise_copy_and_round_trips():
    """The swap data movement: every element of a destination block equals
    the source block's element (checked one element at a time), untouched
    blocks keep their bytes, and out-then-in restores the blocks."""
    rng = np.random.default_rng(5)
    dev = [rng.standard_normal((6, 2, 4, 8)).astype(np.float16) for _ in range(3)]
    host = [np.full((5, 2, 4, 8), np.nan, dtype=np.float16) for _ in range(3)]
    pairs = np.array([[4, 0], [1, 3], [5, 2]], dtype=np.int64)
    before_host = [h.copy() for h in host]
    oracle.move_blocks(host, dev, pairs)
    for i in range(3):
        for s, d in pairs.tolist():
            for idx in np.ndindex(dev[i].shape[1:]):
                assert host[i][(d,) + idx].view(np.uint16) == dev[i][(s,) + idx].view(np.uint16)
        untouched = [b for b in range(5) if b not in pairs[:, 1]]
        assert np.array_equal(host[i][untouched].view(np.uint16), before_host[i][untouched].view(np.uint16))
    back = [np.zeros_like(d) for d in dev]
    oracle.move_blocks(back, host, pairs[:, ::-1].copy())
    for i in range(3):
        assert np.array_equal(back[i][pairs[:, 0]].view(np.uint16), dev[i][pairs[:, 0]].view(np.uint16))
    with pytest.raises(ValueError):
        oracle.move_blocks(host, dev, np.array([[0, 1], [2, 1]], dtype=np.int64))
    with pytest.raises(ValueError):
        oracle.move_blocks(host, dev, np.array([[6, 1]], dtype=np.int64))
