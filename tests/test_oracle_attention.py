"""Pins for the oracle's decode attention.

The pages print no attention values, so the oracle is tied to things other
than itself: torch's scaled_dot_product_attention in float64 (a library
routine) on the logically contiguous K/V, closed forms (one token, a zero
query, two tokens), bitwise invariances that paging must have (relabelled
physical blocks, another block size, the unpaged layout) and the IEEE
half-precision decoder checked against numpy for every bit pattern.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.block_manager import BlockManagerModel


def test_half_decoder_matches_numpy_for_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    L = oracle.lib()
    got = np.array([L.oracle_half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, L.oracle_half_to_double(0x8000)) == -1.0


def _paged_problem(seed, lens, H, Hkv, D, B, NB, poison=True):
    """Logical K/V per sequence, placed into a paged cache by the layout's
    definition: token p of sequence s sits in block table[s][p // B], head
    slab h, row p % B."""
    rng = np.random.default_rng(seed)                 # values: independent of B and NB
    S = len(lens)
    width = max(1, max(-(-n // B) for n in lens))
    perm = np.random.default_rng([seed, B, NB]).permutation(NB)
    tables = np.full((S, width), -1, dtype=np.int32)
    at = 0
    for s, n in enumerate(lens):
        nb = -(-n // B)
        tables[s, :nb] = perm[at:at + nb]
        at += nb
    assert at <= NB
    kc = np.full((NB, Hkv, B, D), np.nan if poison else 0, dtype=np.float16)
    vc = kc.copy()
    Ks, Vs = [], []
    for s, n in enumerate(lens):
        K = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        V = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        Ks.append(K)
        Vs.append(V)
        for p in range(n):
            kc[tables[s, p // B], :, p % B, :] = K[p]
            vc[tables[s, p // B], :, p % B, :] = V[p]
    q = rng.standard_normal((S, H, D)).astype(np.float16)
    return q, kc, vc, tables, np.array(lens, dtype=np.int32), Ks, Vs


def _sdpa(q, K, V, H, Hkv, scale):
    """torch SDPA in float64 for one sequence; K/V [n, Hkv, D]."""
    g = H // Hkv
    qt = torch.from_numpy(q.astype(np.float64)).unsqueeze(1)           # [H, 1, D]
    kt = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2)       # [Hkv, n, D]
    vt = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2)
    kt = kt.repeat_interleave(g, dim=0).contiguous()
    vt = vt.repeat_interleave(g, dim=0).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o.squeeze(1).numpy()


@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 2), (8, 1)])
@pytest.mark.parametrize("B", [1, 4, 16])
def test_matches_library_attention(H, Hkv, B):
    lens = [1, 3, 17, 40, 64, 5]
    D = 16
    q, kc, vc, tables, lens_a, Ks, Vs = _paged_problem(7, lens, H, Hkv, D, B, 80 * 16 // B + 8)
    scale = 0.3
    out = oracle.decode(q, kc, vc, tables, lens_a, scale)
    for s in range(len(lens)):
        ref = _sdpa(q[s], Ks[s], Vs[s], H, Hkv, scale)
        np.testing.assert_allclose(out[s], ref, rtol=1e-12, atol=1e-12)


def test_single_token_returns_its_value_exactly():
    q, kc, vc, tables, lens, Ks, Vs = _paged_problem(1, [1, 1], 2, 2, 16, 4, 8)
    out = oracle.decode(q, kc, vc, tables, lens, 0.25)
    for s in range(2):
        assert np.array_equal(out[s], Vs[s][0].astype(np.float64))


def test_zero_query_is_the_mean_of_values():
    q, kc, vc, tables, lens, Ks, Vs = _paged_problem(2, [9, 33], 2, 2, 16, 4, 32)
    q[:] = 0
    out = oracle.decode(q, kc, vc, tables, lens, 0.25)
    for s in range(2):
        np.testing.assert_allclose(out[s], Vs[s].astype(np.float64).mean(axis=0),
                                   rtol=0, atol=1e-14)


def test_two_tokens_closed_form():
    q, kc, vc, tables, lens, Ks, Vs = _paged_problem(3, [2], 2, 2, 16, 4, 4)
    scale = 0.25
    out = oracle.decode(q, kc, vc, tables, lens, scale)
    K, V = Ks[0].astype(np.float64), Vs[0].astype(np.float64)
    for h in range(2):
        qh = q[0, h].astype(np.float64)
        delta = scale * (qh @ (K[1, h] - K[0, h]))
        ref = (V[0, h] + math.exp(delta) * V[1, h]) / (1.0 + math.exp(delta))
        np.testing.assert_allclose(out[0, h], ref, rtol=1e-13, atol=1e-14)


def test_relabelling_physical_blocks_is_bitwise_invisible():
    lens = [5, 30, 47, 1]
    q, kc, vc, tables, lens_a, _, _ = _paged_problem(4, lens, 4, 2, 16, 4, 64)
    base = oracle.decode(q, kc, vc, tables, lens_a, 0.25)
    sigma = np.random.default_rng(11).permutation(64)          # old id -> new id
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[sigma] = kc
    vc2[sigma] = vc
    t2 = np.where(tables >= 0, sigma[np.maximum(tables, 0)], -1).astype(np.int32)
    again = oracle.decode(q, kc2, vc2, t2, lens_a, 0.25)
    assert np.array_equal(base, again)


def test_block_size_is_bitwise_invisible():
    lens = [7, 40, 64]
    outs = []
    for B in (1, 2, 4, 8, 16):
        q, kc, vc, tables, lens_a, _, _ = _paged_problem(5, lens, 2, 2, 16, B, 120 * 16 // B)
        outs.append(oracle.decode(q, kc, vc, tables, lens_a, 0.25))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_paged_equals_unpaged_bitwise():
    lens = [3, 18, 44]
    q, kc, vc, tables, lens_a, Ks, Vs = _paged_problem(6, lens, 4, 4, 16, 4, 32)
    paged = oracle.decode(q, kc, vc, tables, lens_a, 0.25)
    k = np.ascontiguousarray(np.concatenate(Ks))
    v = np.ascontiguousarray(np.concatenate(Vs))
    starts = np.array([0, 3, 21], dtype=np.int64)
    flat = oracle.attention_contig(q, k, v, starts, lens_a, 0.25)
    assert np.array_equal(paged, flat)


def test_empty_sequence_gives_zeros():
    q, kc, vc, tables, lens, _, _ = _paged_problem(8, [0, 4], 2, 2, 16, 4, 8)
    out = oracle.decode(q, kc, vc, tables, lens, 0.25)
    assert np.array_equal(out[0], np.zeros((2, 16)))
    assert np.all(np.isfinite(out[1]))


def test_poisoned_unused_slots_never_leak():
    # every unused slot is NaN; a correct gather reads only the first n tokens
    q, kc, vc, tables, lens, _, _ = _paged_problem(9, [1, 2, 3, 5, 7], 2, 2, 16, 4, 16)
    out = oracle.decode(q, kc, vc, tables, lens, 0.25)
    assert np.all(np.isfinite(out))


def test_table_entry_outside_pool_is_an_error():
    q, kc, vc, tables, lens, _, _ = _paged_problem(10, [5], 2, 2, 16, 4, 4)
    tables[0, 1] = 4
    with pytest.raises(RuntimeError):
        oracle.decode(q, kc, vc, tables, lens, 0.25)


def test_threads_do_not_change_bits():
    lens = [50, 12, 33, 1, 64]
    q, kc, vc, tables, lens_a, _, _ = _paged_problem(12, lens, 4, 2, 16, 4, 64)
    one = oracle.decode(q, kc, vc, tables, lens_a, 0.25, nthreads=1)
    many = oracle.decode(q, kc, vc, tables, lens_a, 0.25, nthreads=7)
    assert np.array_equal(one, many)


def test_block_manager_slots_feed_the_oracle():
    """End to end on the CPU: the model's slots, the oracle's scatter and the
    oracle's paged decode agree with library attention on the logical K/V."""
    rng = np.random.default_rng(13)
    B, NB, H, Hkv, D = 4, 40, 2, 2, 16
    m = BlockManagerModel(NB, B)
    lens = [6, 13, 20]
    Ks, Vs = [], []
    kc = np.full((NB, Hkv, B, D), np.nan, dtype=np.float16)
    vc = kc.copy()
    for s, n in enumerate(lens):
        slots = np.array(m.add_sequence(s, n), dtype=np.int64)
        K = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        V = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        oracle.reshape_and_cache(K, V, slots, kc, vc)
        Ks.append(K)
        Vs.append(V)
    rows, ls = m.tables(range(3), 5)
    q = rng.standard_normal((3, H, D)).astype(np.float16)
    out = oracle.decode(q, kc, vc, np.array(rows, dtype=np.int32), np.array(ls, dtype=np.int32), 0.25)
    for s in range(3):
        np.testing.assert_allclose(out[s], _sdpa(q[s], Ks[s], Vs[s], H, Hkv, 0.25), rtol=1e-12, atol=1e-12)
