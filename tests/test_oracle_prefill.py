"""Pins for the oracle's paged prefill (several new tokens per sequence,
each attending causally to the cached positions up to its own).

Tied to things other than itself: torch's scaled_dot_product_attention in
float64 with a causal / position mask on the logically contiguous K/V (a
library routine), decode (one new token per sequence), and invariance under
relabelling of the physical blocks."""
import numpy as np
import pytest
import torch

import oracle
from test_oracle_attention import _paged_problem


def _queries(seed, ms, H, D):
    rng = np.random.default_rng([seed, 99])
    T = int(sum(ms))
    q = rng.standard_normal((T, H, D)).astype(np.float16)
    qs = np.concatenate([[0], np.cumsum(ms)]).astype(np.int32)
    return q, qs


def _sdpa(q, Ks, Vs, lens, ms, qs, H, Hkv, scale):
    """torch SDPA (float64) per sequence: queries at positions n-m..n-1,
    mask[i, t] = t <= n - m + i; KV heads repeated for grouped queries."""
    out = np.zeros(q.shape, dtype=np.float64)
    g = H // Hkv
    for s, (n, m) in enumerate(zip(lens, ms)):
        if m == 0:
            continue
        Q = torch.from_numpy(q[qs[s]:qs[s + 1]].astype(np.float64)).permute(1, 0, 2)        # [H, m, D]
        K = torch.from_numpy(Ks[s].astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)
        V = torch.from_numpy(Vs[s].astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)
        pos = torch.arange(n - m, n).unsqueeze(1)
        mask = torch.arange(n).unsqueeze(0) <= pos                                           # [m, n]
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
        out[qs[s]:qs[s + 1]] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("H,Hkv", [(4, 4), (8, 2)])
@pytest.mark.parametrize("B", [1, 4, 16])
def test_full_and_chunked_prefill_match_library_attention(H, Hkv, B):
    D = 16
    lens = [1, 7, 33, 40, 70]
    ms = [1, 7, 10, 40, 25]                 # full prefill where m == n, chunked where m < n
    q0, kc, vc, tables, L, Ks, Vs = _paged_problem(3, lens, H, Hkv, D, B, NB=200)
    q, qs = _queries(3, ms, H, D)
    scale = 1 / np.sqrt(D)
    got = oracle.prefill(q, kc, vc, tables, L, qs, scale)
    want = _sdpa(q, Ks, Vs, lens, ms, qs, H, Hkv, scale)
    assert np.max(np.abs(got - want)) < 1e-12


def test_full_prefill_matches_is_causal_attention():
    """n == m for every sequence: torch's own causal flag, no mask built."""
    H = Hkv = 2
    D, B = 8, 4
    lens = [13, 5]
    q0, kc, vc, tables, L, Ks, Vs = _paged_problem(8, lens, H, Hkv, D, B, NB=40)
    q, qs = _queries(8, lens, H, D)
    got = oracle.prefill(q, kc, vc, tables, L, qs, 0.3)
    for s, n in enumerate(lens):
        Q = torch.from_numpy(q[qs[s]:qs[s + 1]].astype(np.float64)).permute(1, 0, 2)
        K = torch.from_numpy(Ks[s].astype(np.float64)).permute(1, 0, 2)
        V = torch.from_numpy(Vs[s].astype(np.float64)).permute(1, 0, 2)
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=0.3)
        assert np.max(np.abs(got[qs[s]:qs[s + 1]] - o.permute(1, 0, 2).numpy())) < 1e-12


def test_one_new_token_is_decode():
    H, Hkv, D, B = 4, 2, 16, 4
    lens = [9, 1, 30]
    q0, kc, vc, tables, L, Ks, Vs = _paged_problem(5, lens, H, Hkv, D, B, NB=40)
    q, qs = _queries(5, [1, 1, 1], H, D)
    got = oracle.prefill(q, kc, vc, tables, L, qs, 0.25)
    want = oracle.decode(q, kc, vc, tables, L, 0.25)
    assert np.array_equal(got, want)


def test_prefill_is_blind_to_physical_placement():
    H, Hkv, D, B = 4, 4, 16, 4
    lens = [37, 12]
    q0, kc, vc, tables, L, Ks, Vs = _paged_problem(6, lens, H, Hkv, D, B, NB=30)
    q, qs = _queries(6, [20, 12], H, D)
    a = oracle.prefill(q, kc, vc, tables, L, qs, 0.25)
    sigma = np.random.default_rng(1).permutation(30)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[sigma], vc2[sigma] = kc, vc
    t2 = np.where(tables >= 0, sigma[np.maximum(tables, 0)], -1).astype(np.int32)
    b = oracle.prefill(q, kc2, vc2, t2, L, qs, 0.25)
    assert np.array_equal(a, b)


def test_prefill_rejects_inconsistent_query_ranges():
    H, D, B = 2, 8, 4
    q0, kc, vc, tables, L, Ks, Vs = _paged_problem(7, [5], H, H, D, B, NB=8)
    q, qs = _queries(7, [6], H, D)                     # 6 new tokens but only 5 cached
    with pytest.raises(RuntimeError):
        oracle.prefill(q, kc, vc, tables, L, qs, 0.5)
