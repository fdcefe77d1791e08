"""GPU checks of pa_prefill / pa_prefill_append given a dispatch order
(seq_order).

The order decides only which sequences' row tiles start first (longest
first, so that no long prompt starts last and runs alone at the end); each
row tile computes the same thing wherever it runs.  So outputs and cache
writes are compared bit for bit with index order (seq_order NULL) in every
grid form -- (KV head, sequence) pairs fastest, XCD-grouped, a split context
with its merge kernel, the persistent grid -- and index order against the
oracle on the small batches.  An order entry outside [0, num_seqs) is
skipped: a sequence the order leaves out keeps its output rows and (with
append) its new tokens' cache slots untouched."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_390_amd as pa
import workloads
from gpu_common import assert_attention_close, bits, device, say
from test_gpu_decode import _oracle_cache
from test_gpu_prefill import LENS, SHORT_CHUNKS, _append_case, _queries
from test_gpu_prefill_persistent import CASES as PERSISTENT_CASES

pytestmark = pytest.mark.gpu

SENTINEL = 3.0


def _case(name):
    """(case, new-token counts, workspace wanted): 10 sequences with 2 KV
    heads (20 pairs: pairs fastest) or 4 (40: XCD-grouped), 3 long contexts
    with short chunks (split context), and a persistent-grid batch."""
    if name == "pairs fastest":
        return workloads.random_case(1501, LENS, 8, 2, 128, 16), list(LENS)
    if name == "xcd grouped":
        return workloads.random_case(1502, LENS, 8, 4, 64, 16), [max(1, n // 3) for n in LENS]
    if name == "split context":
        return workloads.random_case(1503, [3000, 2500, 1777], 8, 2, 128, 16), list(SHORT_CHUNKS)
    lens_l, H, Hkv, D, B, _, _ = PERSISTENT_CASES["d128 16 heads"]
    return workloads.random_case(1504, lens_l, H, Hkv, D, B), list(lens_l)


def _orders(lens, dev):
    """Longest first as pa_decode_order writes it, shortest first, and a
    random permutation."""
    S = len(lens)
    d_l = torch.from_numpy(lens).to(dev)
    longest = pa.pa_decode_order(d_l, int(lens.max()))
    torch.cuda.synchronize()
    lf = longest.cpu().numpy()
    assert sorted(lf.tolist()) == list(range(S))
    assert np.all(np.diff(lens[lf]) <= int(lens.max()) // 1024 + 1)     # longest class first
    return {"longest first": longest,
            "shortest first": torch.from_numpy(np.ascontiguousarray(lf[::-1])).to(dev),
            "random": torch.from_numpy(np.random.default_rng(S).permutation(S).astype(np.int32)).to(dev)}


def _prefill(dev, q, kc, vc, tables, lens, qs, scale, mq, order=None, fill=float("nan")):
    out = torch.full(q.shape, fill, dtype=torch.float16, device=dev)
    pa.pa_prefill(out, q, kc, vc, tables, lens, qs, scale, max_query_len=mq, seq_order=order)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["pairs fastest", "xcd grouped", "split context", "persistent"])
def test_prefill_order_changes_no_bit(name):
    dev = device()
    case, ms = _case(name)
    kc_h, vc_h, tables_h, lens_h = _oracle_cache(case)
    H, D = case.num_heads, case.head_dim
    q_h, qs_h = _queries(1500 + len(name), ms, H, D)
    mq = max(ms)
    need = pa.pa_prefill_workspace_size(int(qs_h[-1]), len(ms), H, case.num_kv_heads, D, case.block_size,
                                        tables_h.shape[1], mq)
    say(f"prefill order {name}: rows {int(qs_h[-1])}, workspace {need} bytes")
    if name == "split context":
        assert need > 256                                 # partial states: the merge kernel runs
    if name == "persistent":
        assert need == 256                                # the claim counters
    kc, vc, q = (torch.from_numpy(x).to(dev) for x in (kc_h, vc_h, q_h))
    t, l, qs = (torch.from_numpy(x).to(dev) for x in (tables_h, lens_h, qs_h))
    ref = _prefill(dev, q, kc, vc, t, l, qs, case.scale, mq)
    if name != "persistent":
        assert_attention_close(ref, oracle.prefill(q_h, kc_h, vc_h, tables_h, lens_h, qs_h, case.scale),
                               f"index order, {name}")
    for what, order in _orders(lens_h, dev).items():
        out = _prefill(dev, q, kc, vc, t, l, qs, case.scale, mq, order)
        assert np.array_equal(bits(out), bits(ref)), f"{name}: {what} differs from index order"
    # entries outside the batch: sequences 1 and 2 left out, their rows untouched
    S = len(ms)
    partial = np.arange(S, dtype=np.int32)[::-1].copy()
    partial[partial == 1] = -1
    partial[partial == 2] = S
    out = _prefill(dev, q, kc, vc, t, l, qs, case.scale, mq, torch.from_numpy(partial).to(dev), fill=SENTINEL)
    o, r = bits(out), bits(ref)
    for s in range(S):
        a, b = int(qs_h[s]), int(qs_h[s + 1])
        if s in (1, 2):
            assert np.all(out[a:b].cpu().numpy() == np.float16(SENTINEL)), f"{name}: sequence {s} was written"
        else:
            assert np.array_equal(o[a:b], r[a:b]), f"{name}: sequence {s}"


def test_prefill_append_order_changes_no_bit():
    """pa_prefill_append with orders: outputs and caches bit for bit as in
    index order and the caches equal to the oracle's scatter; with sequences
    left out, their new tokens' slots keep the cache's prior contents."""
    dev = device()
    case = workloads.random_case(1510, LENS, 8, 4, 128, 16)
    ms = [max(1, n // 2) for n in LENS]
    kc0, vc0, kc1, vc1, key_h, val_h, tables_h, lens_h = _append_case(case, ms)
    q_h, qs_h = _queries(1510, ms, 8, 128)
    q, key, val = (torch.from_numpy(x).to(dev) for x in (q_h, key_h, val_h))
    t, l, qs = (torch.from_numpy(x).to(dev) for x in (tables_h, lens_h, qs_h))
    say(f"prefill_append order: rows {int(qs_h[-1])}")

    def run(order, fill=float("nan")):
        kc, vc = torch.from_numpy(kc0).to(dev), torch.from_numpy(vc0).to(dev)
        out = torch.full(q.shape, fill, dtype=torch.float16, device=dev)
        pa.pa_prefill_append(out, q, key, val, kc, vc, t, l, qs, case.scale, max_query_len=max(ms),
                             seq_order=order)
        torch.cuda.synchronize()
        return bits(out), bits(kc), bits(vc)

    ro, rk, rv = run(None)
    assert np.array_equal(rk, kc1.view(np.uint16)) and np.array_equal(rv, vc1.view(np.uint16))
    assert_attention_close(ro.view(np.float16), oracle.prefill(q_h, kc1, vc1, tables_h, lens_h, qs_h, case.scale),
                           "append, index order")
    for what, order in _orders(lens_h, dev).items():
        o, k, v = run(order)
        assert np.array_equal(o, ro) and np.array_equal(k, rk) and np.array_equal(v, rv), what
    S = len(ms)
    partial = np.arange(S, dtype=np.int32)
    partial[4] = -7
    o, k, v = run(torch.from_numpy(partial).to(dev), fill=SENTINEL)
    a, b = int(qs_h[4]), int(qs_h[5])
    assert np.all(o[a:b].view(np.float16) == np.float16(SENTINEL))
    keep = np.r_[0:a, b:int(qs_h[-1])]
    assert np.array_equal(o[keep], ro[keep])
    # sequence 4's new slots still hold what the cache held before the call
    # (NaN); every other slot as in index order
    blocks4 = tables_h[4][tables_h[4] >= 0]
    others = np.setdiff1d(np.arange(case.num_blocks), blocks4)
    assert np.array_equal(k[others], rk[others]) and np.array_equal(v[others], rv[others])
    assert np.array_equal(k[blocks4], kc0.view(np.uint16)[blocks4])
    assert np.array_equal(v[blocks4], vc0.view(np.uint16)[blocks4])


def test_prefill_order_must_have_one_entry_per_sequence():
    dev = device()
    case, ms = _case("pairs fastest")
    kc_h, vc_h, tables_h, lens_h = _oracle_cache(case)
    q_h, qs_h = _queries(1520, ms, case.num_heads, case.head_dim)
    kc, vc, q = (torch.from_numpy(x).to(dev) for x in (kc_h, vc_h, q_h))
    t, l, qs = (torch.from_numpy(x).to(dev) for x in (tables_h, lens_h, qs_h))
    with pytest.raises(ValueError):
        pa.pa_prefill(torch.empty_like(q), q, kc, vc, t, l, qs, case.scale,
                      seq_order=torch.zeros(len(ms) - 1, dtype=torch.int32, device=dev))
