"""GPU parity of pa_prefill (several new tokens per sequence, causal over the
paged cache, matrix-core kernel) against the oracle, through the C ABI.

Caches are built on the host by the oracle (model slots + oracle scatter, NaN
in every unused slot) and uploaded, so these tests isolate the kernel; the
full-size case writes the prompt with the product's scatter first."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_390_amd as pa
import workloads
from gpu_common import assert_attention_close, bits, device, say
from oracle.block_manager import BlockManagerModel
from test_gpu_decode import _oracle_cache

pytestmark = pytest.mark.gpu


def _queries(seed, ms, H, D):
    rng = np.random.default_rng([seed, 77])
    q = rng.standard_normal((int(sum(ms)), H, D), dtype=np.float32).astype(np.float16)
    return q, np.concatenate([[0], np.cumsum(ms)]).astype(np.int32)


def _gpu_prefill(dev, q, kc, vc, tables, lens, qs, scale, max_query_len=None, split=True, workspace=None):
    out = torch.full(q.shape, float("nan"), dtype=torch.float16, device=dev)
    pa.pa_prefill(out, torch.from_numpy(q).to(dev), torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev),
                  torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev), torch.from_numpy(qs).to(dev),
                  scale, max_query_len=max_query_len, split=split, workspace=workspace)
    torch.cuda.synchronize()
    return out


LENS = [1, 2, 15, 16, 17, 33, 64, 100, 129, 300]


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("B", [1, 4, 8, 16, 32, 128])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (8, 2), (6, 3), (4, 4), (8, 4)])
@pytest.mark.parametrize("chunk", ["full", "chunked", "decode"])
def test_prefill_matches_oracle(D, B, H, Hkv, chunk):
    """10 sequences: with 2 or 3 KV heads the (KV head, sequence) pairs are
    not a multiple of 8 and the grid takes the pair fastest; with 4 they are
    (40) and the grid is XCD-grouped.  head_dim 64 / 128 / 256 (K/V tiles of
    64, 64 and 32 tokens; 32, 32 and 16 query rows per wave)."""
    dev = device()
    case = workloads.random_case(900 + B + 10 * H + Hkv + D, LENS, H, Hkv, D, B)
    kc, vc, tables, lens = _oracle_cache(case)
    if chunk == "full":
        ms = list(LENS)
    elif chunk == "chunked":
        ms = [max(1, n // 3) for n in LENS]
    else:
        ms = [1] * len(LENS)
    q, qs = _queries(B + H, ms, H, D)
    say(f"prefill D={D} B={B} H={H}/{Hkv} {chunk}: rows {int(qs[-1])}")
    out = _gpu_prefill(dev, q, kc, vc, tables, lens, qs, case.scale)
    ref = oracle.prefill(q, kc, vc, tables, lens, qs, case.scale)
    assert_attention_close(out, ref, f"prefill D={D} B={B} H={H}/{Hkv} {chunk}")
    if chunk == "decode":                                     # one new token per sequence is decode
        dec = torch.empty_like(out)
        pa.pa_decode(dec, torch.from_numpy(q).to(dev), torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev),
                     torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev), case.scale)
        torch.cuda.synchronize()
        assert_attention_close(dec, ref, "decode of the same rows")


def test_prefill_edge_rows_and_bad_sequences():
    """Empty sequences, a sequence whose new tokens exceed its context (NaN
    rows), one beyond max_query_len (NaN for the covered rows), and one whose
    query range leaves [0, T) (skipped: rows untouched)."""
    dev = device()
    case = workloads.random_case(31, [40, 10, 20, 30], 4, 2, 128, 16)
    kc, vc, tables, lens = _oracle_cache(case)
    ms = [40, 0, 25, 5]                                        # seq 2: 25 new > 20 cached
    q, qs = _queries(31, ms, 4, 128)
    out = _gpu_prefill(dev, q, kc, vc, tables, lens, qs, case.scale)
    # rows 0..39: sequence 0; 40..64: sequence 2 (NaN); 65..69: sequence 3
    ref = np.full(q.shape, np.nan)
    sel = np.r_[0:40, 65:70]
    ref[sel] = oracle.prefill(np.ascontiguousarray(q[sel]), kc, vc, np.ascontiguousarray(tables[[0, 3]]),
                              np.ascontiguousarray(lens[[0, 3]]), np.array([0, 40, 45], np.int32), case.scale)
    assert_attention_close(out, ref, "edge rows")
    # max_query_len 30: sequence 0 (40 new tokens) is out of bounds -> its first 30 rows NaN, the rest untouched
    out2 = _gpu_prefill(dev, q, kc, vc, tables, lens, qs, case.scale, max_query_len=30)
    o2 = out2.float().cpu().numpy()
    assert np.all(np.isnan(o2[0:30])) and np.all(np.isnan(o2[30:40]))   # (untouched rows stay NaN too)
    assert_attention_close(out2[65:70], ref[65:70], "other sequences unaffected")
    # a query range outside [0, T): sequence skipped, nothing written for it
    bad_qs = qs.copy()
    bad_qs[4] = int(qs[-1]) + 3
    out3 = torch.zeros(q.shape, dtype=torch.float16, device=dev)
    pa.pa_prefill(out3, torch.from_numpy(q).to(dev), torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev),
                  torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev), torch.from_numpy(bad_qs).to(dev),
                  case.scale)
    torch.cuda.synchronize()
    assert np.all(bits(out3)[65:70] == 0)


@pytest.mark.parametrize("sign", [-1.0, 0.0])
def test_prefill_negative_and_zero_scale(sign):
    """A negative scale flips every score (the kernel carries the sign on
    Q); scale 0 gives the plain mean of the visible values."""
    dev = device()
    case = workloads.random_case(51, [300, 64, 129], 4, 2, 128, 16)
    kc, vc, tables, lens = _oracle_cache(case)
    q, qs = _queries(51, [300, 20, 129], 4, 128)
    scale = sign * case.scale
    out = _gpu_prefill(dev, q, kc, vc, tables, lens, qs, scale)
    ref = oracle.prefill(q, kc, vc, tables, lens, qs, scale)
    assert_attention_close(out, ref, f"scale {scale}")


def test_prefill_skips_table_entries_outside_the_pool():
    """A block id outside the pool drops its tokens from every row that
    would see them, also inside tiles that lie wholly before a row."""
    dev = device()
    n = 200
    case = workloads.random_case(61, [n], 2, 2, 128, 16)
    kc, vc, tables, lens = _oracle_cache(case)
    bad = tables.copy()
    bad[0, 2] = case.num_blocks + 3                  # tokens 32..47 drop out
    q, qs = _queries(61, [n], 2, 128)
    out = _gpu_prefill(dev, q, kc, vc, bad, lens, qs, case.scale)
    kept = np.array([p for p in range(n) if not 32 <= p < 48])
    k = np.ascontiguousarray(case.k_tokens[kept])
    v = np.ascontiguousarray(case.v_tokens[kept])
    seen = np.array([int(np.sum(kept <= i)) for i in range(n)], np.int32)   # row i sits at position i
    ref = oracle.attention_contig(q, k, v, np.zeros(n, np.int64), seen, case.scale)
    assert_attention_close(out, ref, "skipped ids")


def test_prefill_rising_scores_move_the_running_maximum():
    """K rows grow along the context (x0.2 .. x20), so each row's maximum
    climbs by many octaves over its tiles: the lazily moved running
    maximum and the rescale of O are exercised over and over."""
    dev = device()
    n = 700
    case = workloads.random_case(71, [n], 4, 2, 128, 16)
    grow = (0.2 + 19.8 * np.arange(n) / n).astype(np.float32)
    case.k_tokens[:] = (case.k_tokens.astype(np.float32) * grow[:, None, None]).astype(np.float16)
    kc, vc, tables, lens = _oracle_cache(case)
    q, qs = _queries(71, [n], 4, 128)
    out = _gpu_prefill(dev, q, kc, vc, tables, lens, qs, case.scale)
    ref = oracle.prefill(q, kc, vc, tables, lens, qs, case.scale)
    assert_attention_close(out, ref, "rising scores")


SHORT_CHUNKS = (8, 40, 1)      # one row tile per (KV head, sequence) at most
LONG_CHUNKS = (300, 260, 1)    # several row tiles, each walking the split context


@pytest.mark.parametrize("H,Hkv,D,ms", [(8, 2, 128, SHORT_CHUNKS), (4, 4, 128, SHORT_CHUNKS),
                                        (16, 8, 128, SHORT_CHUNKS), (8, 2, 64, SHORT_CHUNKS),
                                        (8, 2, 256, SHORT_CHUNKS), (4, 4, 128, LONG_CHUNKS),
                                        (8, 2, 128, LONG_CHUNKS), (4, 4, 64, LONG_CHUNKS),
                                        (8, 2, 256, LONG_CHUNKS)])
def test_prefill_split_context(H, Hkv, D, ms):
    """Chunks over long contexts with few sequences: the context is split
    into parts merged by a second kernel.  Against the oracle, against the
    unsplit kernel (same math, other summation order), bit for bit when
    repeated, and through one workspace reused by a smaller call."""
    dev = device()
    lens_l = [3000, 2500, 1777]
    ms = list(ms)
    case = workloads.random_case(91 + H + D, lens_l, H, Hkv, D, 16)
    kc, vc, tables, lens = _oracle_cache(case)
    q, qs = _queries(91, ms, H, D)
    T, W = int(qs[-1]), tables.shape[1]
    need = pa.pa_prefill_workspace_size(T, 3, H, Hkv, D, 16, W, max(ms))
    say(f"prefill split H={H}/{Hkv} D={D} ms={ms}: workspace {need} bytes")
    assert need > 0                                                  # this batch splits
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    split = _gpu_prefill(dev, q, kc, vc, tables, lens, qs, case.scale, workspace=ws)
    ref = oracle.prefill(q, kc, vc, tables, lens, qs, case.scale)
    assert_attention_close(split, ref, f"split H={H}/{Hkv} D={D}")
    whole = _gpu_prefill(dev, q, kc, vc, tables, lens, qs, case.scale, split=False)
    assert_attention_close(whole, ref, f"unsplit H={H}/{Hkv} D={D}")
    again = _gpu_prefill(dev, q, kc, vc, tables, lens, qs, case.scale, workspace=ws)
    assert np.array_equal(bits(split), bits(again))
    # the same workspace for a smaller batch (first two sequences)
    m01 = ms[0] + ms[1]
    q2, qs2 = np.ascontiguousarray(q[:m01]), np.array([0, ms[0], m01], np.int32)
    t2, l2 = np.ascontiguousarray(tables[:2]), np.ascontiguousarray(lens[:2])
    small = _gpu_prefill(dev, q2, kc, vc, t2, l2, qs2, case.scale, workspace=ws)
    assert_attention_close(small, oracle.prefill(q2, kc, vc, t2, l2, qs2, case.scale), "split, smaller batch")


def test_prefill_split_with_bad_and_empty_sequences():
    """Split context with a sequence whose new tokens exceed its context
    (NaN rows), an empty one, and one skipped for a range outside [0, T)."""
    dev = device()
    case = workloads.random_case(95, [2000, 10, 1500, 1800], 4, 2, 128, 16)
    kc, vc, tables, lens = _oracle_cache(case)
    ms = [16, 0, 5, 7]
    q, qs = _queries(95, ms, 4, 128)
    lens_bad = lens.copy()
    lens_bad[2] = 3                                                  # 5 new tokens > 3 cached
    out = _gpu_prefill(dev, q, kc, vc, tables, lens_bad, qs, case.scale)
    assert pa.pa_prefill_workspace_size(int(qs[-1]), 4, 4, 2, 128, 16, tables.shape[1], 16) > 0
    o = out.float().cpu().numpy()
    assert np.all(np.isnan(o[16:21]))
    sel = np.r_[0:16, 21:28]
    ref = oracle.prefill(np.ascontiguousarray(q[sel]), kc, vc, np.ascontiguousarray(tables[[0, 3]]),
                         np.ascontiguousarray(lens[[0, 3]]), np.array([0, 16, 23], np.int32), case.scale)
    assert_attention_close(out[sel], ref, "split, other sequences")


def test_prefill_is_deterministic_and_blind_to_placement():
    dev = device()
    case = workloads.random_case(41, [300, 64, 129], 8, 2, 128, 16, spare_blocks=30)
    kc, vc, tables, lens = _oracle_cache(case)
    q, qs = _queries(41, [300, 20, 100], 8, 128)
    a = _gpu_prefill(dev, q, kc, vc, tables, lens, qs, case.scale)
    b = _gpu_prefill(dev, q, kc, vc, tables, lens, qs, case.scale)
    assert np.array_equal(bits(a), bits(b))
    sigma = np.random.default_rng(2).permutation(case.num_blocks)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[sigma], vc2[sigma] = kc, vc
    t2 = np.where(tables >= 0, sigma[np.maximum(tables, 0)], -1).astype(np.int32)
    c = _gpu_prefill(dev, q, kc2, vc2, t2, lens, qs, case.scale)
    assert np.array_equal(bits(a), bits(c))


def test_prompt_prefill_at_the_llama_shape():
    """8 prompts of the block-size-sweep length mix (normal around 500
    tokens) at 32 x 128 heads, B = 16: the product block manager admits
    them, the product scatter writes their K/V, pa_prefill attends; every
    row against the oracle; then pa_prefill_append on a NaN cache writes the
    same caches and the same outputs bit for bit."""
    dev = device()
    rng = np.random.default_rng(12)
    lens_l = [int(x) for x in np.clip(np.rint(rng.normal(500, 150, size=8)), 16, 2048)]
    H = Hkv = 32
    D, B = 128, 16
    NB = sum(-(-n // B) for n in lens_l) + 8
    bm = pa.BlockManager(NB, B)
    slots = np.concatenate([bm.add_sequence(s, n) for s, n in enumerate(lens_l)])
    T = int(sum(lens_l))
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    key = torch.randn((T, Hkv, D), generator=g, device=dev, dtype=torch.float16)
    val = torch.randn((T, Hkv, D), generator=g, device=dev, dtype=torch.float16)
    q = torch.randn((T, H, D), generator=g, device=dev, dtype=torch.float16)
    kc = torch.full((NB, Hkv, B, D), float("nan"), dtype=torch.float16, device=dev)
    vc = torch.full_like(kc, float("nan"))
    pa.pa_reshape_and_cache(key, val, torch.from_numpy(slots).to(dev), kc, vc)
    width = -(-max(lens_l) // B)
    tables, lens = bm.get_tables(range(8), width)
    qs = np.concatenate([[0], np.cumsum(lens_l)]).astype(np.int32)
    out = torch.empty_like(q)
    pa.pa_prefill(out, q, kc, vc, torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev),
                  torch.from_numpy(qs).to(dev), 1 / np.sqrt(D), max_query_len=max(lens_l))
    torch.cuda.synchronize()
    say(f"llama prompts: {lens_l}, T={T}")
    ref = oracle.prefill(q.cpu().numpy(), kc.cpu().numpy(), vc.cpu().numpy(), tables, lens, qs, 1 / np.sqrt(D))
    assert_attention_close(out, ref, "llama prompts")
    # the same prompts through pa_prefill_append on a cache holding only NaN:
    # the caches it writes equal the scatter's bit for bit, and so do the outputs
    # (both calls read the same K/V values, in the same order)
    kc2 = torch.full_like(kc, float("nan"))
    vc2 = torch.full_like(kc, float("nan"))
    out2 = torch.empty_like(q)
    pa.pa_prefill_append(out2, q, key, val, kc2, vc2, torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev),
                         torch.from_numpy(qs).to(dev), 1 / np.sqrt(D), max_query_len=max(lens_l))
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc2), bits(kc)) and np.array_equal(bits(vc2), bits(vc)), "append: caches differ"
    assert np.array_equal(bits(out2), bits(out)), "append: outputs differ from pa_prefill's"


def _append_case(case, ms):
    """The cache before a pa_prefill_append call (positions < n - m written by
    the oracle's scatter, NaN everywhere else, the new tokens' slots
    included), the cache the oracle's scatter of every position gives, and
    the new tokens' K/V packed in query order [T, Hkv, D]."""
    m_model = BlockManagerModel(case.num_blocks, case.block_size)
    for s, (n, t) in enumerate(zip(case.lens, case.tables)):
        m_model.set_table(s, t, n)
    starts = np.concatenate([[0], np.cumsum(case.lens)]).astype(np.int64)
    old = [(s, p) for s, n in enumerate(case.lens) for p in range(n - ms[s])]
    new = [(s, p) for s, n in enumerate(case.lens) for p in range(n - ms[s], n)]
    kc0, vc0, tables, lens = _oracle_cache(case)
    kc0[...] = np.float16(np.nan)
    vc0[...] = np.float16(np.nan)
    kc1, vc1 = kc0.copy(), vc0.copy()
    rows_old = np.array([starts[s] + p for s, p in old], np.int64)
    rows_new = np.array([starts[s] + p for s, p in new], np.int64)
    if len(old):
        oracle.reshape_and_cache(np.ascontiguousarray(case.k_tokens[rows_old]),
                                 np.ascontiguousarray(case.v_tokens[rows_old]),
                                 np.array([m_model.slot(s, p) for s, p in old], np.int64), kc0, vc0)
    kc1[...], vc1[...] = kc0, vc0
    key = np.ascontiguousarray(case.k_tokens[rows_new])
    value = np.ascontiguousarray(case.v_tokens[rows_new])
    if len(new):
        oracle.reshape_and_cache(key, value, np.array([m_model.slot(s, p) for s, p in new], np.int64), kc1, vc1)
    return kc0, vc0, kc1, vc1, key, value, tables, lens


def _gpu_prefill_append(dev, q, key, value, kc0, vc0, tables, lens, qs, scale, pad=0, split=True):
    T, Hkv, D = key.shape
    if pad:
        # key and value as views into wider rows (a fused QKV-like buffer)
        wide = torch.zeros((T, 2, Hkv * D + pad), dtype=torch.float16, device=dev)
        wide[:, 0, :Hkv * D] = torch.from_numpy(key).to(dev).reshape(T, Hkv * D)
        wide[:, 1, :Hkv * D] = torch.from_numpy(value).to(dev).reshape(T, Hkv * D)
        k_t = wide[:, 0].narrow(1, 0, Hkv * D).unflatten(1, (Hkv, D))
        v_t = wide[:, 1].narrow(1, 0, Hkv * D).unflatten(1, (Hkv, D))
    else:
        k_t, v_t = torch.from_numpy(key).to(dev), torch.from_numpy(value).to(dev)
    kc, vc = torch.from_numpy(kc0).to(dev), torch.from_numpy(vc0).to(dev)
    out = torch.full(q.shape, float("nan"), dtype=torch.float16, device=dev)
    pa.pa_prefill_append(out, torch.from_numpy(q).to(dev), k_t, v_t, kc, vc, torch.from_numpy(tables).to(dev),
                         torch.from_numpy(lens).to(dev), torch.from_numpy(qs).to(dev), scale, split=split)
    torch.cuda.synchronize()
    return out, kc, vc


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("B", [1, 4, 16, 128])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (6, 3), (4, 4), (8, 4)])
@pytest.mark.parametrize("chunk", ["full", "chunked", "decode"])
def test_prefill_append_matches_oracle(D, B, H, Hkv, chunk):
    """pa_prefill_append against the oracle's scatter of the new tokens
    followed by its prefill: the caches bit for bit (every new token written
    once, by the workgroup holding its first query row -- with 3 query heads
    per KV head a token's rows can straddle two row tiles), the output within
    tolerance.  The new tokens' slots hold NaN before the call, so any read of
    them from the cache would show."""
    dev = device()
    case = workloads.random_case(700 + B + 10 * H + Hkv + D, LENS, H, Hkv, D, B)
    if chunk == "full":
        ms = list(LENS)
    elif chunk == "chunked":
        ms = [max(1, n // 3) for n in LENS]
    else:
        ms = [1] * len(LENS)
    kc0, vc0, kc1, vc1, key, value, tables, lens = _append_case(case, ms)
    q, qs = _queries(B + H + 5, ms, H, D)
    say(f"prefill_append D={D} B={B} H={H}/{Hkv} {chunk}: rows {int(qs[-1])}")
    out, kc, vc = _gpu_prefill_append(dev, q, key, value, kc0, vc0, tables, lens, qs, case.scale,
                                      pad=24 if B == 16 else 0)
    assert np.array_equal(bits(kc), kc1.view(np.uint16)), "K cache differs from the oracle's scatter"
    assert np.array_equal(bits(vc), vc1.view(np.uint16)), "V cache differs from the oracle's scatter"
    ref = oracle.prefill(q, kc1, vc1, tables, lens, qs, case.scale)
    assert_attention_close(out, ref, f"prefill_append D={D} B={B} H={H}/{Hkv} {chunk}")
    # the same rows through the two-call path on the written cache
    two = _gpu_prefill(dev, q, kc1, vc1, tables, lens, qs, case.scale)
    assert_attention_close(two, ref, "two calls")


@pytest.mark.parametrize("H,Hkv,ms", [(8, 2, SHORT_CHUNKS), (16, 8, SHORT_CHUNKS), (4, 4, LONG_CHUNKS),
                                      (6, 3, LONG_CHUNKS)])
def test_prefill_append_split_context(H, Hkv, ms):
    """Chunks over long contexts, context split into parts: each new token
    is written by the part whose tiles hold it; with and without a
    workspace."""
    dev = device()
    lens_l = [3000, 2500, 1777]
    ms = list(ms)
    case = workloads.random_case(191 + H, lens_l, H, Hkv, 128, 16)
    kc0, vc0, kc1, vc1, key, value, tables, lens = _append_case(case, ms)
    q, qs = _queries(191, ms, H, 128)
    ref = oracle.prefill(q, kc1, vc1, tables, lens, qs, case.scale)
    for split in (True, False):
        out, kc, vc = _gpu_prefill_append(dev, q, key, value, kc0, vc0, tables, lens, qs, case.scale, split=split)
        assert np.array_equal(bits(kc), kc1.view(np.uint16)) and np.array_equal(bits(vc), vc1.view(np.uint16))
        assert_attention_close(out, ref, f"append split={split} H={H}/{Hkv}")


def test_prefill_append_skips_ids_outside_the_pool():
    """A new token whose table entry lies outside the pool is neither written
    nor attended to (as for a cached token behind such an entry); the other
    tokens are written and the rest of the batch is unaffected."""
    dev = device()
    case = workloads.random_case(77, [40, 33], 4, 2, 128, 16)
    ms = [40, 20]
    kc0, vc0, kc1, vc1, key, value, tables, lens = _append_case(case, ms)
    bad = tables.copy()
    bad[1, 2] = case.num_blocks + 5                          # block of position 32, sequence 1's last new token
    q, qs = _queries(77, ms, 4, 128)
    out, kc, vc = _gpu_prefill_append(dev, q, key, value, kc0, vc0, bad, lens, qs, case.scale)
    # expected cache: the oracle's, with the block of the bad entry left as before the call
    blk = tables[1, 2]
    kc_exp, vc_exp = kc1.copy(), vc1.copy()
    kc_exp[blk], vc_exp[blk] = kc0[blk], vc0[blk]
    assert np.array_equal(bits(kc), kc_exp.view(np.uint16)) and np.array_equal(bits(vc), vc_exp.view(np.uint16))
    # sequence 0 is untouched by the bad entry; sequence 1's rows match pa_prefill over the written cache with the
    # same bad table (the pool-id mask is the same in both calls)
    ref0 = oracle.prefill(np.ascontiguousarray(q[:40]), kc1, vc1, np.ascontiguousarray(tables[:1]),
                          np.ascontiguousarray(lens[:1]), np.array([0, 40], np.int32), case.scale)
    assert_attention_close(out[:40], ref0, "sequence 0")
    two = _gpu_prefill(dev, q, kc_exp, vc_exp, bad, lens, qs, case.scale)
    assert_attention_close(out[40:], two[40:].float().cpu().numpy(), "sequence 1 against pa_prefill")
