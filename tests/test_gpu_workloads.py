"""Full-size workloads through the product path against the oracle: the
block-size sweep (one set of token values laid out at B = 8/16/32/64) and
parallel sampling with copy-on-write over a shared 1000-token prompt.

Both are compared in full: every sequence's slots, table and output, every
cache byte, and -- for parallel sampling -- every one of the 256 steps."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_390_amd as pa
import workloads
from gpu_common import assert_attention_close, bits, device, poisoned_cache, say
from oracle.block_manager import BlockManagerModel

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
def test_block_size_sweep():
    """The 5688vip.com page's block-size experiment (section 案例: 256
    concurrent sequences, prompts of mean 500 tokens, up to 1024 generated):
    at every block size, all 256 sequences' slots and tables equal the
    block-manager model's, the product's scatter writes exactly the bytes
    the oracle's scatter writes (unused tail rows stay NaN), and every
    output row is within tolerance of the oracle, whose own paged result is
    bit for bit its attention over the contiguous tokens at every B."""
    dev = device()
    w = workloads.block_size_sweep(seed=0)
    S = len(w.lens)
    Hkv, D = w.num_kv_heads, w.head_dim
    k, v = w.tokens(dev)
    q = w.query(dev)
    k_h, v_h, q_h = k.cpu().numpy(), v.cpu().numpy(), q.cpu().numpy()
    lens_all = w.lens.astype(np.int32)
    say(f"sweep: S={S} tokens={int(w.lens.sum())} max n={int(w.lens.max())}")
    # the reference every block size is held to: attention over the contiguous tokens
    ref = oracle.attention_contig(q_h, k_h, v_h, w.seq_start.astype(np.int64), lens_all, w.scale)
    for B in (8, 16, 32, 64):
        tables = w.perm_tables(B)
        NB = sum(len(t) for t in tables)
        bm = pa.BlockManager(NB, B)
        m = BlockManagerModel(NB, B)
        for s in range(S):
            bm.set_table(s, tables[s], int(w.lens[s]))
            m.set_table(s, tables[s].tolist(), int(w.lens[s]))
        slots = np.concatenate([bm.get_slots(s, 0, int(w.lens[s])) for s in range(S)])
        want_slots = np.array([m.slot(s, p) for s in range(S) for p in range(int(w.lens[s]))], dtype=np.int64)
        assert np.array_equal(slots, want_slots), f"B={B}: slots differ from the model's"
        width = max(len(t) for t in tables)
        tab, lens = bm.get_tables(range(S), width)
        rows, lens_m = m.tables(range(S), width)
        tab_m = np.array(rows, dtype=np.int32)
        assert np.array_equal(tab, tab_m) and lens.tolist() == lens_m, f"B={B}: tables differ from the model's"

        kc = torch.full((NB, Hkv, B, D), float("nan"), dtype=torch.float16, device=dev)
        vc = torch.full_like(kc, float("nan"))
        pa.pa_reshape_and_cache(k, v, torch.from_numpy(slots).to(dev), kc, vc)
        out = torch.empty_like(q)
        pa.pa_decode(out, q, kc, vc, torch.from_numpy(tab).to(dev), torch.from_numpy(lens).to(dev), w.scale, B)
        torch.cuda.synchronize()

        # the oracle's scatter of the same tokens through the model's slots
        kc_h = poisoned_cache(NB, Hkv, B, D)
        vc_h = kc_h.copy()
        oracle.reshape_and_cache(k_h, v_h, want_slots, kc_h, vc_h)
        assert np.array_equal(bits(kc), kc_h.view(np.uint16)), f"B={B}: K cache bytes differ"
        assert np.array_equal(bits(vc), vc_h.view(np.uint16)), f"B={B}: V cache bytes differ"
        del kc, vc
        ref_b = oracle.decode(q_h, kc_h, vc_h, tab_m, np.array(lens_m, dtype=np.int32), w.scale)
        assert np.array_equal(ref_b, ref), f"B={B}: the oracle's paged result is not its contiguous one"
        waste = sum(len(t) * B - int(n) for t, n in zip(tables, w.lens)) * Hkv * D * 2 * 2
        say(f"  B={B}: NB={NB} tail-waste {waste / 1e6:.1f} MB")
        assert_attention_close(out, ref_b, f"sweep B={B} (all {S} rows)")
        del kc_h, vc_h
        torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fused", [False, True])
def test_parallel_sampling_copy_on_write(fused):
    """lpnh.cn/news/2758356 section 4.2: one 1000-token prompt forked into 32
    samples; the first append copies the shared, partly filled tail block
    for samples 0..30, and every later step appends into the samples' own
    blocks, taking a fresh block whenever the last one is full (positions
    1008, 1024, ...).  At every one of the 256 steps: slots, COW pairs,
    tables, the free list and every cache byte equal the model's and the
    oracle's; every sample's output is within tolerance of the oracle.

    fused: each step's write goes through pa_decode_append (after the
    step's copy-on-write copies) instead of pa_reshape_and_cache +
    pa_decode."""
    dev = device()
    w = workloads.parallel_sampling(seed=0)
    NB, B, N = w.num_blocks, w.block_size, w.num_samples
    Hkv, D = w.num_kv_heads, w.head_dim
    bm = pa.BlockManager(NB, B)
    m = BlockManagerModel(NB, B)
    kp, vp = w.prompt_tokens(dev)
    slots = bm.add_sequence(0, w.prompt_len)
    assert slots.tolist() == m.add_sequence(0, w.prompt_len)
    kc_h = poisoned_cache(NB, Hkv, B, D)
    vc_h = kc_h.copy()
    kc, vc = torch.from_numpy(kc_h).to(dev), torch.from_numpy(vc_h).to(dev)
    pa.pa_reshape_and_cache(kp, vp, torch.from_numpy(slots).to(dev), kc, vc)
    oracle.reshape_and_cache(kp.cpu().numpy(), vp.cpu().numpy(), slots, kc_h, vc_h)
    for c in range(1, N):
        bm.fork(0, c)
        m.fork(0, c)
    tail = m.table(0)[-1]
    assert bm.refcount(tail) == N
    seqs = list(range(N))
    width = workloads.ceil_div(w.prompt_len + w.steps, B)
    grew = 0
    for step in range(w.steps):
        q, key, val = w.step_tokens(step, dev)
        blocks_before = len(m.table(0))
        slots, pairs = bm.append_tokens(seqs)
        want = [m.append_token(s) for s in seqs]
        assert slots.tolist() == [x[0] for x in want]
        assert [tuple(p) for p in pairs.tolist()] == [x[1] for x in want if x[1]]
        if step == 0:
            assert len(pairs) == N - 1 and all(p[0] == tail for p in pairs.tolist())
        else:
            assert len(pairs) == 0
        grew += len(m.table(0)) > blocks_before
        if len(pairs):
            pa.pa_copy_blocks([kc], [vc], torch.from_numpy(pairs).to(dev))
            oracle.copy_blocks([kc_h], [vc_h], np.ascontiguousarray(pairs))
        if not fused:
            pa.pa_reshape_and_cache(key, val, torch.from_numpy(slots).to(dev), kc, vc)
        oracle.reshape_and_cache(key.cpu().numpy(), val.cpu().numpy(), slots, kc_h, vc_h)
        tables, lens = bm.get_tables(seqs, width)
        rows, lens_m = m.tables(seqs, width)
        assert np.array_equal(tables, np.array(rows, np.int32)) and lens.tolist() == lens_m
        assert bm.free_list() == m.free
        out = torch.empty_like(q)
        if fused:
            pa.pa_decode_append(out, q, key, val, kc, vc, torch.from_numpy(tables).to(dev),
                                torch.from_numpy(lens).to(dev), w.scale, B)
        else:
            pa.pa_decode(out, q, kc, vc, torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev), w.scale, B)
        torch.cuda.synchronize()
        assert np.array_equal(bits(kc), kc_h.view(np.uint16)), f"step {step}: K cache bytes differ"
        assert np.array_equal(bits(vc), vc_h.view(np.uint16)), f"step {step}: V cache bytes differ"
        ref = oracle.decode(q.cpu().numpy(), kc_h, vc_h, np.array(rows, np.int32), np.array(lens_m, np.int32),
                            w.scale)
        quiet = step % 32 != 31 and step != 0
        if quiet:
            g = out.float().cpu().numpy().astype(np.float64)
            assert not np.any(np.isnan(g)), f"cow step {step}: NaN output"
            assert np.all(np.abs(g - ref) <= 2e-3 + 1e-2 * np.abs(ref)), f"cow step {step}: outside tolerance"
        else:
            say(f"  cow step {step} fused={fused}: len {lens[0]}, blocks {len(m.table(0))}, "
                f"free {bm.num_free()}")
            assert_attention_close(out, ref, f"cow step {step}")
    # positions 1008, 1024, ..., 1248 each opened a new block
    assert grew == len(range(1008, w.prompt_len + w.steps, B))
    for b in range(NB):
        assert bm.refcount(b) == m.refcount[b]
    assert all(bm.seq_len(s) == w.prompt_len + w.steps for s in seqs)
    assert all(len(bm.table(s)) == 79 for s in seqs)
    for s in seqs:
        bm.free_sequence(s)
        m.free_sequence(s)
    assert bm.num_free() == NB and bm.free_list() == m.free
