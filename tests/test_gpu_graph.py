"""A decode step (and a prefill with its K/V write) captured in a HIP graph
(torch.cuda.graph over the C ABI's calls on the capture stream) replays the
same results as eager launches:
the calls allocate nothing, synchronise with nothing and record no memset.

Each replay starts from the cache as it was before the step (history only,
NaN in the slots the step writes), restored by eager work between replays,
and must reproduce the eager outputs and cache writes bit for bit (the
kernels are deterministic; the dispatch order changes no bit)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_390_amd as pa
import workloads
from gpu_common import assert_attention_close, bits, device, poisoned_cache, say
from oracle.block_manager import BlockManagerModel

pytestmark = pytest.mark.gpu

LENS = [1, 16, 17, 129, 300, 511, 512, 777, 1024, 1031]


def _history_cache(case):
    """Cache with every token but each sequence's last (oracle scatter, NaN
    elsewhere); tables, lengths, the last tokens' K/V, and the full cache."""
    m = BlockManagerModel(case.num_blocks, case.block_size)
    for s, (n, t) in enumerate(zip(case.lens, case.tables)):
        m.set_table(s, t, n)
    rows, lens = m.tables(range(len(case.lens)), max(len(t) for t in case.tables))
    hist = [int(case.seq_start[s]) + p for s, n in enumerate(case.lens) for p in range(n - 1)]
    hist_slots = np.array([m.slot(s, p) for s, n in enumerate(case.lens) for p in range(n - 1)], np.int64)
    last = [int(case.seq_start[s]) + n - 1 for s, n in enumerate(case.lens)]
    last_slots = np.array([m.slot(s, n - 1) for s, n in enumerate(case.lens)], np.int64)
    kc = poisoned_cache(case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim)
    vc = kc.copy()
    oracle.reshape_and_cache(case.k_tokens[hist], case.v_tokens[hist], hist_slots, kc, vc)
    kc_full, vc_full = kc.copy(), vc.copy()
    nk, nv = np.ascontiguousarray(case.k_tokens[last]), np.ascontiguousarray(case.v_tokens[last])
    oracle.reshape_and_cache(nk, nv, last_slots, kc_full, vc_full)
    return kc, vc, kc_full, vc_full, np.array(rows, np.int32), np.array(lens, np.int32), nk, nv


@pytest.mark.parametrize("H,Hkv,P", [(8, 8, 0), (16, 2, 0), (8, 8, 128), (16, 2, 256)])
def test_decode_step_replays_in_a_hip_graph(H, Hkv, P):
    dev = device()
    L, B, D = 3, 16, 128
    case = workloads.random_case(500 + H + P, LENS, H, Hkv, D, B)
    kc_h, vc_h, kc_full, vc_full, tables, lens, nk, nv = _history_cache(case)
    S = len(LENS)
    maxlen = tables.shape[1] * B
    say(f"graph H={H}/{Hkv} P={P} layers={L}")
    kc0, vc0 = torch.from_numpy(kc_h).to(dev), torch.from_numpy(vc_h).to(dev)
    kcs = [kc0.clone() for _ in range(L)]
    vcs = [vc0.clone() for _ in range(L)]
    q = torch.from_numpy(case.q).to(dev)
    key, val = torch.from_numpy(nk).to(dev), torch.from_numpy(nv).to(dev)
    d_t, d_l = torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev)
    order = torch.empty(S, dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, pa.pa_decode_workspace_size(S, H, Hkv, D, B, maxlen, P)), dtype=torch.uint8,
                     device=dev)
    outs = [torch.empty((S, H, D), dtype=torch.float16, device=dev) for _ in range(L)]

    def step():
        pa.pa_decode_order(d_l, maxlen, out=order)
        for l in range(L):
            pa.pa_decode_append(outs[l], q, key, val, kcs[l], vcs[l], d_t, d_l, case.scale, B,
                                max_context_len=maxlen, partition_size=P, workspace=ws, seq_order=order)

    def reset():
        for l in range(L):
            kcs[l].copy_(kc0)
            vcs[l].copy_(vc0)
            outs[l].fill_(float("nan"))

    step()                                                   # eager
    torch.cuda.synchronize()
    eager_out = [bits(o).copy() for o in outs]
    ref = oracle.decode(case.q, kc_full, vc_full, tables, lens, case.scale)
    for l in range(L):
        assert np.array_equal(bits(kcs[l]), kc_full.view(np.uint16))
        assert np.array_equal(bits(vcs[l]), vc_full.view(np.uint16))
        assert_attention_close(outs[l], ref, f"eager layer {l}")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        reset()
        step()                                               # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        reset()                                              # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(L):
            assert np.array_equal(bits(outs[l]), eager_out[l]), f"replay {rep} layer {l}: output differs"
            assert np.array_equal(bits(kcs[l]), kc_full.view(np.uint16)), f"replay {rep} layer {l}: K cache"
            assert np.array_equal(bits(vcs[l]), vc_full.view(np.uint16)), f"replay {rep} layer {l}: V cache"


@pytest.mark.parametrize("split", [False, True])
def test_prefill_append_replays_in_a_hip_graph(split):
    """Chunks of new tokens over cached contexts (pa_prefill_append: the
    chunks' K/V written and attended in one call), captured and replayed with
    eager work between replays; with a caller workspace the context is split
    and the merge kernel is captured too.  Every replay reproduces the eager
    output and cache writes bit for bit."""
    from test_gpu_prefill import _append_case, _queries
    dev = device()
    lens_l = [3000, 2500, 1777] if split else [40, 300, 129, 777]
    ms = [8, 40, 1] if split else [40, 100, 17, 300]
    H, Hkv, D, B = 8, 2, 128, 16
    case = workloads.random_case(620 + len(lens_l), lens_l, H, Hkv, D, B)
    kc_h, vc_h, kc_full, vc_full, key_h, val_h, tables, lens = _append_case(case, ms)
    q_h, qs = _queries(620, ms, H, D)
    T = int(qs[-1])
    say(f"graph prefill_append split={split} rows={T}")
    kc0, vc0 = torch.from_numpy(kc_h).to(dev), torch.from_numpy(vc_h).to(dev)
    kc, vc = kc0.clone(), vc0.clone()
    q, key, val = (torch.from_numpy(x).to(dev) for x in (q_h, key_h, val_h))
    d_t, d_l, d_q = (torch.from_numpy(x).to(dev) for x in (tables, lens, qs))
    need = pa.pa_prefill_workspace_size(T, len(lens_l), H, Hkv, D, B, tables.shape[1], max(ms))
    assert need > 0 or not split                               # the split batch needs a workspace
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H, D), dtype=torch.float16, device=dev)

    def call():
        pa.pa_prefill_append(out, q, key, val, kc, vc, d_t, d_l, d_q, case.scale, max_query_len=max(ms),
                             workspace=ws if split else None, split=split)

    def reset():
        kc.copy_(kc0)
        vc.copy_(vc0)
        out.fill_(float("nan"))

    call()                                                   # eager
    torch.cuda.synchronize()
    eager_out = bits(out).copy()
    assert np.array_equal(bits(kc), kc_full.view(np.uint16)) and np.array_equal(bits(vc), vc_full.view(np.uint16))
    ref = oracle.prefill(q_h, kc_full, vc_full, tables, lens, qs, case.scale)
    assert_attention_close(out, ref, "eager")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        reset()
        call()                                               # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        reset()                                              # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), eager_out), f"replay {rep}: output differs"
        assert np.array_equal(bits(kc), kc_full.view(np.uint16)), f"replay {rep}: K cache"
        assert np.array_equal(bits(vc), vc_full.view(np.uint16)), f"replay {rep}: V cache"
