"""GPU checks of the persistent prefill grid.

When a pa_prefill / pa_prefill_append call has more row-tile workgroups than
the GPU holds at once, one query head per KV head, at least 1024 query rows
per (KV head, sequence) and a workspace for the claim counters, one round of
resident workgroups takes the items from per-XCD counters (one counter when
the (KV head, sequence) pairs are not a multiple of 8).  Each item runs the
same code as with one workgroup per item, so outputs and cache writes are
compared bit for bit with a call given no workspace (one workgroup per item),
and a subset of sequences against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_390_amd as pa
import workloads
from gpu_common import assert_attention_close, bits, device, say
from test_gpu_decode import _oracle_cache
from test_gpu_prefill import _append_case, _queries

pytestmark = pytest.mark.gpu

MIX = [700, 333, 1024, 90, 512, 640, 257, 800]

# name: (full prompt lengths, H, Hkv, D, B, rows per workgroup, sequences checked against the oracle)
CASES = {
    "d128 pairs x8": (MIX * 2, 8, 8, 128, 16, 128, [3, 6]),
    "d64 pairs x8": (MIX * 2, 8, 8, 64, 16, 128, [0, 3]),
    "d256 pairs x8": (MIX * 2, 8, 8, 256, 16, 64, [1, 3]),
    "d128 16 heads": (MIX * 2, 16, 16, 128, 16, 128, [3, 6]),
    "d128 pairs not x8": ([3600, 1500, 200, 2900, 64, 2048, 1000], 4, 4, 128, 32, 128, [4, 6]),
}


def _row_tiles(lens, H, Hkv, rows_per_wg):
    return -(-max(lens) * (H // Hkv) // rows_per_wg)


def _items(lens, H, Hkv, rows_per_wg):
    return Hkv * len(lens) * _row_tiles(lens, H, Hkv, rows_per_wg)


def _setup(name):
    lens_l, H, Hkv, D, B, rpw, check = CASES[name]
    dev = device()
    case = workloads.random_case(1300 + len(name), lens_l, H, Hkv, D, B)
    kc, vc, tables, lens = _oracle_cache(case)
    q, qs = _queries(1300 + D, lens_l, H, D)
    items = _items(lens_l, H, Hkv, rpw)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    # more items than any occupancy (at most 3 workgroups per CU) holds at once
    assert items > 3 * cus, (items, cus)
    assert H == Hkv and _row_tiles(lens_l, H, Hkv, rpw) * rpw >= 1024    # one query head per KV head, rows per pair
    need = pa.pa_prefill_workspace_size(int(qs[-1]), len(lens_l), H, Hkv, D, B, tables.shape[1], max(lens_l))
    assert need == 256, need                                  # unsplit: the claim counters only
    return dev, case, kc, vc, tables, lens, q, qs, check


def _run(dev, q, kc, vc, tables, lens, qs, scale, workspace=None, split=True):
    out = torch.full(q.shape, float("nan"), dtype=torch.float16, device=dev)
    pa.pa_prefill(out, q, kc, vc, tables, lens, qs, scale, max_query_len=int((qs[1:] - qs[:-1]).max().item()),
                  workspace=workspace, split=split)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_persistent_grid_matches_one_workgroup_per_item(name):
    dev, case, kc_h, vc_h, tables_h, lens_h, q_h, qs_h, check = _setup(name)
    # one sequence whose context is shorter than its new tokens: its rows come out NaN either way
    bad = 5
    lens_h = lens_h.copy()
    lens_h[bad] = int(qs_h[bad + 1] - qs_h[bad]) - 1
    kc, vc, q = (torch.from_numpy(x).to(dev) for x in (kc_h, vc_h, q_h))
    t, l, qs = (torch.from_numpy(x).to(dev) for x in (tables_h, lens_h, qs_h))
    say(f"persistent prefill {name}: rows {int(qs_h[-1])}")
    p = _run(dev, q, kc, vc, t, l, qs, case.scale)                     # workspace allocated: persistent
    o = _run(dev, q, kc, vc, t, l, qs, case.scale, split=False)        # no workspace: one workgroup per item
    assert np.array_equal(bits(p), bits(o)), "persistent grid differs from one workgroup per item"
    assert torch.isnan(p[int(qs_h[bad]):int(qs_h[bad + 1])]).all()
    for s in check:
        a, b = int(qs_h[s]), int(qs_h[s + 1])
        ref = oracle.prefill(np.ascontiguousarray(q_h[a:b]), kc_h, vc_h, np.ascontiguousarray(tables_h[[s]]),
                             np.ascontiguousarray(lens_h[[s]]), np.array([0, b - a], np.int32), case.scale)
        assert_attention_close(p[a:b], ref, f"{name}, sequence {s}")


def test_persistent_grid_resets_its_counters_on_every_call():
    """The same workspace on consecutive calls, and filled with 0xFF between
    them: the claim counters are zeroed by each call before its grid runs."""
    dev, case, kc_h, vc_h, tables_h, lens_h, q_h, qs_h, _ = _setup("d128 pairs x8")
    kc, vc, q = (torch.from_numpy(x).to(dev) for x in (kc_h, vc_h, q_h))
    t, l, qs = (torch.from_numpy(x).to(dev) for x in (tables_h, lens_h, qs_h))
    ws = torch.zeros(256, dtype=torch.uint8, device=dev)
    a = _run(dev, q, kc, vc, t, l, qs, case.scale, workspace=ws)
    b = _run(dev, q, kc, vc, t, l, qs, case.scale, workspace=ws)
    ws.fill_(255)
    c = _run(dev, q, kc, vc, t, l, qs, case.scale, workspace=ws)
    o = _run(dev, q, kc, vc, t, l, qs, case.scale, split=False)
    for x, what in ((a, "first"), (b, "second"), (c, "after 0xFF")):
        assert np.array_equal(bits(x), bits(o)), what


@pytest.mark.parametrize("chunked", [False, True])
def test_persistent_prefill_append_matches_one_workgroup_per_item(chunked):
    """pa_prefill_append on the persistent grid: outputs and the new tokens'
    cache writes bit for bit as with one workgroup per item, and the caches
    equal to the oracle's scatter."""
    lens_l = [2 * n for n in MIX] * 2 if chunked else MIX * 2
    H, Hkv, D, B = 16, 16, 128, 16
    case = workloads.random_case(1400 + chunked, lens_l, H, Hkv, D, B)
    ms = [max(1, n // 2) for n in lens_l] if chunked else list(lens_l)
    kc0, vc0, kc1, vc1, key_h, val_h, tables_h, lens_h = _append_case(case, ms)
    q_h, qs_h = _queries(1400, ms, H, D)
    dev = device()
    assert _items(ms, H, Hkv, 128) > 3 * torch.cuda.get_device_properties(dev).multi_processor_count
    assert _row_tiles(ms, H, Hkv, 128) * 128 >= 1024
    assert pa.pa_prefill_workspace_size(int(qs_h[-1]), len(lens_l), H, Hkv, D, B, tables_h.shape[1], max(ms)) == 256
    say(f"persistent prefill_append chunked={chunked}: rows {int(qs_h[-1])}")
    q, key, val = (torch.from_numpy(x).to(dev) for x in (q_h, key_h, val_h))
    t, l, qs = (torch.from_numpy(x).to(dev) for x in (tables_h, lens_h, qs_h))
    res = []
    for split in (True, False):
        kc, vc = torch.from_numpy(kc0).to(dev), torch.from_numpy(vc0).to(dev)
        out = torch.full(q.shape, float("nan"), dtype=torch.float16, device=dev)
        pa.pa_prefill_append(out, q, key, val, kc, vc, t, l, qs, case.scale, max_query_len=max(ms), split=split)
        torch.cuda.synchronize()
        res.append((bits(out), bits(kc), bits(vc)))
    (po, pk, pv), (oo, ok, ov) = res
    assert np.array_equal(po, oo) and np.array_equal(pk, ok) and np.array_equal(pv, ov)
    assert np.array_equal(pk, kc1.view(np.uint16)) and np.array_equal(pv, vc1.view(np.uint16))
    s = 3
    a, b = int(qs_h[s]), int(qs_h[s + 1])
    ref = oracle.prefill(np.ascontiguousarray(q_h[a:b]), kc1, vc1, np.ascontiguousarray(tables_h[[s]]),
                         np.ascontiguousarray(lens_h[[s]]), np.array([0, b - a], np.int32), case.scale)
    assert_attention_close(po[a:b].view(np.float16), ref, f"append chunked={chunked}, sequence {s}")


def test_persistent_grid_replays_in_a_hip_graph():
    """The counter reset and the persistent grid captured in one graph,
    replayed three times with eager work between (workspace filled with 0xFF,
    output with NaN): every replay reproduces the eager output bit for bit."""
    dev, case, kc_h, vc_h, tables_h, lens_h, q_h, qs_h, _ = _setup("d128 16 heads")
    kc, vc, q = (torch.from_numpy(x).to(dev) for x in (kc_h, vc_h, q_h))
    t, l, qs = (torch.from_numpy(x).to(dev) for x in (tables_h, lens_h, qs_h))
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    out = torch.empty(q.shape, dtype=torch.float16, device=dev)
    mq = max(CASES["d128 16 heads"][0])

    def call():
        pa.pa_prefill(out, q, kc, vc, t, l, qs, case.scale, max_query_len=mq, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = bits(out).copy()
    assert np.array_equal(eager, bits(_run(dev, q, kc, vc, t, l, qs, case.scale, split=False)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        call()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        ws.fill_(255)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), eager), f"replay {rep}"
