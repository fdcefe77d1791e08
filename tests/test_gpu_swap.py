"""GPU parity of the swap path: pa_bm_swap_out / pa_bm_swap_in pairs and
pa_swap_blocks (device <-> pinned host block copies) against the oracle's
block model and block moves, through the C ABI; decode after a swap round
trip must be bitwise what it was before (the kernel's arithmetic depends
only on logical positions, not on where the blocks live)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_390_amd as pa
from gpu_common import bits, device, say
from oracle.block_manager import BlockManagerModel

pytestmark = pytest.mark.gpu


def _pools(dev, layers, NB, Hkv, B, D, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    caches = []
    for _ in range(layers):
        caches.append(torch.randn((NB, Hkv, B, D), generator=g, device=dev, dtype=torch.float16))
        caches.append(torch.randn((NB, Hkv, B, D), generator=g, device=dev, dtype=torch.float16))
    return caches                                     # K0, V0, K1, V1, ...


def _decode(dev, caches, layer, q, bm, seqs, width, B):
    tables, lens = bm.get_tables(seqs, width)
    out = torch.empty_like(q)
    pa.pa_decode(out, q, caches[2 * layer], caches[2 * layer + 1], torch.from_numpy(tables).to(dev),
                 torch.from_numpy(lens).to(dev), 1 / np.sqrt(q.shape[-1]), B, partition_size=128)
    return out


@pytest.mark.parametrize("H,Hkv,B", [(8, 4, 16), (4, 4, 8), (16, 2, 32)])
def test_swap_round_trip_is_exact(H, Hkv, B):
    dev = device()
    D, NB, NH, L = 128, 48, 40, 2
    caches = _pools(dev, L, NB, Hkv, B, D, seed=11 + B)
    hosts = [torch.zeros((NH, Hkv, B, D), dtype=torch.float16).pin_memory() for _ in range(2 * L)]
    bm = pa.BlockManager(NB, B, NH)
    m = BlockManagerModel(NB, B, NH)
    for obj in (bm, m):
        obj.add_sequence(0, 5 * B + 3)
        obj.add_sequence(1, 2 * B)
        obj.fork(0, 2)
        obj.add_sequence(3, B + 1)
    seqs = [0, 1, 2, 3]
    q = torch.randn((4, H, D), device=dev, dtype=torch.float16)
    width = 8
    before = [_decode(dev, caches, l, q, bm, seqs, width, B) for l in range(L)]
    torch.cuda.synchronize()

    group = [0, 2, 1]                                 # sequence 3 stays resident
    out_pairs = bm.swap_out(group)
    assert [tuple(p) for p in out_pairs.tolist()] == m.swap_out(group)
    dev_ref = [c.cpu().numpy() for c in caches]
    say(f"swap out H={H}/{Hkv} B={B}: {len(out_pairs)} blocks x {2 * L} caches")
    pa.pa_swap_blocks(caches, hosts, torch.from_numpy(out_pairs).to(dev), pa.PA_SWAP_OUT)
    torch.cuda.synchronize()
    host_ref = [np.zeros((NH, Hkv, B, D), np.float16) for _ in range(2 * L)]
    oracle.move_blocks(host_ref, dev_ref, out_pairs)
    for h, r in zip(hosts, host_ref):
        assert np.array_equal(h.numpy().view(np.uint16), r.view(np.uint16))

    for c in caches:                                  # the freed blocks get reused by others
        freed = torch.from_numpy(np.array(bm.free_list(), dtype=np.int64)).to(dev)
        c.index_fill_(0, freed, float("nan"))
    in_pairs = bm.swap_in(group)
    assert [tuple(p) for p in in_pairs.tolist()] == m.swap_in(group)
    dev_ref = [c.cpu().numpy() for c in caches]
    pa.pa_swap_blocks(caches, hosts, torch.from_numpy(in_pairs).to(dev), pa.PA_SWAP_IN)
    torch.cuda.synchronize()
    oracle.move_blocks(dev_ref, [h.numpy() for h in hosts], in_pairs)
    for c, r in zip(caches, dev_ref):
        assert np.array_equal(bits(c), r.view(np.uint16))
    after = [_decode(dev, caches, l, q, bm, seqs, width, B) for l in range(L)]
    torch.cuda.synchronize()
    for a, b in zip(before, after):
        assert np.array_equal(bits(a), bits(b))


def test_swap_of_a_long_sequence_at_the_llama_shape():
    """One 2048-token sequence of the Llama-2-7B head shape (32 x 128,
    B = 16): 128 blocks of 128 KiB per cache, out and back, bit for bit."""
    dev = device()
    Hkv, B, D, NB, NH = 32, 16, 128, 160, 130
    caches = _pools(dev, 1, NB, Hkv, B, D, seed=3)
    hosts = [torch.zeros((NH, Hkv, B, D), dtype=torch.float16).pin_memory() for _ in range(2)]
    bm = pa.BlockManager(NB, B, NH)
    bm.add_sequence(0, 2048)
    orig = [c.clone() for c in caches]
    table0 = bm.table(0)
    pairs = bm.swap_out([0])
    assert len(pairs) == 128
    pa.pa_swap_blocks(caches, hosts, torch.from_numpy(pairs).to(dev), pa.PA_SWAP_OUT)
    torch.cuda.synchronize()
    for c in caches:
        c.fill_(float("nan"))
    back = bm.swap_in([0])
    pa.pa_swap_blocks(caches, hosts, torch.from_numpy(back).to(dev), pa.PA_SWAP_IN)
    torch.cuda.synchronize()
    table1 = bm.table(0)
    for c, o in zip(caches, orig):
        assert torch.equal(c[torch.tensor(table1, device=dev)].view(torch.int16),
                           o[torch.tensor(table0, device=dev)].view(torch.int16))


def test_swap_rejects_memory_of_the_wrong_kind():
    """Checked on the host before anything is enqueued: an unpinned host
    buffer, a device buffer given as the host side, host memory given as
    the device side, and pairs that are not device memory."""
    dev = device()
    L = pa.lib()
    NB, blk = 4, 2 * 16 * 8
    d = torch.zeros((NB, 2, 16, 8), dtype=torch.float16, device=dev)
    pinned = torch.zeros((NB, 2, 16, 8), dtype=torch.float16).pin_memory()
    unpinned = torch.zeros((NB, 2, 16, 8), dtype=torch.float16)
    pairs = torch.tensor([[0, 1]], dtype=torch.int64, device=dev)
    host_pairs = torch.tensor([[0, 1]], dtype=torch.int64)

    def call(dp, hp, pr, direction=pa.PA_SWAP_OUT):
        da = (ctypes.c_void_p * 1)(dp)
        ha = (ctypes.c_void_p * 1)(hp)
        return L.pa_swap_blocks(ctypes.cast(da, ctypes.c_void_p), ctypes.cast(ha, ctypes.c_void_p), 1, pr, 1,
                                NB, NB, blk, direction, pa.PA_DTYPE_F16, None)

    assert call(d.data_ptr(), unpinned.data_ptr(), pairs.data_ptr()) == pa.PA_ERR_INVALID
    assert call(d.data_ptr(), d.data_ptr(), pairs.data_ptr()) == pa.PA_ERR_INVALID
    assert call(pinned.data_ptr(), pinned.data_ptr(), pairs.data_ptr()) == pa.PA_ERR_INVALID
    assert call(d.data_ptr(), pinned.data_ptr(), host_pairs.data_ptr()) == pa.PA_ERR_INVALID
    assert call(d.data_ptr(), pinned.data_ptr(), pairs.data_ptr(), direction=7) == pa.PA_ERR_INVALID
    assert call(d.data_ptr(), pinned.data_ptr(), pairs.data_ptr()) == pa.PA_OK
    torch.cuda.synchronize()
