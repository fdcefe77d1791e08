"""GPU parity of pa_reshape_and_cache and pa_copy_blocks (through the C ABI):
bit for bit against the oracle, untouched bytes included."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_390_amd as pa
from gpu_common import bits, device, say

pytestmark = pytest.mark.gpu


def _random_pool(rng, NB, Hkv, B, D):
    return rng.integers(0, 1 << 16, size=(NB, Hkv, B, D), dtype=np.uint16).view(np.float16)


@pytest.mark.parametrize("D,B,T,Hkv", [(128, 16, 64, 4), (128, 16, 3000, 4), (16, 4, 19, 4), (256, 1, 40, 4),
                                       (64, 64, 500, 4), (32, 128, 257, 4),
                                       # several lane groups per token; a block size that is no power of two
                                       (128, 16, 64, 32), (256, 16, 33, 40), (64, 12, 100, 3), (16, 48, 70, 5)])
@pytest.mark.parametrize("layout", ["contiguous", "strided", "misaligned"])
def test_scatter_bit_exact(D, B, T, Hkv, layout):
    dev = device()
    rng = np.random.default_rng(D + B + T + Hkv)
    NB = (T + B - 1) // B + 5
    kc_h, vc_h = _random_pool(rng, NB, Hkv, B, D), _random_pool(rng, NB, Hkv, B, D)
    slots = rng.permutation(NB * B)[:T].astype(np.int64)
    slots[::7] = -1                                      # padding: skipped
    slots[3::11] = NB * B + 2                            # outside the pool: skipped
    if layout == "contiguous":
        base = rng.standard_normal((T, Hkv, D)).astype(np.float16)
        key_d = torch.from_numpy(base).to(dev)
        val_d = torch.from_numpy(base[::-1].copy()).to(dev)
    elif layout == "strided":                            # K and V views into a fused [T, 3, Hkv, D]
        base = rng.standard_normal((T, 3, Hkv, D)).astype(np.float16)
        fused = torch.from_numpy(base).to(dev)
        key_d, val_d = fused[:, 1], fused[:, 2]
    else:                                                # 2-byte offset: no 16-byte vectors
        base = rng.standard_normal((T * Hkv * D + 1,)).astype(np.float16)
        flat = torch.from_numpy(base).to(dev)
        key_d = flat[1:].view(T, Hkv, D)
        val_d = flat[:-1].view(T, Hkv, D)
    key_h = np.ascontiguousarray(key_d.cpu().numpy())
    val_h = np.ascontiguousarray(val_d.cpu().numpy())
    kc, vc = torch.from_numpy(kc_h).to(dev), torch.from_numpy(vc_h).to(dev)
    say(f"scatter D={D} B={B} T={T} Hkv={Hkv} {layout}")
    pa.pa_reshape_and_cache(key_d, val_d, torch.from_numpy(slots).to(dev), kc, vc)
    torch.cuda.synchronize()
    valid = (slots >= 0) & (slots < NB * B)
    sl = np.where(valid, slots, -1)
    oracle.reshape_and_cache(key_h, val_h, sl, kc_h, vc_h)
    assert np.array_equal(bits(kc), kc_h.view(np.uint16))
    assert np.array_equal(bits(vc), vc_h.view(np.uint16))


@pytest.mark.parametrize("L", [1, 3, 70])
@pytest.mark.parametrize("D,B", [(128, 16), (16, 4), (256, 64)])
def test_copy_blocks_bit_exact(L, D, B):
    dev = device()
    rng = np.random.default_rng(L * 100 + D + B)
    Hkv, NB = 2, 24
    ks_h = [_random_pool(rng, NB, Hkv, B, D) for _ in range(L)]
    vs_h = [_random_pool(rng, NB, Hkv, B, D) for _ in range(L)]
    ks = [torch.from_numpy(a).to(dev) for a in ks_h]
    vs = [torch.from_numpy(a).to(dev) for a in vs_h]
    pairs = np.array([[3, 10], [3, 11], [5, 12], [0, 23], [7, 99], [-1, 13]], dtype=np.int64)
    say(f"copy L={L} D={D} B={B}")
    pa.pa_copy_blocks(ks, vs, torch.from_numpy(pairs).to(dev))
    torch.cuda.synchronize()
    oracle.copy_blocks(ks_h, vs_h, pairs[:4].copy())     # ids outside the pool are skipped
    for l in range(L):
        assert np.array_equal(bits(ks[l]), ks_h[l].view(np.uint16))
        assert np.array_equal(bits(vs[l]), vs_h[l].view(np.uint16))


def test_copy_blocks_misaligned_fallback():
    dev = device()
    rng = np.random.default_rng(1)
    NB, Hkv, B, D = 10, 1, 4, 16
    flat_h = rng.integers(0, 1 << 16, size=NB * Hkv * B * D + 1, dtype=np.uint16).view(np.float16)
    flat = torch.from_numpy(flat_h).to(dev)
    k = flat[1:].view(NB, Hkv, B, D)                     # 2-byte offset
    v_h = _random_pool(rng, NB, Hkv, B, D)
    v = torch.from_numpy(v_h).to(dev)
    pairs = np.array([[1, 2], [1, 9]], dtype=np.int64)
    pa.pa_copy_blocks([k], [v], torch.from_numpy(pairs).to(dev))
    torch.cuda.synchronize()
    k_h = np.ascontiguousarray(flat_h[1:].reshape(NB, Hkv, B, D))
    oracle.copy_blocks([k_h], [v_h], pairs)
    assert np.array_equal(bits(k), k_h.view(np.uint16))
    assert np.array_equal(bits(v), v_h.view(np.uint16))
