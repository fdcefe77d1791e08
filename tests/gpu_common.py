"""Shared helpers for the GPU parity tests (test infrastructure).

Inputs come from `workloads` (seeded); expected values come from `oracle`
only, computed on host copies of those inputs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

ATOL = 2e-3   # absolute part of the attention tolerance (fp16 KV, fp32 accumulate)
RTOL = 1e-2   # relative part: |gpu - oracle| <= ATOL + RTOL * |oracle|, per element


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def assert_attention_close(got, ref, what=""):
    """got: fp16 tensor/array, ref: float64 array; NaN rows must agree."""
    g = got.float().cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.array_equal(np.isnan(g), np.isnan(r)), f"{what}: NaN pattern differs"
    m = ~np.isnan(r)
    err = np.abs(g[m] - r[m])
    bound = ATOL + RTOL * np.abs(r[m])
    worst = np.argmax(err - bound) if err.size else 0
    ok = bool(np.all(err <= bound))
    rel = err / np.maximum(np.abs(r[m]), 1e-30)
    say(f"  {what}: max abs {err.max() if err.size else 0:.3e}  max rel(|r|>0.1) "
        f"{rel[np.abs(r[m]) > 0.1].max() if np.any(np.abs(r[m]) > 0.1) else 0:.3e}")
    assert ok, f"{what}: |got-ref|={err[worst]:.3e} > {bound[worst]:.3e} (ref {r[m][worst]:.4f})"


def bits(t):
    """Raw 16-bit patterns of an fp16 tensor/array (host numpy)."""
    a = t.cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)
    return a.view(np.uint16)


def poisoned_cache(NB, Hkv, B, D):
    return np.full((NB, Hkv, B, D), np.nan, dtype=np.float16)
