"""Helpers for the GPU tests: upload seeded inputs, run the library, compare
with the oracle."""
from __future__ import annotations

import math

import numpy as np

import exact_attention_123_amd as ea
from seeded_inputs import QKV

TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3)}  # (O max abs, LSE max abs)


def to_device(a: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def run(x: QKV, causal: bool, scale: float | None = None):
    """Upload x, run the fused forward, return (O float64 numpy, LSE numpy)."""
    import torch
    q, k, v = (to_device(a, x.dtype) for a in (x.q, x.k, x.v))
    d = x.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = ea.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def max_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.all(np.isfinite(a)), "non-finite values in GPU output"
    return float(np.max(np.abs(a - b))) if a.size else 0.0
