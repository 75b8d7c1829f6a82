"""The allocation-free decode entry point (attn_decode_noalloc) against
attn_decode, through the C ABI.

attn_decode_noalloc runs the same kernels as attn_decode but keeps the split
partial results in the library's own device scratch instead of a caller
workspace.  Two calls in a row (the second on a smaller problem, so that it
runs over what the first left in the scratch) must each give outputs
bit-identical to attn_decode on the same inputs, and both are checked
against the float64 decode oracle at the bf16 tolerances (2e-2 on O, 1e-3
on LSE).  A problem whose split results exceed the scratch is rejected.
"""
import gc
import math
import sys

import numpy as np
import pytest

import oracle
from gpu_util import to_device
from seeded_inputs import bf16_bits_to_f32, make_decode

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_pair(B, H, Hkv, Tq, Tk, d, seed, causal=True):
    import torch

    import exact_attention_123_amd as ea
    x = make_decode(B, H, Hkv, Tq, Tk, d, seed=seed, Tk_cap=Tk + 64)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    scale = 1.0 / math.sqrt(d)
    splits = ea.decode_splits(B, H, Hkv, Tq, Tk)
    need = ea.decode_workspace_bytes(B, H, Hkv, Tq, Tk, d)
    say(f"[no-alloc decode] B={B} H={H} H_kv={Hkv} Tq={Tq} Tk={Tk} d={d} splits={splits} "
        f"scratch bytes={need}")
    assert splits > 1 and 0 < need <= ea.DECODE_NOALLOC_MAX_BYTES
    # reference: the existing entry point with a caller workspace
    o_ref, l_ref = ea.decode(q, k, v, Tk=Tk, causal=causal, scale=scale)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Tq), float("nan"), dtype=torch.float32, device=q.device)
    torch.cuda.synchronize()
    # the collector stays off while the allocation count is compared, so
    # that no earlier test's tensors are freed in between
    gc.collect()
    gc.disable()
    try:
        before = torch.cuda.memory_allocated()
        st = ea.attn_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), B, H, Hkv, Tq, Tk, Tk + 64, d, causal, scale,
                                    torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        after = torch.cuda.memory_allocated()
    finally:
        gc.enable()
    assert st == 0, ea.status_string(st)
    assert after == before
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    O = o.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    G = H // Hkv
    eo = el = 0.0
    for b in range(B):
        for h in (0, H - 1):
            ref = oracle.attention_decode_head(
                bf16_bits_to_f32(x.q[b, h]).astype(np.float64),
                bf16_bits_to_f32(x.k[b, h // G, :Tk]).astype(np.float64),
                bf16_bits_to_f32(x.v[b, h // G, :Tk]).astype(np.float64),
                causal=causal, scale=scale)
            eo = max(eo, float(np.abs(O[b, h] - ref["O"]).max()))
            el = max(el, float(np.abs(L[b, h] - ref["LSE"]).max()))
    say(f"    bitwise equal to attn_decode; max|O err|={eo:.3e} max|LSE err|={el:.3e}")
    assert eo <= 2e-2 and el <= 1e-3


def test_noalloc_decode_two_calls_then_smaller():
    run_pair(4, 32, 8, 1, 20000, 128, seed=9500)  # 5 splits
    run_pair(2, 8, 2, 3, 9000, 64, seed=9501)     # smaller: 3 splits, d = 64


def test_noalloc_decode_rejects_oversized():
    import torch

    import exact_attention_123_amd as ea
    B, H, Hkv, Tq, Tk, d = 1, 300, 300, 32, 8192, 128
    assert ea.decode_workspace_bytes(B, H, Hkv, Tq, Tk, d) > ea.DECODE_NOALLOC_MAX_BYTES
    q = torch.zeros((B, H, Tq, d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, Hkv, Tk, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device="cuda")
    st = ea.attn_decode_noalloc(q.data_ptr(), kv.data_ptr(), kv.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), B, H, Hkv, Tq, Tk, Tk, d, 1, 0.1, 0)
    assert st == 9, ea.status_string(st)
