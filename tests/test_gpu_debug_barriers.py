"""Race check on the GPU: the library built with -DATTN_DEBUG_BARRIERS
(full workgroup barriers added after each key/value tile's loads are issued
and after its compute) must give bitwise the same outputs as the normal
build, for the forward instances, the backward and decode.  The kernels have
no atomics and a fixed reduction order, so the only way the two builds can
differ is a missing wait in the normal build (an LDS stage read before its
loads landed, or overwritten while still read)."""
import ctypes
import math
import os
import sys

import numpy as np
import pytest

import exact_attention_123_amd as ea
from gpu_util import to_device
from seeded_inputs import make_decode, make_dout, make_qkv

pytestmark = pytest.mark.gpu

DEBUG_LIB = os.path.join(os.path.dirname(ea.LIB_PATH), "libattn_debug_barriers.so")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dbg():
    if not os.path.exists(DEBUG_LIB):
        pytest.fail(f"{DEBUG_LIB} is missing: build() compiles it next to libattn.so")
    ea.load_library()  # torch first, then the library: one HIP runtime
    lib = ctypes.CDLL(DEBUG_LIB)
    for name, (res, args) in ea.EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


@pytest.mark.parametrize("B,H,T,d,causal", [(1, 32, 2000, 128, 1), (1, 8, 4000, 128, 0),
                                            (1, 32, 2000, 64, 1), (2, 2, 700, 128, 1)],
                         ids=["w8", "w4", "w8_d64", "rows"])
def test_forward_matches_debug_build(dbg, B, H, T, d, causal):
    import torch
    name = ea.fwd_kernel_name_for(B, H, T, d, causal)
    say(f"[debug barriers fwd] {name} B={B} H={H} T={T} d={d}")
    x = make_qkv(B, H, T, d, dtype="bf16", seed=9600 + T, qk_mult=4.0)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    scale = 1.0 / math.sqrt(d)
    o1, l1 = ea.forward(q, k, v, causal=bool(causal), scale=scale)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    st = dbg.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                      B, H, T, d, causal, scale, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_backward_matches_debug_build(dbg):
    import torch
    B, H, T, d = 1, 4, 1000, 128
    say(f"[debug barriers bwd] B={B} H={H} T={T} d={d}")
    x = make_qkv(B, H, T, d, dtype="bf16", seed=9700, qk_mult=2.0)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    dout = to_device(make_dout(B, H, T, d, seed=9701), "bf16")
    scale = 1.0 / math.sqrt(d)
    o, lse = ea.forward(q, k, v, causal=True, scale=scale)
    g1 = ea.backward(q, k, v, o, lse, dout, causal=True, scale=scale)
    g2 = [torch.empty_like(t) for t in (q, k, v)]
    ws = torch.empty(2 * B * H * T, dtype=torch.float32, device=q.device)
    st = dbg.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                      lse.data_ptr(), g2[0].data_ptr(), g2[1].data_ptr(), g2[2].data_ptr(),
                      ws.data_ptr(), B, H, T, d, 1, scale,
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_decode_matches_debug_build(dbg):
    import torch
    B, H, Hkv, Tq, Tk, d = 2, 16, 4, 1, 20000, 128
    say(f"[debug barriers decode] B={B} H={H} H_kv={Hkv} Tq={Tq} Tk={Tk}")
    x = make_decode(B, H, Hkv, Tq, Tk, d, seed=9800)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    scale = 1.0 / math.sqrt(d)
    o1, l1 = ea.decode(q, k, v, causal=True, scale=scale)
    need = ea.decode_workspace_bytes(B, H, Hkv, Tq, Tk, d)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    st = dbg.attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                         ws.data_ptr(), need, B, H, Hkv, Tq, Tk, Tk, d, 1, scale,
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
