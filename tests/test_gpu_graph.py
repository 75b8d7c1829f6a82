"""HIP graph capture of the entry points: the forward (one kernel), the
backward (three kernels and a workspace) and the decode path (several key
splits with a merge kernel and a workspace; a prefill chunk on the row-chunk
kernel; a large chunk on the forward kernel over the cache) are captured into a
torch.cuda.CUDAGraph and replayed several times.  Between replays the inputs
are overwritten eagerly (host-to-device copies, then a synchronisation), and
every replay's outputs must equal, bit for bit, an eager call on the same
inputs: the kernels are deterministic and the library allocates nothing and
enqueues no memset, so a replay has nothing that could go stale.
"""
import math
import sys

import numpy as np
import pytest

from gpu_util import to_device
from seeded_inputs import f32_to_bf16_bits, make_decode, make_dout, make_qkv

pytestmark = pytest.mark.gpu

REPLAYS = 3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def fresh_bf16(shape, rng, mult=1.0):
    """A new seeded N(0,1) (times mult) bf16 tensor on the GPU."""
    import torch
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(mult)
    return torch.from_numpy(f32_to_bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)


def capture(fn):
    """Warm fn up on a side stream, then capture it into a graph."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("B,H,T", [(2, 4, 1000), (1, 48, 2048)], ids=["rows", "w8"])
def test_forward_graph_replays(B, H, T):
    import torch

    import exact_attention_123_amd as ea
    d = 128
    say(f"[graph fwd] {ea.fwd_kernel_name_for(B, H, T, d, True)} B={B} H={H} T={T}")
    if (B, H, T) == (1, 48, 2048):
        assert ea.fwd_kernel_name_for(B, H, T, d, True).endswith("_w8")
    x = make_qkv(B, H, T, d, dtype="bf16", seed=8100)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(d)
    g = capture(lambda: ea.forward(q, k, v, causal=True, scale=scale, out=o, lse=lse))
    rng = np.random.Generator(np.random.PCG64(8101))
    for rep in range(REPLAYS):
        q.copy_(fresh_bf16((B, H, T, d), rng, 2.0))
        k.copy_(fresh_bf16((B, H, T, d), rng))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_ref, l_ref = ea.forward(q, k, v, causal=True, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), rep


def test_backward_graph_replays():
    import torch

    import exact_attention_123_amd as ea
    say("[graph bwd]")
    B, H, T, d = 1, 4, 700, 128
    x = make_qkv(B, H, T, d, dtype="bf16", seed=8200)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    dout = to_device(make_dout(B, H, T, d, seed=8201), "bf16")
    scale = 1.0 / math.sqrt(d)
    o, lse = ea.forward(q, k, v, causal=True, scale=scale)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(2 * B * H * T, dtype=torch.float32, device=q.device)
    g = capture(lambda: ea.backward(q, k, v, o, lse, dout, causal=True, scale=scale, dq=dq,
                                    dk=dk, dv=dv, ws=ws))
    rng = np.random.Generator(np.random.PCG64(8202))
    for rep in range(REPLAYS):
        dout.copy_(fresh_bf16((B, H, T, d), rng))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = ea.backward(q, k, v, o, lse, dout, causal=True, scale=scale)
        torch.cuda.synchronize()
        for got, want in zip((dq, dk, dv), ref):
            assert torch.equal(got, want), rep


# Three decode routes: several key splits (split kernel, merge kernel,
# workspace); a prefill chunk of 600 rows per key/value head on the
# row-chunk kernel (one split, no workspace); and a chunk large enough for
# the forward kernel over the cache (key offset Tk - Tq).
@pytest.mark.parametrize("B,H,Hkv,Tq,Tk,d", [(1, 8, 2, 2, 20000, 128), (1, 8, 2, 150, 3000, 64),
                                            (2, 32, 8, 520, 1700, 128)],
                         ids=["splits", "rows", "forward"])
def test_decode_graph_replays(B, H, Hkv, Tq, Tk, d):
    import torch

    import exact_attention_123_amd as ea
    say(f"[graph decode] B={B} H={H} Hkv={Hkv} Tq={Tq} Tk={Tk} d={d}")
    splits = ea.decode_splits(B, H, Hkv, Tq, Tk)
    need = ea.decode_workspace_bytes(B, H, Hkv, Tq, Tk, d)
    assert (splits > 1) == (need > 0) == (Tq == 2)
    x = make_decode(B, H, Hkv, Tq, Tk, d, seed=8300 + Tq)
    q, kc, vc = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    scale = 1.0 / math.sqrt(d)
    g = capture(lambda: ea.decode(q, kc, vc, Tk=Tk, causal=True, scale=scale, out=o, lse=lse,
                                  ws=ws))
    rng = np.random.Generator(np.random.PCG64(8301 + Tq))
    for rep in range(REPLAYS):
        q.copy_(fresh_bf16((B, H, Tq, d), rng, 2.0))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_ref, l_ref = ea.decode(q, kc, vc, Tk=Tk, causal=True, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), rep
