"""GPU parity across the two workgroup orders of the large-grid kernels.

The 8-wave forward, the dK/dV and the dQ kernels place two heads at a time
on each XCD when the head count is a multiple of 16 (eight XCDs, two heads
in flight), and otherwise walk all heads within each block index.  The
order changes which workgroup computes which (head, block), nothing else;
these cases pin both branches against the float64 oracle (bf16 tolerances
for the forward, the per-element bound of the backward tests)."""
import math
import sys

import numpy as np
import pytest

import oracle
from gpu_util import to_device
from seeded_inputs import make_dout, make_qkv
from test_gpu_bwd import U, check_head, gpu_backward, sampled
from test_gpu_gqa import check_bwd

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("B,H,T", [(1, 48, 1500), (1, 24, 2816), (3, 8, 2816)],
                         ids=["heads48_two_in_flight", "heads24_all", "heads24_batched"])
def test_forward_orders(B, H, T):
    import torch

    import exact_attention_123_amd as ea
    d = 128
    name = ea.fwd_kernel_name_for(B, H, T, d, True)
    assert name.endswith("_w8"), name
    say(f"[order fwd] {name} B={B} H={H} T={T} (B*H % 16 == {B * H % 16})")
    x = make_qkv(B, H, T, d, dtype="bf16", seed=9900 + H + T, qk_mult=4.0)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    scale = 1.0 / math.sqrt(d)
    o, lse = ea.forward(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    O = o.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    rng = np.random.Generator(np.random.PCG64(9901))
    rows = np.unique(np.r_[0, 255, 256, T - 1, rng.choice(T, 40, replace=False)])
    for b in range(B):
        for h in range(H):  # every head: each one lands on a different workgroup set
            ref = oracle.attention_head(x.q64(b, h), x.k64(b, h), x.v64(b, h), causal=True,
                                        scale=scale, rows=rows)
            assert np.abs(O[b, h, rows] - ref["O"]).max() <= 2e-2, (b, h)
            assert np.abs(L[b, h, rows] - ref["LSE"]).max() <= 1e-3, (b, h)


@pytest.mark.parametrize("H,T", [(16, 700), (8, 700)], ids=["heads16_two_in_flight",
                                                            "heads8_all"])
def test_backward_orders(H, T):
    B, d = 1, 128
    say(f"[order bwd] B={B} H={H} T={T}")
    x = make_qkv(B, H, T, d, seed=9910 + H, qk_mult=2.0)
    do = make_dout(B, H, T, d, seed=9911 + H)
    scale = 1.0 / math.sqrt(d)
    res = gpu_backward(x, do, True, scale)
    for h in (0, 5, H - 1):
        idx = sampled(T, 9912 + h, n=48)
        check_head(x, do, 0, h, res, True, scale, rows=idx, keys=idx, ub=2 * U)


@pytest.mark.parametrize("H,Hkv", [(32, 16), (32, 8)], ids=["kv16_two_in_flight", "kv8_all"])
def test_grouped_backward_orders(H, Hkv):
    """Grouped heads: with 16 key/value heads both backward kernels take the
    two-heads-in-flight order; with 8 the dK/dV kernel walks all of them
    while the dQ kernel (32 query heads) still takes two in flight."""
    import torch

    import exact_attention_123_amd as ea
    B, T, d = 1, 300, 64
    say(f"[order gqa bwd] H={H} H_kv={Hkv} T={T} d={d}")
    scale = 1.0 / math.sqrt(d)
    x = make_qkv(B, H, T, d, seed=9920 + Hkv, qk_mult=2.0, H_kv=Hkv)
    do_bits = make_dout(B, H, T, d, seed=9921)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    o, lse = ea.forward(q, k, v, causal=True, scale=scale)
    dq, dk, dv = ea.backward(q, k, v, o, lse, to_device(do_bits, "bf16"), causal=True,
                             scale=scale)
    torch.cuda.synchronize()
    O = o.float().cpu().numpy().astype(np.float64)
    dQ, dK, dV = (t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))
    for g in range(Hkv):
        check_bwd(x, do_bits, dQ, dK, dV, O, True, scale, 0, g, ub=2 * U)
