"""GPU parity of the backward pass: attn_bwd against the float64 backward
oracle on the same seeded inputs, element by element.

Tolerance (per element, derived from the arithmetic).  With u = 2^-8 (twice
bf16's unit roundoff 2^-9):

  |dV - ref| <= u (P^T |dO| + |ref|)
  |dK - ref| <= u |scale| (|dS|^T |Q| + P^T diag(b) |Q|) + u |ref|
  |dQ - ref| <= u |scale| (|dS| |K| + diag(b) P |K|) + u |ref|
  |Delta - ref| <= u b + 1e-6,   b_i = sum_c |dO_ic| |O_ic|

The kernels round P (for dV) and dS (for dK, dQ) to bf16, each term of the
contraction then carries a relative error <= 2^-9, so the sum is off by at
most 2^-9 times the sum of the terms' magnitudes (the abs-value products
above); the bf16 output adds 2^-9 |ref|; fp32 accumulation over T <= 8192
terms adds at most 2^-11 of the magnitude sum.  Delta is computed from the
bf16-rounded O (relative error 2^-9 per element), which moves Delta_i by at
most 2^-9 b_i and dS_ij by P_ij times that: the diag(b) terms.  When O comes
from the GPU forward instead of the oracle (the chained tests), O's error is
larger and u for the b terms is doubled.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from gpu_util import to_device
from seeded_inputs import (bf16_bits_to_f32, f32_to_bf16_bits, make_dout, make_qkv,
                           make_workload)

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def gpu_backward(x, do_bits, causal, scale, o_lse=None):
    """Run attn_bwd on x, dO.  o_lse: (O bits [B,H,T,d], LSE float32) to feed
    in, or None to take them from the GPU forward.  Returns float64 dQ, dK,
    dV, the workspace, and the O and LSE used."""
    import torch

    import exact_attention_123_amd as ea
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    do = to_device(do_bits, "bf16")
    if o_lse is None:
        o, lse = ea.forward(q, k, v, causal=causal, scale=scale)
    else:
        o = to_device(o_lse[0], "bf16")
        lse = torch.from_numpy(np.ascontiguousarray(o_lse[1], dtype=np.float32)).cuda()
    dq, dk, dv = ea.backward(q, k, v, o, lse, do, causal=causal, scale=scale)
    B, H, T, d = x.shape
    ws = torch.full((2 * B * H * T,), float("nan"), dtype=torch.float32, device=q.device)
    dq2, dk2, dv2 = ea.backward(q, k, v, o, lse, do, causal=causal, scale=scale, ws=ws)
    torch.cuda.synchronize()
    # the call with a caller-supplied workspace gives the same bits
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    out = [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]
    o_bits = o.view(torch.int16).cpu().numpy().view(np.uint16)
    return out + [ws.cpu().numpy(), o_bits, lse.cpu().numpy()]


def oracle_inputs(x, causal, scale):
    """O (bf16 bits) and LSE (fp32) of the oracle forward, to isolate the
    backward from the forward kernel."""
    B, H, T, d = x.shape
    O = np.empty((B, H, T, d), dtype=np.uint16)
    L = np.empty((B, H, T), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            r = oracle.attention_head(x.q64(b, h), x.k64(b, h), x.v64(b, h), causal=causal,
                                      scale=scale)
            O[b, h] = f32_to_bf16_bits(r["O"].astype(np.float32))
            L[b, h] = r["LSE"].astype(np.float32)
    return O, L


def check_head(x, do_bits, b, h, res, causal, scale, rows=None, keys=None, ub=U):
    """Compare one head's gradients (selected rows / keys) with the oracle
    under the per-element bound; returns the largest error / bound ratio."""
    dQ, dK, dV, ws, o_bits, _ = res
    B, H, T, d = x.shape
    q, k, v, do = x.q64(b, h), x.k64(b, h), x.v64(b, h), f64(do_bits[b, h])
    ref = oracle.attention_head_bwd(q, k, v, do, causal=causal, scale=scale, rows=rows,
                                    keys=keys)
    r, j = ref["rows"], ref["keys"]
    P, dS = ref["P"], ref["dS"]
    O_used = f64(o_bits[b, h])
    bnd = (np.abs(do) * np.abs(O_used)).sum(1)           # b_i
    s = abs(scale)
    A_V = P[:, j].T @ np.abs(do)
    A_K = s * (np.abs(dS[:, j]).T @ np.abs(q) + P[:, j].T @ (bnd[:, None] * np.abs(q)))
    A_Q = s * (np.abs(dS[r]) @ np.abs(k) + (bnd[r, None] * P[r]) @ np.abs(k))
    worst = 0.0
    for name, got, want, A, u_a in (("dV", dV[b, h][j], ref["dV"], A_V, U),
                                     ("dK", dK[b, h][j], ref["dK"], A_K, ub),
                                     ("dQ", dQ[b, h][r], ref["dQ"], A_Q, ub)):
        assert np.all(np.isfinite(got)), f"non-finite {name}"
        tol = u_a * A + U * np.abs(want) + 1e-6
        ratio = np.abs(got - want) / tol
        i = np.unravel_index(np.argmax(ratio), ratio.shape)
        assert ratio[i] <= 1.0, (f"{name} head ({b},{h}) at {i}: got {got[i]:.6g} want "
                                 f"{want[i]:.6g} tol {tol[i]:.3g}")
        worst = max(worst, float(ratio.max()))
    n = B * H * T
    # the workspace: -Delta, and -LSE / scale (-LSE log2(e) for |scale| < 2^-32)
    delta = -ws[:n].reshape(B, H, T)[b, h][r]
    assert np.all(np.abs(delta - ref["Delta"]) <= ub * bnd[r] + 1e-6), "Delta"
    stat = ws[n:].reshape(B, H, T)[b, h][r]
    want = -ref["LSE"][r] / scale if abs(scale) >= 2.0 ** -32 else -ref["LSE"][r] * math.log2(math.e)
    assert np.all(np.abs(stat - want) <= 1e-5 * (1 + np.abs(want))), "LSE statistic"
    return worst


# ---------------------------------------------------------------------------
# Small and ragged shapes, every element, O and LSE from the oracle
# ---------------------------------------------------------------------------

EDGE_T = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 257, 1000]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("T", EDGE_T)
def test_bwd_ragged(T, causal, d):
    say(f"[bwd ragged] T={T} causal={causal} d={d}")
    B, H = 1, 2
    scale = 1.0 / math.sqrt(d)
    x = make_qkv(B, H, T, d, seed=3000 + T + d, qk_mult=2.0)
    do = make_dout(B, H, T, d, seed=4000 + T + d)
    res = gpu_backward(x, do, causal, scale, o_lse=oracle_inputs(x, causal, scale))
    for h in range(H):
        check_head(x, do, 0, h, res, causal, scale)


# 1e-12 and 0 take the kernels' unfolded exponent (|scale| < 2^-32), the
# others the folded one (score accumulator started from -LSE / scale; at
# 2^-31 that start value is about 1e10)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [-0.3, 0.0, 1e-12, 2.0 ** -31, 0.5, 1.0])
def test_bwd_other_scales(scale, d):
    say(f"[bwd scale] {scale} d={d}")
    B, H, T = 1, 2, 300
    x = make_qkv(B, H, T, d, seed=5000)
    do = make_dout(B, H, T, d, seed=5001)
    for causal in (True, False):
        res = gpu_backward(x, do, causal, scale, o_lse=oracle_inputs(x, causal, scale))
        for h in range(H):
            check_head(x, do, 0, h, res, causal, scale)


def test_bwd_chained_after_gpu_forward():
    """The training-step order: GPU forward, then GPU backward on its O, LSE."""
    say("[bwd chained] B=2 H=3 T=777 d=128")
    B, H, T, d = 2, 3, 777, 128
    scale = 1.0 / math.sqrt(d)
    x = make_qkv(B, H, T, d, seed=5100, qk_mult=4.0)
    do = make_dout(B, H, T, d, seed=5101)
    for causal in (True, False):
        res = gpu_backward(x, do, causal, scale)
        for b in range(B):
            for h in range(H):
                check_head(x, do, b, h, res, causal, scale, ub=2 * U)


def test_bwd_deterministic():
    import torch

    import exact_attention_123_amd as ea
    say("[bwd deterministic]")
    B, H, T, d = 1, 4, 1500, 128
    x = make_qkv(B, H, T, d, seed=5200)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    do = to_device(make_dout(B, H, T, d, seed=5201), "bf16")
    o, lse = ea.forward(q, k, v, causal=True)
    g1 = ea.backward(q, k, v, o, lse, do, causal=True)
    g2 = ea.backward(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------------------
# Full sizes: sampled rows and keys of some heads, invariants on every head
# ---------------------------------------------------------------------------

def sampled(T, seed, n=48):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, T // 2, T - 129, T - 65, T - 64, T - 1]
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.unique(np.clip(np.r_[fixed, rng.choice(T, n, replace=False)], 0, T - 1))


@pytest.mark.parametrize("name,causal,heads", [
    ("bf16_b1h32_t8192_d128_causal_qk4", True, [(0, 0), (0, 31)]),
    ("bf16_b4h16_t4096_d128", False, [(3, 15)]),
    ("bf16_b1h8_t2048_d64_causal", True, [(0, 5)]),
], ids=["t8192_causal_qk4", "t4096_full", "t2048_d64_causal"])
def test_bwd_full_size(name, causal, heads):
    say(f"[bwd full size] {name} causal={causal}")
    x = make_workload(name)
    B, H, T, d = x.shape
    scale = 1.0 / math.sqrt(d)
    do = make_dout(B, H, T, d, seed=x.seed + 7000)
    res = gpu_backward(x, do, causal, scale)
    dQ, dK, dV = res[:3]
    for (b, h) in heads:
        say(f"  head ({b},{h})")
        check_head(x, do, b, h, res, causal, scale, rows=sampled(T, 11 * h + b),
                   keys=sampled(T, 13 * h + b + 1), ub=2 * U)
    # invariants on every head: key gradients sum to zero, value gradients
    # sum to the summed dO (rows of P sum to one)
    dof = f64(do)
    for b in range(B):
        for h in range(H):
            sk = np.abs(dK[b, h].sum(0)).max()
            assert sk <= 2 * U * np.abs(dK[b, h]).sum(0).max() + 1e-3, (b, h, sk)
            dv_sum, do_sum = dV[b, h].sum(0), dof[b, h].sum(0)
            assert np.abs(dv_sum - do_sum).max() <= U * np.abs(dV[b, h]).sum(0).max() + 1e-3
