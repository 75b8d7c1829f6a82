"""GPU parity of the grouped-query variants (attn_fwd_gqa, attn_bwd_gqa)
against the float64 grouped-query oracle, on the same seeded inputs.

Forward tolerances as for the forward (bf16: 2e-2 on O, 1e-3 on LSE, max
abs).  Backward: the per-element bound of the backward parity tests, with the
magnitude sums of dK and dV taken over every query head of the group (a
key/value head's gradient is the sum of its query heads' contributions).
"""
import math
import sys

import numpy as np
import pytest

import oracle
from gpu_util import to_device
from seeded_inputs import bf16_bits_to_f32, make_dout, make_qkv, make_workload

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def gpu_fwd(x, causal, scale):
    import torch

    import exact_attention_123_amd as ea
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    o, lse = ea.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (q, k, v, o, lse), o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("H,Hkv", [(8, 1), (8, 2), (8, 4), (6, 3)])
@pytest.mark.parametrize("T", [1, 100, 257, 1000])
def test_gqa_forward(T, H, Hkv, causal, d):
    say(f"[gqa fwd] T={T} H={H} Hkv={Hkv} causal={causal} d={d}")
    B = 2
    scale = 1.0 / math.sqrt(d)
    x = make_qkv(B, H, T, d, seed=6000 + T + H + Hkv + d, qk_mult=2.0, H_kv=Hkv)
    _, O, L = gpu_fwd(x, causal, scale)
    Oref, Lref = oracle.attention_gqa(x.q64(), x.k64(), x.v64(), causal=causal, scale=scale)
    assert np.isfinite(O).all()
    assert np.abs(O - Oref).max() <= 2e-2
    assert np.abs(L - Lref).max() <= 1e-3


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_gqa_forward_row_chunks_long(causal):
    """Grouped heads on the row-chunk kernel with 8 waves (a small grid of a
    long sequence): 32-row chunks of the group's rows, keys split 8 ways."""
    import exact_attention_123_amd as ea
    B, H, Hkv, T, d = 1, 4, 2, 4500, 64
    assert ea.fwd_kernel_name_for(B, H, T, d, causal).endswith("_w8")
    say(f"[gqa fwd rows] T={T} H={H} Hkv={Hkv} causal={causal} d={d}")
    scale = 1.0 / math.sqrt(d)
    x = make_qkv(B, H, T, d, seed=6100 + int(causal), qk_mult=2.0, H_kv=Hkv)
    _, O, L = gpu_fwd(x, causal, scale)
    Oref, Lref = oracle.attention_gqa(x.q64(), x.k64(), x.v64(), causal=causal, scale=scale)
    assert np.isfinite(O).all()
    assert np.abs(O - Oref).max() <= 2e-2
    assert np.abs(L - Lref).max() <= 1e-3


def check_bwd(x, do_bits, dQ, dK, dV, O_used, causal, scale, b, g, keys=None, ub=U):
    """Gradients of key/value head (b, g) and of its query heads against the
    oracle under the per-element bound (rows: the query heads' sampled keys
    positions too when `keys` is given)."""
    H, Hkv = x.q.shape[1], x.k.shape[1]
    G = H // Hkv
    T = x.q.shape[2]
    j = np.arange(T) if keys is None else np.asarray(keys)
    k64, v64 = x.k64(b, g), x.v64(b, g)
    dK_ref = np.zeros((len(j), k64.shape[1]))
    dV_ref = np.zeros_like(dK_ref)
    A_K = np.zeros_like(dK_ref)
    A_V = np.zeros_like(dK_ref)
    s = abs(scale)
    for m in range(G):
        h = g * G + m
        q64, do = x.q64(b, h), f64(do_bits[b, h])
        ref = oracle.attention_head_bwd(q64, k64, v64, do, causal=causal, scale=scale,
                                        rows=j, keys=j)
        P, dS = ref["P"], ref["dS"]
        bnd = (np.abs(do) * np.abs(O_used[b, h])).sum(1)
        dK_ref += ref["dK"]
        dV_ref += ref["dV"]
        A_V += P[:, j].T @ np.abs(do)
        A_K += s * (np.abs(dS[:, j]).T @ np.abs(q64) + P[:, j].T @ (bnd[:, None] * np.abs(q64)))
        A_Q = s * (np.abs(dS[j]) @ np.abs(k64) + (bnd[j, None] * P[j]) @ np.abs(k64))
        tol = ub * A_Q + U * np.abs(ref["dQ"]) + 1e-6
        assert (np.abs(dQ[b, h][j] - ref["dQ"]) <= tol).all(), f"dQ head {h}"
    tol = U * A_V + U * np.abs(dV_ref) + 1e-6
    assert (np.abs(dV[b, g][j] - dV_ref) <= tol).all(), f"dV kv head {g}"
    tol = ub * A_K + U * np.abs(dK_ref) + 1e-6
    assert (np.abs(dK[b, g][j] - dK_ref) <= tol).all(), f"dK kv head {g}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (6, 2)])
@pytest.mark.parametrize("T", [65, 300])
def test_gqa_backward(T, H, Hkv, causal, d):
    import torch

    import exact_attention_123_amd as ea
    say(f"[gqa bwd] T={T} H={H} Hkv={Hkv} causal={causal} d={d}")
    B = 1
    scale = 1.0 / math.sqrt(d)
    x = make_qkv(B, H, T, d, seed=6500 + T + H + Hkv + d, qk_mult=2.0, H_kv=Hkv)
    do_bits = make_dout(B, H, T, d, seed=6600 + T + d)
    (q, k, v, o, lse), O, _ = gpu_fwd(x, causal, scale)
    dq, dk, dv = ea.backward(q, k, v, o, lse, to_device(do_bits, "bf16"), causal=causal,
                             scale=scale)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape and dq.shape == q.shape
    dQ, dK, dV = (t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))
    for g in range(Hkv):
        check_bwd(x, do_bits, dQ, dK, dV, O, causal, scale, 0, g, ub=2 * U)


def test_gqa_matches_repeated_heads():
    """Grouped call == ordinary call on K, V repeated G times per group (the
    GPU path against itself, bit for bit: the grouping changes only which
    head's memory is read)."""
    import torch

    import exact_attention_123_amd as ea
    say("[gqa repeat]")
    B, H, Hkv, T, d = 2, 8, 2, 700, 128
    x = make_qkv(B, H, T, d, seed=6700, H_kv=Hkv)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    G = H // Hkv
    kr = k.repeat_interleave(G, dim=1).contiguous()
    vr = v.repeat_interleave(G, dim=1).contiguous()
    o1, l1 = ea.forward(q, k, v, causal=True)
    o2, l2 = ea.forward(q, kr, vr, causal=True)
    do = to_device(make_dout(B, H, T, d, seed=6701), "bf16")
    g1 = ea.backward(q, k, v, o1, l1, do, causal=True)
    g2 = ea.backward(q, kr, vr, o2, l2, do, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    assert torch.equal(g1[0].view(torch.int16), g2[0].view(torch.int16))
    # dK, dV: the group sum of the repeated call's per-head gradients, up to
    # fp32 summation order (the grouped kernel accumulates the whole group
    # in one register sum before rounding to bf16)
    for a, b in ((g1[1], g2[1]), (g1[2], g2[2])):
        summed = b.float().view(B, Hkv, G, T, d).sum(2)
        err = (a.float() - summed).abs().max().item()
        assert err <= 2 * U * summed.abs().max().item() + 1e-3, err


def test_gqa_full_size():
    import torch

    import exact_attention_123_amd as ea
    name = "bf16_b1h32kv8_t8192_d128_causal"
    say(f"[gqa full size] {name}")
    x = make_workload(name)
    B, H, T, d = x.shape
    Hkv = x.k.shape[1]
    scale = 1.0 / math.sqrt(d)
    (q, k, v, o, lse), O, L = gpu_fwd(x, True, scale)
    rng = np.random.Generator(np.random.PCG64(61))
    rows = np.unique(np.r_[0, 1, 63, 64, 255, 256, T // 2, T - 1, rng.choice(T, 40)])
    for h in (0, 3, 4, 31):
        g = h // (H // Hkv)
        ref = oracle.attention_head(x.q64(0, h), x.k64(0, g), x.v64(0, g), causal=True,
                                    scale=scale, rows=rows)
        assert np.abs(O[0, h][rows] - ref["O"]).max() <= 2e-2, h
        assert np.abs(L[0, h][rows] - ref["LSE"]).max() <= 1e-3, h
    do_bits = make_dout(B, H, T, d, seed=x.seed + 7000)
    dq, dk, dv = ea.backward(q, k, v, o, lse, to_device(do_bits, "bf16"), causal=True,
                             scale=scale)
    torch.cuda.synchronize()
    dQ, dK, dV = (t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))
    check_bwd(x, do_bits, dQ, dK, dV, O, True, scale, 0, 7, keys=rows, ub=2 * U)
