"""GPU runs of the kernel instances that the other GPU tests do not launch.

A kernel trace of the whole GPU suite lists, per template instance of the
library, whether any test launched it.  The cases here launch the rest,
each first asserting by name which instance its sizes select:

  - the 8-wave dK/dV kernel with the unfolded exponent: |scale| < 2^-32
    (zero, 1e-12) on grids with at least as many 256-key blocks as CUs
    (twice as many, and T > 4096, under the causal mask),
    both masks, d in {64, 128}; gradients against the float64 backward
    oracle under the per-element bound of the backward tests;
  - the row-chunk forward with 8 waves at d = 128 without a mask (grids
    below the CU count with T >= 4096); output against the float64 oracle
    at the bf16 tolerances;
  - the row-chunk forward with 4 waves at d = 128 (its software-pipelined
    block loop) for every count of 32-key blocks per wave from 0 to 9,
    both masks, every row against the float64 oracle;
  - the matrix-core probe (both MFMA shapes): the sum of a wave's sink
    values equals, in closed form, the number of trips times the sum of
    all outputs of the wave's MFMAs, and the sum of all outputs of one MFMA
    is sum_k (column sum of A)[k] (row sum of B)[k].
"""
import math
import sys

import numpy as np
import pytest

import oracle
from gpu_util import to_device
from seeded_inputs import bf16_bits_to_f32, make_dout, make_qkv
from test_gpu_bwd import U, check_head, gpu_backward, sampled

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


# ---------------------------------------------------------------------------
# dK/dV, 8 waves, unfolded exponent
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("scale", [0.0, 1e-12], ids=["s0", "s1e-12"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("d", [64, 128])
def test_dkdv_w8_unfolded(d, causal, scale):
    import exact_attention_123_amd as ea
    # 256 key blocks of 256 (ragged end); under the causal mask 576 of a
    # sequence longer than 4096, since shorter or smaller causal grids take
    # the paired instance
    B, H, T = (1, 32, 4500) if causal else (1, 32, 2000)
    assert B * H * ((T + 255) // 256) >= (2 if causal else 1) * cus()
    name = ea.bwd_kernel_name_for(B, H, H, T, d, causal, 1)
    assert name.endswith("_bk256_bq64_w8"), name
    say(f"[dkdv w8 unfolded] {name} scale={scale}")
    x = make_qkv(B, H, T, d, seed=9300 + d + (1 if causal else 0), qk_mult=2.0)
    do = make_dout(B, H, T, d, seed=9310 + d)
    res = gpu_backward(x, do, causal, scale)
    for h in (0, 13, H - 1):
        check_head(x, do, 0, h, res, causal, scale, rows=sampled(T, 40 + h),
                   keys=sampled(T, 50 + h), ub=2 * U)


# ---------------------------------------------------------------------------
# Row-chunk forward, 8 waves, d = 128, no mask
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [4096, 4500])
def test_rows_w8_d128_full(T):
    import torch

    import exact_attention_123_amd as ea
    B, H, d = 1, 2, 128
    name = ea.fwd_kernel_name_for(B, H, T, d, False)
    assert name == "attn_fwd_rows_bf16_d128_full_br32_bc32_w8", name
    say(f"[rows w8] {name} T={T}")
    x = make_qkv(B, H, T, d, dtype="bf16", seed=9400 + T, qk_mult=2.0)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    scale = 1.0 / math.sqrt(d)
    o, lse = ea.forward(q, k, v, causal=False, scale=scale)
    torch.cuda.synchronize()
    O = o.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    rows = np.unique(np.r_[np.arange(0, 64), np.arange(T - 64, T),
                           np.random.Generator(np.random.PCG64(T)).choice(T, 256, replace=False)])
    for h in range(H):
        ref = oracle.attention_head(x.q64(0, h), x.k64(0, h), x.v64(0, h), causal=False,
                                    scale=scale, rows=rows)
        eo = float(np.abs(O[0, h, rows] - ref["O"]).max())
        el = float(np.abs(L[0, h, rows] - ref["LSE"]).max())
        say(f"    head {h}: max|O err|={eo:.3e} max|LSE err|={el:.3e}")
        assert eo <= 2e-2 and el <= 1e-3


# ---------------------------------------------------------------------------
# Row-chunk forward, 4 waves, d = 128 (software-pipelined block loop)
# ---------------------------------------------------------------------------

# Wave w of a chunk takes the chunk's 32-key blocks w, w + 4, ...: these
# lengths give the waves 0 .. 9 blocks each (ragged last blocks included).
ROWS_W4_T = [1, 31, 32, 33, 64, 96, 127, 128, 129, 160, 161, 255, 256, 300, 640, 1000, 1100]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("T", ROWS_W4_T)
def test_rows_w4_d128_block_counts(T, causal):
    import torch

    import exact_attention_123_amd as ea
    B, H, d = 1, 2, 128
    name = ea.fwd_kernel_name_for(B, H, T, d, causal)
    mask = "causal" if causal else "full"
    assert name == f"attn_fwd_rows_bf16_d128_{mask}_br32_bc32_w4", name
    say(f"[rows w4 d128] {name} T={T}")
    x = make_qkv(B, H, T, d, dtype="bf16", seed=9450 + T, qk_mult=2.0)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    scale = 1.0 / math.sqrt(d)
    o, lse = ea.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    O = o.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    for h in range(H):
        ref = oracle.attention_head(x.q64(0, h), x.k64(0, h), x.v64(0, h), causal=causal,
                                    scale=scale)
        eo = float(np.abs(O[0, h] - ref["O"]).max())
        el = float(np.abs(L[0, h] - ref["LSE"]).max())
        assert eo <= 2e-2 and el <= 1e-3, (h, eo, el)


# ---------------------------------------------------------------------------
# Matrix-core probe
# ---------------------------------------------------------------------------

M32 = 0xFFFFFFFF


def _mix(x):
    x &= M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & M32
    x ^= x >> 16
    return x


def _bf16(bits):
    return float(bf16_bits_to_f32(np.array([bits], dtype=np.uint16))[0])


def _operand(seed):
    """The eight bf16 values of the probe's operand(seed), as stated in its
    source: per 32-bit word i, x = mix(4 seed + i); each half keeps x's sign
    and low mantissa bits and takes exponent 126 + (byte) mod 3."""
    seed, out = int(seed), []
    for i in range(4):
        x = _mix((seed * 4 + i) & M32)
        lo = (x & 0x807F) | ((126 + ((x >> 8) & 0xFFFFFF) % 3) << 7)
        hi = ((x >> 16) & 0x807F) | ((126 + (x >> 24) % 3) << 7)
        out += [_bf16(lo), _bf16(hi)]
    return np.array(out)


def _wave_total(shape, wg, wave, iters):
    """Expected sum of the 64 sink values of one wave, and the sum of the
    magnitudes of its terms (for the rounding bound)."""
    groups = 2 if shape == 0 else 4          # k groups of 8 per MFMA
    lanes = 64 // groups
    gids = wg * 256 + wave * 64 + np.arange(64)
    a = np.array([[_operand(g * 8 + i) for i in range(4)] for g in gids])      # [64][4][8]
    b = np.array([[_operand(g * 8 + 4 + i) for i in range(4)] for g in gids])
    # column sums of A and row sums of B by k group: lane l holds k = 8 (l // lanes) + e
    ca = a.reshape(groups, lanes, 4, 8).sum(1)   # [group][operand][e]
    rb = b.reshape(groups, lanes, 4, 8).sum(1)
    pairs = ([((i + x) & 3, (i + 2 * x) & 3) for i in range(4) for x in range(4)] if shape == 0
             else [((i + x) & 3, (i + 3 * x) & 3) for i in range(4) for x in range(8)])
    tot = sum(float((ca[:, ia] * rb[:, ib]).sum()) for ia, ib in pairs)
    aa = np.abs(a).reshape(groups, lanes, 4, 8).sum(1)
    ab = np.abs(b).reshape(groups, lanes, 4, 8).sum(1)
    mag = sum(float((aa[:, ia] * ab[:, ib]).sum()) for ia, ib in pairs)
    return iters * tot, iters * mag


@pytest.mark.parametrize("shape", [0, 1])
def test_probe_mfma(shape):
    import torch

    import exact_attention_123_amd as ea
    lib = ea.load_library()
    wg, iters = 2, 3
    sink = torch.full((wg * 256,), float("nan"), dtype=torch.float32, device="cuda")
    st = lib.attn_probe_mfma(shape, wg, iters, sink.data_ptr(), None)
    assert st == 0, st
    torch.cuda.synchronize()
    s = sink.cpu().numpy().astype(np.float64)
    assert np.isfinite(s).all()
    flops = lib.attn_probe_mfma_flops(shape, wg, iters)
    per_mfma = 2 * 32 * 32 * 16 if shape == 0 else 2 * 16 * 16 * 32
    assert flops == (16 if shape == 0 else 32) * per_mfma * iters * wg * 4
    for w in range(wg * 4):
        want, mag = _wave_total(shape, w // 4, w % 4, iters)
        got = float(s[w * 64:(w + 1) * 64].sum())
        say(f"[probe {shape}] wave {w}: got {got:.6g} want {want:.6g}")
        assert abs(got - want) <= 1e-5 * mag + 1e-3, (w, got, want)
