"""GPU parity: the HIP path against the float64 oracle on the same seeded
inputs, element by element.

Tolerances (max abs over every compared element): fp32 path 1e-5 on O and
on LSE; bf16 path 2e-2 on O and 1e-3 on LSE.  Small and ragged shapes are
compared in full; the large workloads are compared on every row of some
heads and on sampled rows (tile boundaries, the ragged end and seeded random
rows) of every head.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from gpu_util import TOL, max_err, run
from seeded_inputs import WORKLOADS, make_qkv, make_workload, sample_rows

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def boundary_rows(T, n_random, seed):
    fixed = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257,
             T // 2, T - 65, T - 64, T - 63, T - 2, T - 1]
    rng = np.random.Generator(np.random.PCG64(seed))
    rnd = rng.choice(T, size=min(n_random, T), replace=False)
    return np.unique(np.clip(np.concatenate([fixed, rnd]), 0, T - 1))


def compare(x, O, L, causal, scale, rows_for=None, full_heads=()):
    """Max abs errors of O and LSE against the oracle over the chosen rows."""
    B, H, T, d = x.shape
    eo = el = 0.0
    for b in range(B):
        for h in range(H):
            rows = None if (b, h) in full_heads or rows_for is None else rows_for(b, h)
            ref = oracle.attention_head(x.q64(b, h), x.k64(b, h), x.v64(b, h),
                                        causal=causal, scale=scale, rows=rows)
            r = ref["rows"]
            eo = max(eo, max_err(O[b, h][r], ref["O"]))
            el = max(el, max_err(L[b, h][r], ref["LSE"]))
    return eo, el


# ---------------------------------------------------------------------------
# Small and ragged shapes, full comparison
# ---------------------------------------------------------------------------

EDGE_T = [1, 2, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 255, 257, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("T", EDGE_T)
def test_ragged_shapes(T, causal, d, dtype):
    B, H = (2, 3) if T <= 129 else (1, 2)
    seed = 1000 + T * 4 + d + (1 if causal else 0)
    say(f"ragged T={T} d={d} {dtype} causal={causal} seed={seed}")
    x = make_qkv(B, H, T, d, dtype=dtype, seed=seed)
    scale = 1.0 / math.sqrt(d)
    O, L = run(x, causal, scale)
    eo, el = compare(x, O, L, causal, scale)
    to, tl = TOL[dtype]
    assert eo <= to and el <= tl, (eo, el)


# Ragged lengths on grids of at least one 8-wave workgroup per CU (the small
# shapes above run the row-chunk kernel), and the instance choice itself.
@pytest.mark.parametrize("B,H,T,d,causal", [(2, 64, 1000, 128, True), (2, 64, 1000, 128, False),
                                            (1, 128, 777, 64, True)])
def test_ragged_large_grid(B, H, T, d, causal):
    import exact_attention_123_amd as ea
    name = ea.fwd_kernel_name_for(B, H, T, d, causal)
    say(f"ragged large grid B={B} H={H} T={T} d={d} causal={causal}: {name}")
    assert name is not None and name.endswith("_w8")
    x = make_qkv(B, H, T, d, dtype="bf16", seed=1500 + T + d + int(causal))
    scale = 1.0 / math.sqrt(d)
    O, L = run(x, causal, scale)
    eo, el = compare(x, O, L, causal, scale)
    to, tl = TOL["bf16"]
    assert eo <= to and el <= tl, (eo, el)


# Shapes between the two small-grid rules run the 4-wave instance: ragged
# and aligned lengths, both masks.
@pytest.mark.parametrize("B,H,T,d,causal", [(1, 8, 4000, 128, True), (1, 8, 4096, 128, False),
                                            (2, 4, 3000, 128, True)])
def test_four_wave_instance(B, H, T, d, causal):
    import exact_attention_123_amd as ea
    name = ea.fwd_kernel_name_for(B, H, T, d, causal)
    say(f"4-wave instance B={B} H={H} T={T} d={d} causal={causal}: {name}")
    assert name is not None and name.endswith("_br128_bc64_w4")
    seed = 1700 + T + d + int(causal)
    x = make_qkv(B, H, T, d, dtype="bf16", seed=seed)
    scale = 1.0 / math.sqrt(d)
    O, L = run(x, causal, scale)
    eo, el = compare(x, O, L, causal, scale,
                     rows_for=lambda b, h: boundary_rows(T, 64, seed + 31 * b + h),
                     full_heads={(0, 0), (B - 1, H - 1)})
    to, tl = TOL["bf16"]
    assert eo <= to and el <= tl, (eo, el)


# Long sequences on grids too small for 256-row workgroups run the
# row-chunk kernel with 8 waves splitting the keys.
@pytest.mark.parametrize("B,H,T,d,causal", [(1, 1, 16384, 128, True), (1, 2, 4100, 64, False),
                                            (1, 2, 4100, 64, True)])
def test_row_chunk_eight_waves(B, H, T, d, causal):
    import exact_attention_123_amd as ea
    name = ea.fwd_kernel_name_for(B, H, T, d, causal)
    say(f"row-chunk 8 waves B={B} H={H} T={T} d={d} causal={causal}: {name}")
    assert name is not None and name.startswith("attn_fwd_rows_") and name.endswith("_w8")
    seed = 1800 + T + d + int(causal)
    x = make_qkv(B, H, T, d, dtype="bf16", seed=seed)
    scale = 1.0 / math.sqrt(d)
    O, L = run(x, causal, scale)
    eo, el = compare(x, O, L, causal, scale,
                     rows_for=lambda b, h: boundary_rows(T, 96, seed + 31 * b + h))
    to, tl = TOL["bf16"]
    assert eo <= to and el <= tl, (eo, el)


# fp32: small grids at d = 64 run the fp32 row-chunk kernel (the ragged
# shapes above); here the 128-row fp32 kernel on a grid that fills the GPU,
# and the instance choice.
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_f32_large_grid(causal):
    import exact_attention_123_amd as ea
    B, H, T, d = 2, 64, 1000, 64
    name = ea.fwd_f32_kernel_name_for(B, H, T, d, causal)
    say(f"f32 large grid B={B} H={H} T={T} d={d} causal={causal}: {name}")
    assert name == ea.kernel_name(True, d, causal)
    seed = 1900 + int(causal)
    x = make_qkv(B, H, T, d, dtype="f32", seed=seed)
    scale = 1.0 / math.sqrt(d)
    O, L = run(x, causal, scale)
    eo, el = compare(x, O, L, causal, scale,
                     rows_for=lambda b, h: boundary_rows(T, 16, seed + 31 * b + h),
                     full_heads={(0, 0)})
    to, tl = TOL["f32"]
    assert eo <= to and el <= tl, (eo, el)


def test_f32_instance_choice():
    import exact_attention_123_amd as ea
    assert (ea.fwd_f32_kernel_name_for(1, 1, 256, 64, True)
            == "attn_fwd_f32_rows_d64_causal_br32_bc32_w4")
    assert (ea.fwd_f32_kernel_name_for(1, 1, 256, 64, False)
            == "attn_fwd_f32_rows_d64_full_br32_bc32_w4")
    assert ea.fwd_f32_kernel_name_for(1, 1, 256, 128, True) == ea.kernel_name(True, 128, True)
    assert ea.fwd_f32_kernel_name_for(0, 1, 256, 64, True) is None


def test_small_grid_uses_row_chunks():
    """Problems too small to fill the GPU with 256-row workgroups take the
    row-chunk kernel when the 4-wave grid (in d = 64 units) fits the CUs
    once, else the 4-wave kernel."""
    import exact_attention_123_amd as ea
    assert (ea.fwd_kernel_name_for(1, 8, 2048, 64, True)
            == "attn_fwd_rows_bf16_d64_causal_br32_bc32_w4")
    assert (ea.fwd_kernel_name_for(1, 1, 16384, 128, True)
            == "attn_fwd_rows_bf16_d128_causal_br32_bc32_w8")
    assert (ea.fwd_kernel_name_for(1, 2, 1000, 128, False)
            == "attn_fwd_rows_bf16_d128_full_br32_bc32_w4")
    assert (ea.fwd_kernel_name_for(1, 8, 4096, 128, False)
            == "attn_fwd_bf16_d128_full_br128_bc64_w4")
    assert ea.fwd_kernel_name_for(1, 32, 8192, 128, True) == ea.kernel_name(False, 128, True)
    assert ea.fwd_kernel_name_for(0, 8, 2048, 64, True) is None


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

def _workload_case(name, causal, rows_for, full_heads):
    w = WORKLOADS[name]
    say(f"workload {name} causal={causal}: generating inputs")
    x = make_workload(name)
    scale = 1.0 / math.sqrt(w["d"])
    O, L = run(x, causal, scale)
    say(f"workload {name} causal={causal}: GPU done, comparing with the oracle")
    eo, el = compare(x, O, L, causal, scale, rows_for=rows_for, full_heads=full_heads)
    say(f"workload {name} causal={causal}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    to, tl = TOL[w["dtype"]]
    assert eo <= to and el <= tl, (eo, el)


def test_f32_b1h1_t256_d64_causal():
    _workload_case("f32_b1h1_t256_d64_causal", True, None, ())


def test_bf16_b1h8_t2048_d64_causal():
    _workload_case("bf16_b1h8_t2048_d64_causal", True, None, ())


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_bf16_b4h16_t4096_d128(causal):
    T = 4096
    _workload_case("bf16_b4h16_t4096_d128", causal,
                   lambda b, h: boundary_rows(T, 48, 31 + 16 * b + h),
                   full_heads=((0, 0), (3, 15)))


def test_bf16_b1h32_t8192_d128_causal_qk4():
    T = 8192
    _workload_case("bf16_b1h32_t8192_d128_causal_qk4", True,
                   lambda b, h: boundary_rows(T, 64, 41 + h),
                   full_heads=((0, 0), (0, 31)))


def test_bf16_b1h8_t65536_d128_causal():
    w = WORKLOADS["bf16_b1h8_t65536_d128_causal"]
    rows = sample_rows(w["T"], w["sample_rows"], w["row_seed"], w["B"] * w["H"])
    _workload_case("bf16_b1h8_t65536_d128_causal", True,
                   lambda b, h: rows[b * w["H"] + h], full_heads=())
