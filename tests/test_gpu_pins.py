"""Facts the pages fix, checked on the HIP path itself (GPU).

Several hold bitwise because of how the kernel computes: a masked score
contributes exp2(-inf) = 0 exactly and never enters the running max, and
every output column of an MFMA depends only on its own query's operand.
"""
import gc
import math
import sys

import numpy as np
import pytest

import exact_attention_123_amd as ea
import oracle
from gpu_util import TOL, max_err, run, to_device
from seeded_inputs import bf16_bits_to_f32, f32_to_bf16_bits, make_qkv

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


SHAPES = [  # (B, H, T, d, dtype)
    (1, 8, 2048, 64, "bf16"),
    (1, 4, 8192, 128, "bf16"),
    (1, 2, 1000, 128, "bf16"),
    (1, 1, 256, 64, "f32"),
    (1, 2, 300, 128, "f32"),
]


def _ids(s):
    return "x".join(map(str, s))


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_causal_row0_is_v0(shape):
    """Causal row 0 sees only key 0: O[0] = V[0] bitwise, LSE[0] = scale q0.k0.
    ("Why Attention Is Difficult to Optimize", The Attention Computation Flow)"""
    B, H, T, d, dt = shape
    say("row0", shape)
    x = make_qkv(B, H, T, d, dtype=dt, seed=77, qk_mult=4.0)
    scale = 1.0 / math.sqrt(d)
    O, L = run(x, True, scale)
    for b in range(B):
        for h in range(H):
            np.testing.assert_array_equal(O[b, h, 0], x.v64(b, h)[0])
            ref = scale * float(x.q64(b, h)[0] @ x.k64(b, h)[0])
            assert abs(L[b, h, 0] - ref) <= 1e-5 * max(1.0, abs(ref))


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_equal_scores_give_prefix_mean(shape, causal):
    """scale = 0 makes every permitted score equal: row i is the mean of the
    permitted V rows and LSE = ln(#permitted).  (Figure 4, uniform row)"""
    B, H, T, d, dt = shape
    say("equal scores", shape, causal)
    x = make_qkv(B, H, T, d, dtype=dt, seed=78)
    O, L = run(x, causal, 0.0)
    to, tl = TOL[dt]
    n = np.arange(1, T + 1, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            v = x.v64(b, h)
            if causal:
                ref_o = np.cumsum(v, axis=0) / n[:, None]
                ref_l = np.log(n)
            else:
                ref_o = np.tile(v.mean(axis=0), (T, 1))
                ref_l = np.full(T, math.log(T))
            assert max_err(O[b, h], ref_o) <= to
            assert max_err(L[b, h], ref_l) <= tl


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_values_one_gives_one(dt):
    """Rows of P sum to one: with V = 1 every output is 1.  fp32: the MFMA sum
    of p and the normaliser's sum of p round in different orders, so they
    agree to the fp32 parity bound, not exactly."""
    x = make_qkv(1, 2, 777, 128, dtype=dt, seed=79, qk_mult=2.0)
    one = np.ones_like(x.v) if dt == "f32" else np.full_like(x.v, 0x3F80)
    x.v = one
    for causal in (True, False):
        O, _ = run(x, causal)
        assert max_err(O, np.ones_like(O)) <= (TOL["f32"][0] if dt == "f32" else 8e-3)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_values_identity_exposes_p(dt, d):
    """With T = d and V = I the output rows are the probability rows P."""
    T = d
    x = make_qkv(1, 1, T, d, dtype=dt, seed=80)
    eye = np.eye(T, dtype=np.float32)[None, None]
    x.v = eye if dt == "f32" else f32_to_bf16_bits(eye)
    scale = 1.0 / math.sqrt(d)
    for causal in (True, False):
        O, _ = run(x, causal, scale)
        ref = oracle.attention_head(x.q64(0, 0), x.k64(0, 0), x.v64(0, 0),
                                    causal=causal, scale=scale)
        assert max_err(O[0, 0], ref["P"]) <= TOL[dt][0]
        if causal:
            assert np.all(O[0, 0][np.triu_indices(T, 1)] == 0.0)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_future_keys_do_not_matter(dt):
    """Changing K and V after row i0 leaves rows 0..i0 bitwise unchanged
    under the causal mask.  (The Attention Computation Flow; From a Score
    Tile to Probabilities)"""
    T, d, i0 = 700, 128, 333
    x = make_qkv(1, 2, T, d, dtype=dt, seed=81)
    O1, L1 = run(x, True)
    rng = np.random.Generator(np.random.PCG64(5))
    noise = (rng.standard_normal((1, 2, T - i0 - 1, d)) * 8).astype(np.float32)
    if dt == "bf16":
        noise = f32_to_bf16_bits(noise)
    x.k = x.k.copy()
    x.v = x.v.copy()
    x.k[:, :, i0 + 1:] = noise
    x.v[:, :, i0 + 1:] = noise[..., ::-1]
    O2, L2 = run(x, True)
    np.testing.assert_array_equal(O1[:, :, :i0 + 1], O2[:, :, :i0 + 1])
    np.testing.assert_array_equal(L1[:, :, :i0 + 1], L2[:, :, :i0 + 1])
    assert np.abs(O1[:, :, i0 + 1:] - O2[:, :, i0 + 1:]).max() > 1e-2


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_query_rows_independent(causal):
    """Changing query row r changes only row r of O and LSE, bitwise.
    (From a Score Tile to Probabilities: other query rows are not needed)"""
    T, d, r = 513, 128, 200
    x = make_qkv(1, 2, T, d, dtype="bf16", seed=82)
    O1, L1 = run(x, causal)
    x.q = x.q.copy()
    x.q[:, :, r] = f32_to_bf16_bits(np.full((1, 2, d), 1.5, dtype=np.float32))
    O2, L2 = run(x, causal)
    keep = np.arange(T) != r
    np.testing.assert_array_equal(O1[:, :, keep], O2[:, :, keep])
    np.testing.assert_array_equal(L1[:, :, keep], L2[:, :, keep])
    assert np.abs(O1[:, :, r] - O2[:, :, r]).max() > 1e-3


def test_run_to_run_deterministic():
    x = make_qkv(2, 4, 1500, 128, dtype="bf16", seed=83, qk_mult=4.0)
    for causal in (True, False):
        O1, L1 = run(x, causal)
        O2, L2 = run(x, causal)
        np.testing.assert_array_equal(O1, O2)
        np.testing.assert_array_equal(L1, L2)


@pytest.mark.parametrize("scale", [-0.2, 0.5, 1.0, 1e-4])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_other_scales(scale, dt):
    """Any finite multiplier, including negative ones (scale, then mask).

    The fp32 scores carry a rounding error proportional to their magnitude
    (|scale| * sqrt(d) standard deviations here), so the fp32 bound of 1e-5,
    stated for unit-spread scores, is widened by that factor."""
    x = make_qkv(1, 3, 300, 64, dtype=dt, seed=84)
    spread = max(1.0, abs(scale) * math.sqrt(64))
    tol_o = TOL[dt][0] * (spread if dt == "f32" else 1.0)
    tol_l = TOL[dt][1] * (spread if dt == "f32" else 1.0)
    for causal in (True, False):
        O, L = run(x, causal, scale)
        eo = el = 0.0
        for h in range(3):
            ref = oracle.attention_head(x.q64(0, h), x.k64(0, h), x.v64(0, h),
                                        causal=causal, scale=scale)
            eo = max(eo, max_err(O[0, h], ref["O"]))
            el = max(el, max_err(L[0, h], ref["LSE"]))
        assert eo <= tol_o and el <= tol_l, (eo, el)


def test_empty_and_stream_and_no_allocation():
    import torch
    # empty problem: nothing launched, no error
    q = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = ea.forward(q, q.clone(), q.clone(), causal=True)
    assert o.shape == q.shape and lse.shape == (1, 2, 0)
    # a non-default stream, with preallocated outputs and no device memory
    # allocated by the call
    x = make_qkv(1, 4, 1024, 128, dtype="bf16", seed=85)
    qd, kd, vd = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    out = torch.empty_like(qd)
    lse = torch.empty((1, 4, 1024), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ea.forward(qd, kd, vd, causal=True, out=out, lse=lse)  # warm-up
        out.zero_()
        lse.zero_()
    torch.cuda.synchronize()
    # the collector stays off while the allocation counts are compared, so
    # that no earlier test's tensors are freed in between
    gc.collect()
    gc.disable()
    try:
        free0, _ = torch.cuda.mem_get_info()
        alloc0 = torch.cuda.memory_allocated()
        with torch.cuda.stream(s):
            for _ in range(3):
                ea.forward(qd, kd, vd, causal=True, out=out, lse=lse)
        s.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        alloc1 = torch.cuda.memory_allocated()
    finally:
        gc.enable()
    assert alloc1 == alloc0
    assert free1 == free0
    O = out.float().cpu().numpy().astype(np.float64)
    eo = 0.0
    for h in range(4):
        ref = oracle.attention_head(x.q64(0, h), x.k64(0, h), x.v64(0, h), causal=True,
                                    scale=1 / math.sqrt(128))
        eo = max(eo, max_err(O[0, h], ref["O"]))
    assert eo <= TOL["bf16"][0]


def test_launches_follow_the_stream():
    """The binding launches on the stream it is given (stream=) or, without
    one, on the current stream: after work queued there before it.  Q is
    copied in on a side stream behind about 20 ms of matrix products; a launch
    on any other stream would run while Q is still zero (O would be the mean
    of the visible V rows)."""
    import torch
    x = make_qkv(1, 4, 1024, 128, dtype="bf16", seed=86)
    qd, kd, vd = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    s = torch.cuda.Stream()
    refs = [oracle.attention_head(x.q64(0, h), x.k64(0, h), x.v64(0, h), causal=True,
                                  scale=1 / math.sqrt(128))["O"] for h in range(4)]
    for how in ("stream=", "current stream"):
        say(f"[stream] {how}")
        q2 = torch.zeros_like(qd)
        out = torch.empty_like(qd)
        lse = torch.empty((1, 4, 1024), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            for _ in range(16):
                b = a @ a
            q2.copy_(qd)
            if how == "current stream":
                ea.forward(q2, kd, vd, causal=True, out=out, lse=lse)
        if how == "stream=":
            ea.forward(q2, kd, vd, causal=True, out=out, lse=lse, stream=s)
        s.synchronize()
        del b
        O = out.float().cpu().numpy().astype(np.float64)
        eo = max(max_err(O[0, h], refs[h]) for h in range(4))
        assert eo <= TOL["bf16"][0], (how, eo)
