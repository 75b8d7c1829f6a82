"""GPU parity of the decode path (attn_decode) against the float64 decode
oracle on the same seeded inputs.

Tolerances as for the bf16 forward: max abs error 2e-2 on O and 1e-3 on LSE.
Cache rows past the valid length hold NaN bit patterns, so any read beyond
Tk shows up as a non-finite output.  Shapes cover one and several new
queries, grouped key/value heads (G = 1, 4, 8), more query rows per
key/value head than one workgroup takes (256 rows, and thousands: a prefill
in chunks appended to a cache), caches shorter than one block, ragged
lengths, a single split and many splits (the cross-split merge), and the
full decode workloads on sampled heads.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from gpu_util import to_device
from seeded_inputs import DECODE_WORKLOADS, bf16_bits_to_f32, make_decode

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_decode(x, causal, scale, Tk):
    import torch

    import exact_attention_123_amd as ea
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    o, lse = ea.decode(q, k, v, Tk=Tk, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(x, O, L, causal, scale, Tk, heads=None):
    B, H, Tq, d = x.q.shape
    Hkv = x.k.shape[1]
    G = H // Hkv
    assert np.isfinite(O).all() and np.isfinite(L).all()
    eo = el = 0.0
    for (b, h) in heads or [(b, h) for b in range(B) for h in range(H)]:
        g = h // G
        ref = oracle.attention_decode_head(
            bf16_bits_to_f32(x.q[b, h]).astype(np.float64),
            bf16_bits_to_f32(x.k[b, g, :Tk]).astype(np.float64),
            bf16_bits_to_f32(x.v[b, g, :Tk]).astype(np.float64), causal=causal, scale=scale)
        eo = max(eo, float(np.abs(O[b, h] - ref["O"]).max()))
        el = max(el, float(np.abs(L[b, h] - ref["LSE"]).max()))
    assert eo <= 2e-2, eo
    assert el <= 1e-3, el
    return eo, el


CASES = []
for Tq, H, Hkv in ((1, 8, 8), (1, 32, 8), (1, 8, 1), (2, 8, 2), (4, 8, 8), (4, 16, 2),
                   (32, 4, 4), (8, 32, 4), (5, 16, 1), (64, 2, 2), (32, 32, 4)):
    for Tk in (1, 7, 33, 100, 1000, 5000):
        if Tk >= Tq:
            CASES.append((Tq, H, Hkv, Tk))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("Tq,H,Hkv,Tk", CASES)
def test_decode_shapes(Tq, H, Hkv, Tk, causal, d):
    say(f"[decode] Tq={Tq} H={H} Hkv={Hkv} Tk={Tk} causal={causal} d={d}")
    B = 2
    scale = 1.0 / math.sqrt(d)
    x = make_decode(B, H, Hkv, Tq, Tk, d, seed=9000 + Tq + H + Hkv + Tk + d, Tk_cap=Tk + 37,
                    qk_mult=2.0)
    O, L = run_decode(x, causal, scale, Tk)
    check(x, O, L, causal, scale, Tk)


# Many new queries appended to a cache (a prefill in chunks): row chunks
# by the hundred, each reading only the keys its rows see under the causal
# mask; Tq = Tk is the square forward.
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("B,H,Hkv,Tq,Tk,d", [(1, 8, 2, 300, 1500, 128), (1, 4, 4, 1000, 1000, 64),
                                            (2, 2, 1, 777, 2049, 64)])
def test_decode_chunked_prefill(B, H, Hkv, Tq, Tk, d, causal):
    say(f"[decode prefill chunk] B={B} H={H} Hkv={Hkv} Tq={Tq} Tk={Tk} d={d} causal={causal}")
    scale = 1.0 / math.sqrt(d)
    x = make_decode(B, H, Hkv, Tq, Tk, d, seed=9500 + Tq + Tk + d, Tk_cap=Tk + 5, qk_mult=2.0)
    O, L = run_decode(x, causal, scale, Tk)
    check(x, O, L, causal, scale, Tk)


# Many new queries on a grid of at least one 128-row workgroup per CU:
# the forward kernel runs them over the cache (query i at key position
# Tk - Tq + i); sampled heads against the oracle.
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("B,H,Hkv,Tq,Tk,d", [(2, 32, 8, 520, 1700, 128), (4, 32, 8, 300, 900, 64),
                                            (1, 64, 64, 513, 513, 128)])
def test_decode_over_forward_kernel(B, H, Hkv, Tq, Tk, d, causal):
    import exact_attention_123_amd as ea
    say(f"[decode on the forward kernel] B={B} H={H} Hkv={Hkv} Tq={Tq} Tk={Tk} d={d} "
        f"causal={causal}")
    assert B * H * ((Tq + 127) // 128) >= 256 and Tq * (H // Hkv) >= 256
    assert ea.decode_splits(B, H, Hkv, Tq, Tk) == 1
    assert ea.decode_workspace_bytes(B, H, Hkv, Tq, Tk, d) == 0
    scale = 1.0 / math.sqrt(d)
    x = make_decode(B, H, Hkv, Tq, Tk, d, seed=9600 + Tq + Tk + d, Tk_cap=Tk + 9, qk_mult=2.0)
    O, L = run_decode(x, causal, scale, Tk)
    heads = [(0, 0), (0, H - 1), (B - 1, H // 2), (B - 1, 1)]
    check(x, O, L, causal, scale, Tk, heads=heads)
    # every row finite (rows past the valid cache hold NaN bit patterns)
    assert np.isfinite(O).all()


@pytest.mark.parametrize("scale", [-0.25, 0.0, 1.0])
def test_decode_other_scales(scale):
    say(f"[decode scale] {scale}")
    x = make_decode(1, 8, 2, 3, 3000, 128, seed=9100)
    for causal in (True, False):
        O, L = run_decode(x, causal, scale, 3000)
        check(x, O, L, causal, scale, 3000)


def test_decode_many_splits():
    import exact_attention_123_amd as ea
    say("[decode splits] B=1 H=8 Hkv=1 Tq=2 Tk=40000")
    B, H, Hkv, Tq, Tk, d = 1, 8, 1, 2, 40000, 128
    assert ea.decode_splits(B, H, Hkv, Tq, Tk) >= 8
    x = make_decode(B, H, Hkv, Tq, Tk, d, seed=9200, qk_mult=4.0)
    scale = 1.0 / math.sqrt(d)
    for causal in (True, False):
        O, L = run_decode(x, causal, scale, Tk)
        check(x, O, L, causal, scale, Tk)


@pytest.mark.parametrize("Tk,nsplit,d", [(262144, 64, 128), (266240, 65, 64),
                                          (326680, 80, 128)])
def test_decode_splits_past_one_wave(Tk, nsplit, d):
    """More key splits than a wave has lanes: the merge of the splits takes
    their log-sum-exps 64 at a time (64, 65 and 80 splits; ragged length)."""
    import exact_attention_123_amd as ea
    B, H, Hkv, Tq = 1, 4, 1, 2
    assert ea.decode_splits(B, H, Hkv, Tq, Tk) == nsplit
    say(f"[decode {nsplit} splits] B={B} H={H} Hkv={Hkv} Tq={Tq} Tk={Tk} d={d}")
    x = make_decode(B, H, Hkv, Tq, Tk, d, seed=9250 + nsplit, qk_mult=4.0)
    scale = 1.0 / math.sqrt(d)
    for causal in (True, False):
        O, L = run_decode(x, causal, scale, Tk)
        check(x, O, L, causal, scale, Tk)


def test_decode_matches_square_forward_rows():
    """The GPU decode of the last Tq positions against the GPU forward over
    the full square problem (its last Tq rows): the two paths agree within
    the bf16 tolerance."""
    import torch

    import exact_attention_123_amd as ea
    say("[decode vs forward]")
    B, H, T, d, Tq = 2, 8, 777, 128, 4
    rng = np.random.Generator(np.random.PCG64(9300))
    q, k, v = (torch.from_numpy(rng.standard_normal((B, H, T, d), dtype=np.float32))
               .cuda().to(torch.bfloat16) for _ in range(3))
    o_full, l_full = ea.forward(q, k, v, causal=True)
    o_dec, l_dec = ea.decode(q[:, :, T - Tq:].contiguous(), k, v, causal=True)
    torch.cuda.synchronize()
    assert (o_full[:, :, T - Tq:].float() - o_dec.float()).abs().max().item() <= 2e-2
    assert (l_full[:, :, T - Tq:] - l_dec).abs().max().item() <= 1e-3


def test_decode_workspace_checked():
    import torch

    import exact_attention_123_amd as ea
    B, H, Hkv, Tq, Tk, d = 1, 8, 8, 1, 8192, 128
    need = ea.decode_workspace_bytes(B, H, Hkv, Tq, Tk, d)
    assert need > 0
    x = make_decode(B, H, Hkv, Tq, Tk, d, seed=9400)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    small = torch.empty(need - 16, dtype=torch.uint8, device=q.device)
    with pytest.raises(ea.AttnError) as e:
        ea.decode(q, k, v, ws=small)
    assert e.value.code == 9
    ok = torch.empty(need, dtype=torch.uint8, device=q.device)
    o, _ = ea.decode(q, k, v, ws=ok)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("name", sorted(DECODE_WORKLOADS))
def test_decode_full_size(name):
    w = DECODE_WORKLOADS[name]
    say(f"[decode full size] {name}")
    x = make_decode(w["B"], w["H"], w["H_kv"], w["Tq"], w["Tk"], w["d"], seed=w["seed"])
    scale = 1.0 / math.sqrt(w["d"])
    O, L = run_decode(x, w["causal"], scale, w["Tk"])
    B, H = w["B"], w["H"]
    heads = [(0, 0), (0, 3), (0, 4), (B - 1, H - 1), (B // 2, H // 2)]
    check(x, O, L, w["causal"], scale, w["Tk"], heads=heads)


def test_decode_rejects_wrong_buffers():
    """Caller-supplied out, lse and ws of the wrong shape, dtype or device
    raise ValueError before any launch."""
    import torch

    import exact_attention_123_amd as ea
    B, H, Hkv, Tq, Tk, d = 1, 8, 2, 1, 20000, 128
    x = make_decode(B, H, Hkv, Tq, Tk, d, seed=8800)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    dev = q.device
    with pytest.raises(ValueError, match="out"):
        ea.decode(q, k, v, out=torch.empty((B, H, Tq + 1, d), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError, match="out"):
        ea.decode(q, k, v, out=torch.empty((B, H, Tq, d), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError, match="lse"):
        ea.decode(q, k, v, lse=torch.empty((B, H), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError, match="lse"):
        ea.decode(q, k, v, lse=torch.empty((B, H, Tq), dtype=torch.float32))
    with pytest.raises(ValueError, match="ws"):
        ea.decode(q, k, v, ws=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ea.AttnError):  # too small: the library's own check
        ea.decode(q, k, v, ws=torch.empty(16, dtype=torch.uint8, device=dev))
