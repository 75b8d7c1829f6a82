"""GPU parity on seeded random problems: each case draws its entry point
(bf16 forward, fp32 forward, grouped-query forward, decode), sizes, mask,
scale and score spread from its own PCG64 seed, so that the sizes fall on
every forward instance (row-chunk with 4 or 8 waves, 4-wave, 8-wave, fp32
row-chunk and 128-row) and on ragged lengths, and compares sampled rows
(tile boundaries, the ends, random rows) with the oracle at the stated
tolerances: bf16 2e-2 on O and 1e-3 on LSE, fp32 1e-5 on both.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from gpu_util import TOL, max_err, to_device
from oracle.decode import attention_decode_head
from seeded_inputs import bf16_bits_to_f32, make_decode, make_qkv

pytestmark = pytest.mark.gpu

CASES = 48


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def sampled_rows(rng, T, n):
    fixed = [0, 1, 31, 32, 33, 63, 64, 127, 128, 255, 256, T // 2, T - 33, T - 32, T - 2, T - 1]
    r = np.concatenate([fixed, rng.integers(0, T, size=n)])
    return np.unique(np.clip(r, 0, T - 1))


def to64(t, dt):
    if dt == "bf16":
        bits = t.view(__import__("torch").int16).cpu().numpy().view(np.uint16)
        return bf16_bits_to_f32(bits).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("case", range(CASES))
def test_random_problem(case):
    import torch

    import exact_attention_123_amd as ea
    rng = np.random.Generator(np.random.PCG64(90000 + case))
    kind = str(rng.choice(["fwd", "fwd", "fwd", "f32", "gqa", "decode"]))
    d = int(rng.choice([64, 128]))
    causal = bool(rng.integers(2))
    if kind == "decode":
        Hkv = int(rng.choice([1, 2, 8]))
        G = int(rng.choice([1, 4, 8]))
        H, B = Hkv * G, int(rng.choice([1, 2]))
        Tq = int(rng.integers(1, min(8, 256 // G) + 1))
        Tk = max(Tq, int(np.exp(rng.uniform(0, np.log(20000)))))
        cap = Tk + int(rng.integers(0, 65))
        scale = 1.0 / math.sqrt(d)
        say(f"case {case}: decode B={B} H={H} Hkv={Hkv} Tq={Tq} Tk={Tk} cap={cap} d={d} "
            f"causal={causal}")
        x = make_decode(B, H, Hkv, Tq, Tk, d, seed=91000 + case, Tk_cap=cap)
        q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
        o, lse = ea.decode(q, k, v, Tk=Tk, causal=causal, scale=scale)
        torch.cuda.synchronize()
        O, L = to64(o, "bf16"), lse.cpu().numpy().astype(np.float64)
        eo = el = 0.0
        for b in range(B):
            for h in rng.choice(H, size=min(3, H), replace=False):
                ref = attention_decode_head(x.q64(b, h), x.k64(b, h // G)[:Tk],
                                            x.v64(b, h // G)[:Tk], causal=causal, scale=scale)
                eo = max(eo, max_err(O[b, h], ref["O"]))
                el = max(el, max_err(L[b, h], ref["LSE"]))
        to, tl = TOL["bf16"]
    else:
        dt = "f32" if kind == "f32" else "bf16"
        T = int(np.exp(rng.uniform(0, np.log(2000 if dt == "f32" else 6000))))
        B = int(rng.choice([1, 2]))
        if kind == "gqa":
            Hkv = int(rng.choice([1, 2, 4]))
            H = Hkv * int(rng.choice([2, 4]))
        else:
            H = int(rng.choice([1, 2, 3, 8, 16]))
            Hkv = H
        mult = float(rng.choice([1.0, 4.0])) if dt == "bf16" else 1.0
        # any finite scale (0 and negative included) for bf16; the fp32
        # bound assumes scores of unit spread
        scale = (float(rng.choice([1.0, 1.0, 0.5, -0.7, 0.0])) if dt == "bf16" else 1.0) / math.sqrt(d)
        name = (ea.fwd_f32_kernel_name_for(B, H, T, d, causal) if dt == "f32"
                else ea.fwd_kernel_name_for(B, H, T, d, causal))
        say(f"case {case}: {kind} B={B} H={H} Hkv={Hkv} T={T} d={d} causal={causal} "
            f"scale={scale:.4f} qk x{mult}: {name}")
        x = make_qkv(B, H, T, d, dtype=dt, seed=92000 + case, qk_mult=mult, H_kv=Hkv)
        q, k, v = (to_device(a, dt) for a in (x.q, x.k, x.v))
        o, lse = ea.forward(q, k, v, causal=causal, scale=scale)
        torch.cuda.synchronize()
        O, L = to64(o, dt), lse.cpu().numpy().astype(np.float64)
        G = H // Hkv
        heads = [(b, h) for b in range(B) for h in range(H)]
        eo = el = 0.0
        for i in rng.choice(len(heads), size=min(3, len(heads)), replace=False):
            b, h = heads[i]
            r = sampled_rows(rng, T, 24)
            ref = oracle.attention_head(x.q64(b, h), x.k64(b, h // G), x.v64(b, h // G),
                                        causal=causal, scale=scale, rows=r)
            eo = max(eo, max_err(O[b, h][r], ref["O"]))
            el = max(el, max_err(L[b, h][r], ref["LSE"]))
        to, tl = TOL[dt]
    assert eo <= to and el <= tl, (eo, el)


LARGE_CASES = 12


@pytest.mark.parametrize("case", range(LARGE_CASES))
def test_random_large_forward(case):
    """Seeded random bf16 forward problems on grids that fill the GPU (the
    4-wave and 8-wave instances, which the draws above reach only twice):
    B in {1, 2, 4}, 4 to 32 key/value heads with G = 1, 2 or 4 query heads
    each, T from 512 to 8192 (at most 2^27 elements per tensor), both masks,
    the scales 1, 0.5, -0.7 and 0 (over sqrt(d)) in turn, Q and K times 1, 2
    or 4; sampled rows of three heads against the oracle at the bf16
    tolerances."""
    import torch

    import exact_attention_123_amd as ea
    rng = np.random.Generator(np.random.PCG64(93000 + case))
    B = int(rng.choice([1, 2, 4]))
    Hkv = int(rng.choice([4, 8, 16, 32]))
    G = int(rng.choice([1, 2, 4]))
    H = Hkv * G
    d = int(rng.choice([64, 128]))
    T = int(np.exp(rng.uniform(np.log(512), np.log(8192))))
    T = min(T, (1 << 27) // (B * H * d))
    causal = bool(rng.integers(2))
    scale = (1.0, 0.5, -0.7, 0.0)[case % 4] / math.sqrt(d)
    mult = float(rng.choice([1.0, 2.0, 4.0]))
    name = ea.fwd_kernel_name_for(B, H, T, d, causal)
    say(f"case {case}: fwd B={B} H={H} Hkv={Hkv} T={T} d={d} causal={causal} "
        f"scale={scale:.4f} qk x{mult}: {name}")
    x = make_qkv(B, H, T, d, seed=94000 + case, qk_mult=mult, H_kv=Hkv)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    o, lse = ea.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(H)]
    eo = el = 0.0
    for i in rng.choice(len(heads), size=3, replace=False):
        b, h = heads[i]
        r = sampled_rows(rng, T, 24)
        got_o = to64(o[b, h][torch.from_numpy(r).cuda()], "bf16")
        got_l = lse[b, h][torch.from_numpy(r).cuda()].cpu().numpy().astype(np.float64)
        ref = oracle.attention_head(x.q64(b, h), x.k64(b, h // G), x.v64(b, h // G),
                                    causal=causal, scale=scale, rows=r)
        eo = max(eo, max_err(got_o, ref["O"]))
        el = max(el, max_err(got_l, ref["LSE"]))
    to, tl = TOL["bf16"]
    assert eo <= to and el <= tl, (eo, el)
