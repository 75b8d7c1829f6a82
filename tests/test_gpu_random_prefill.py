"""GPU parity of prefill in chunks on seeded random problems: each case draws
its sizes (batch, key/value heads, group size, new queries Tq, cached keys
Tk >= Tq, spare cache capacity), head dimension, mask, scale and score
spread from its own PCG64 seed and runs the decode entry point, which sends
the problem to the split-key kernel, the row-chunk kernel or the forward
kernel over the cache (query i at key position Tk - Tq + i) depending on
the sizes.  Two heads per case are compared, every new query row, with the
float64 decode oracle at the bf16 tolerances (2e-2 on O, 1e-3 on LSE)."""
import math
import sys

import numpy as np
import pytest

import oracle
from gpu_util import max_err, to_device
from seeded_inputs import bf16_bits_to_f32, make_decode

pytestmark = pytest.mark.gpu

CASES = 20


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def draw(case):
    rng = np.random.Generator(np.random.PCG64(99000 + case))
    B = int(rng.choice([1, 2, 4]))
    Hkv = int(rng.choice([1, 2, 8, 16]))
    G = int(rng.choice([1, 2, 4, 8]))
    Tq = int(np.exp(rng.uniform(np.log(9), np.log(1200))))
    Tk = Tq + int(np.exp(rng.uniform(0, np.log(6000)))) - 1
    cap = Tk + int(rng.integers(0, 65))
    d = int(rng.choice([64, 128]))
    causal = bool(rng.integers(2))
    scale = float(rng.choice([1.0, 0.5, -0.7])) / math.sqrt(d)
    mult = float(rng.choice([1.0, 2.0]))
    return rng, B, Hkv * G, Hkv, Tq, Tk, cap, d, causal, scale, mult


@pytest.mark.parametrize("case", range(CASES))
def test_random_prefill(case):
    import torch

    import exact_attention_123_amd as ea
    rng, B, H, Hkv, Tq, Tk, cap, d, causal, scale, mult = draw(case)
    G = H // Hkv
    splits = ea.decode_splits(B, H, Hkv, Tq, Tk)
    ws = ea.decode_workspace_bytes(B, H, Hkv, Tq, Tk, d)
    say(f"case {case}: prefill B={B} H={H} Hkv={Hkv} Tq={Tq} Tk={Tk} cap={cap} d={d} "
        f"causal={causal} scale={scale:.4f} qk x{mult}: {splits} splits, {ws} workspace bytes")
    x = make_decode(B, H, Hkv, Tq, Tk, d, seed=99500 + case, Tk_cap=cap, qk_mult=mult)
    q, k, v = (to_device(a, "bf16") for a in (x.q, x.k, x.v))
    o, lse = ea.decode(q, k, v, Tk=Tk, causal=causal, scale=scale)
    torch.cuda.synchronize()
    O = bf16_bits_to_f32(o.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    heads = [(b, h) for b in range(B) for h in range(H)]
    eo = el = 0.0
    for i in rng.choice(len(heads), size=min(2, len(heads)), replace=False):
        b, h = heads[i]
        ref = oracle.attention_decode_head(x.q64(b, h), x.k64(b, h // G)[:Tk],
                                           x.v64(b, h // G)[:Tk], causal=causal, scale=scale)
        eo = max(eo, max_err(O[b, h], ref["O"]))
        el = max(el, max_err(L[b, h], ref["LSE"]))
    assert eo <= 2e-2 and el <= 1e-3, (eo, el)
