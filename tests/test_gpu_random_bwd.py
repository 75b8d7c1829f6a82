"""GPU parity of the backward pass on seeded random problems: each case
draws its sizes, mask, scale and score spread from its own PCG64 seed, runs
the GPU forward and then the GPU backward on its O and LSE (the training
order), and checks sampled query rows and key rows of two heads against the
float64 gradient oracle under the per-element bound of the backward parity
tests (doubled for the terms fed by the GPU forward's O).  The first set
draws small grids (up to 6 heads, T < 3000); the second draws grids that
fill the GPU (8 to 64 key/value heads, T from 1024 to 4096) with grouped
query heads (G = 1, 2, 4) and scales including 0 and negative ones."""
import math

import numpy as np
import pytest

from seeded_inputs import make_dout, make_qkv
from test_gpu_bwd import U, check_head, gpu_backward, sampled, say

pytestmark = pytest.mark.gpu

CASES = 16


@pytest.mark.parametrize("case", range(CASES))
def test_random_backward(case):
    rng = np.random.Generator(np.random.PCG64(95000 + case))
    B = int(rng.choice([1, 2]))
    H = int(rng.choice([1, 2, 3]))
    T = int(np.exp(rng.uniform(0, np.log(3000))))
    d = int(rng.choice([64, 128]))
    causal = bool(rng.integers(2))
    scale = float(rng.choice([1.0, 0.5, -0.7])) / math.sqrt(d)
    mult = float(rng.choice([1.0, 2.0]))
    say(f"case {case}: bwd B={B} H={H} T={T} d={d} causal={causal} scale={scale:.4f} "
        f"qk x{mult}")
    x = make_qkv(B, H, T, d, seed=96000 + case, qk_mult=mult)
    do = make_dout(B, H, T, d, seed=97000 + case)
    res = gpu_backward(x, do, causal, scale)
    heads = [(b, h) for b in range(B) for h in range(H)]
    for i in rng.choice(len(heads), size=min(2, len(heads)), replace=False):
        b, h = heads[i]
        idx = sampled(T, 98000 + case, n=min(32, T)) if T > 256 else None
        check_head(x, do, b, h, res, causal, scale, rows=idx, keys=idx, ub=2 * U)


LARGE_CASES = 8


@pytest.mark.parametrize("case", range(LARGE_CASES))
def test_random_backward_large(case):
    """Seeded random problems on grids that fill the GPU (the 8-wave dK/dV
    instance, or the 4-wave one near the switch), with grouped key/value
    heads (G = 1, 2 or 4): the gradients of one key/value head and of its
    query heads, on sampled rows and keys, against the oracle."""
    import torch

    import exact_attention_123_amd as ea
    from gpu_util import to_device
    from test_gpu_gqa import check_bwd, gpu_fwd
    rng = np.random.Generator(np.random.PCG64(99000 + case))
    B = int(rng.choice([1, 2]))
    Hkv = int(rng.choice([8, 16, 32]))
    G = int(rng.choice([1, 2, 4]))
    H = Hkv * G
    T = int(np.exp(rng.uniform(np.log(1024), np.log(4096))))
    d = int(rng.choice([64, 128]))
    causal = bool(rng.integers(2))
    scale = float(rng.choice([1.0, 0.5, -0.7, 0.0])) / math.sqrt(d)
    mult = float(rng.choice([1.0, 2.0]))
    name = ea.bwd_kernel_name_for(B, H, Hkv, T, d, causal, 1)
    say(f"case {case}: bwd B={B} H={H} Hkv={Hkv} T={T} d={d} causal={causal} "
        f"scale={scale:.4f} qk x{mult}: {name}")
    x = make_qkv(B, H, T, d, seed=99500 + case, qk_mult=mult, H_kv=Hkv)
    do_bits = make_dout(B, H, T, d, seed=99700 + case)
    (q, k, v, o, lse), O, _ = gpu_fwd(x, causal, scale)
    dq, dk, dv = ea.backward(q, k, v, o, lse, to_device(do_bits, "bf16"), causal=causal,
                             scale=scale)
    torch.cuda.synchronize()
    b, g = int(rng.integers(B)), int(rng.integers(Hkv))
    dQ = np.zeros((B, H, T, d))
    dQ[b, g * G:(g + 1) * G] = dq[b, g * G:(g + 1) * G].float().cpu().numpy()
    dK = np.zeros((B, Hkv, T, d))
    dV = np.zeros_like(dK)
    dK[b, g] = dk[b, g].float().cpu().numpy()
    dV[b, g] = dv[b, g].float().cpu().numpy()
    check_bwd(x, do_bits, dQ, dK, dV, O, causal, scale, b, g,
              keys=sampled(T, 99900 + case, n=24), ub=2 * U)
