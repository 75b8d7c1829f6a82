"""GPU parity of the backward pass on seeded random problems: each case
draws its sizes, mask, scale and score spread from its own PCG64 seed, runs
the GPU forward and then the GPU backward on its O and LSE (the training
order), and checks sampled query rows and key rows of two heads against the
float64 gradient oracle under the per-element bound of the backward parity
tests (doubled for the terms fed by the GPU forward's O)."""
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
