"""GPU parity of the dK/dV and dQ kernels' two instances each.

The backward's dK/dV kernel takes 256-key workgroups of 8 waves (32 keys
each), or 128-key workgroups of 8 waves, two per 32 keys splitting every
query tile, when the 256-key blocks of all key/value heads are fewer than
the device's CUs (under the causal mask, than twice the CUs, or at most
four times with T <= 4096).  The dQ kernel takes 128-query workgroups of 4 waves, or
of 8 waves, two per 32 queries splitting every key tile, when its 128-query
blocks are fewer than twice the CUs (under the causal mask, at most twice).  Each case asserts both instances first,
then checks sampled (or all) rows and keys of some heads against the
float64 oracle under the per-element bound of the backward tests.
"""
import math
import sys

import numpy as np
import pytest

from seeded_inputs import make_dout, make_qkv
from test_gpu_bwd import U, check_head, gpu_backward, sampled

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


# (B, H, T, d): grids below and above the switches on a 256-CU device
# (B H = 16, T = 2048: paired dK/dV and dQ; B H = 32: both causal ones
# paired, neither unmasked one; T = 100: one block, its second 32 rows
# past the end; B H = 48, T = 2048: causal dK/dV paired at 384 blocks;
# B H = 16, T = 5000: causal 320 blocks of a longer sequence, paired)
CASES = [(1, 8, 2048, 64), (1, 8, 2048, 128), (2, 3, 700, 128), (1, 1, 5000, 64),
         (1, 32, 2048, 128), (2, 16, 2048, 64), (1, 16, 2048, 64), (1, 2, 100, 128),
         (3, 1, 33, 64), (1, 48, 2048, 64), (1, 16, 5000, 64)]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("B,H,T,d", CASES)
def test_bwd_instances(B, H, T, d, causal):
    import exact_attention_123_amd as ea
    name = ea.bwd_kernel_name_for(B, H, H, T, d, causal, 1)
    blocks = B * H * ((T + 255) // 256)
    small = (blocks < 2 * cus() or (T <= 4096 and blocks <= 4 * cus())) if causal \
        else blocks < cus()
    assert name.endswith("bk128_bq64_w8" if small else "bk256_bq64_w8"), name
    qname = ea.bwd_kernel_name_for(B, H, H, T, d, causal, 2)
    qsmall = B * H * ((T + 127) // 128) < 2 * cus() + (1 if causal else 0)
    assert qname.endswith("bq128_bk64_w8" if qsmall else "bq128_bk64_w4"), qname
    say(f"[bwd instance] {name} {qname} B={B} H={H} T={T}")
    scale = 1.0 / math.sqrt(d)
    x = make_qkv(B, H, T, d, seed=8100 + T + d + H, qk_mult=2.0)
    do = make_dout(B, H, T, d, seed=8200 + T + d)
    res = gpu_backward(x, do, causal, scale)
    for (b, h) in ((0, 0), (B - 1, H - 1)):
        idx = sampled(T, 8300 + h) if T > 512 else None
        check_head(x, do, b, h, res, causal, scale, rows=idx, keys=idx, ub=2 * U)
