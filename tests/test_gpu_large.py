"""GPU parity with tensors larger than 4 GiB.

Every per-head offset of the kernels is formed in 64-bit arithmetic; these
cases put heads past the 2^31- and 2^32-byte marks of their tensors, where a
32-bit offset would wrap:

  - forward and backward at B = 16, H = 130, T = 8192, d = 128, causal (each
    [B, H, T, d] tensor 4.36 GB; head 1024 starts at byte 2^31 and head 2048
    at byte 2^32), and the grouped forward with 13 key/value heads;
  - decode over a cache of 16 sequences x 8 key/value heads x 140000 keys
    (4.59 GB per cache tensor; ragged length);
  - decode of one head at the longest cache the library accepts
    (8388543 keys at d = 128), against a closed form, and the shape error
    one key beyond it.

Inputs are seeded draws made on the device (torch's generator), so the
large tensors never cross to the host; the heads that are checked (the
first, those on either side of each mark, the last) are copied back and
compared with the float64 oracle on sampled rows (and keys) at the
tolerances of the other tests.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from seeded_inputs import QKV
from test_gpu_bwd import U, check_head, sampled

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def draw(shape, seed):
    """bf16 N(0, 1) on the device from a seeded generator."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def bits(t):
    """Host uint16 bit patterns of a bf16 device tensor."""
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def free():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


B, H, T, D = 16, 130, 8192, 128
FLAT = (0, 1023, 1024, 2047, 2048, B * H - 1)   # heads either side of 2^31 and 2^32 bytes


def test_forward_over_4gib():
    import torch

    import exact_attention_123_amd as ea
    assert B * H * T * D * 2 > 2 ** 32
    assert ea.fwd_kernel_name_for(B, H, T, D, True).endswith("_w8")
    say(f"[large fwd] B={B} H={H} T={T} d={D}: {B * H * T * D * 2 / 1e9:.2f} GB per tensor")
    q, k, v = draw((B, H, T, D), 71), draw((B, H, T, D), 72), draw((B, H, T, D), 73)
    scale = 1.0 / math.sqrt(D)
    o, lse = ea.forward(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    for f in FLAT:
        b, h = divmod(f, H)
        rows = sampled(T, 60 + f, n=24)
        ref = oracle.attention_head(*(QKV("bf16", bits(t[b, h])[None, None], None, None, 0)
                                      .q64(0, 0) for t in (q, k, v)),
                                    causal=True, scale=scale, rows=rows)
        got_o = o[b, h, rows].float().cpu().numpy().astype(np.float64)
        got_l = lse[b, h, rows].cpu().numpy().astype(np.float64)
        eo, el = float(np.abs(got_o - ref["O"]).max()), float(np.abs(got_l - ref["LSE"]).max())
        say(f"    head {f} ({b},{h}) at byte {f * T * D * 2}: O err {eo:.3e} LSE err {el:.3e}")
        assert eo <= TOL_O and el <= TOL_LSE
    del q, k, v, o, lse
    free()


def test_grouped_forward_over_4gib():
    import torch

    import exact_attention_123_amd as ea
    Hkv = 13
    say(f"[large gqa fwd] B={B} H={H} H_kv={Hkv} T={T}")
    q = draw((B, H, T, D), 81)
    k, v = draw((B, Hkv, T, D), 82), draw((B, Hkv, T, D), 83)
    scale = 1.0 / math.sqrt(D)
    o, lse = ea.forward(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    G = H // Hkv
    for f in (1024, 2048, B * H - 1):
        b, h = divmod(f, H)
        rows = sampled(T, 90 + f, n=24)
        f64 = lambda t: QKV("bf16", bits(t)[None, None], None, None, 0).q64(0, 0)
        ref = oracle.attention_head(f64(q[b, h]), f64(k[b, h // G]), f64(v[b, h // G]),
                                    causal=True, scale=scale, rows=rows)
        eo = float(np.abs(o[b, h, rows].float().cpu().numpy() - ref["O"]).max())
        el = float(np.abs(lse[b, h, rows].cpu().numpy() - ref["LSE"]).max())
        say(f"    head {f} ({b},{h}): O err {eo:.3e} LSE err {el:.3e}")
        assert eo <= TOL_O and el <= TOL_LSE
    del q, k, v, o, lse
    free()


def test_backward_over_4gib():
    import torch

    import exact_attention_123_amd as ea
    name = ea.bwd_kernel_name_for(B, H, H, T, D, True, 1)
    assert name.endswith("_bk256_bq64_w8"), name
    say(f"[large bwd] {name} B={B} H={H} T={T}")
    q, k, v, do = (draw((B, H, T, D), s) for s in (91, 92, 93, 94))
    scale = 1.0 / math.sqrt(D)
    o, lse = ea.forward(q, k, v, causal=True, scale=scale)
    ws = torch.empty(2 * B * H * T, dtype=torch.float32, device="cuda")
    dq, dk, dv = ea.backward(q, k, v, o, lse, do, causal=True, scale=scale, ws=ws)
    torch.cuda.synchronize()
    n = B * H * T
    for f in FLAT:
        b, h = divmod(f, H)
        # one head as a [1, 1, T, d] problem for the shared per-element check
        x = QKV("bf16", bits(q[b, h])[None, None], bits(k[b, h])[None, None],
                bits(v[b, h])[None, None], 0)
        g64 = [t[b, h].float().cpu().numpy().astype(np.float64)[None, None] for t in (dq, dk, dv)]
        ws_h = np.concatenate([ws[f * T:(f + 1) * T].cpu().numpy(),
                               ws[n + f * T:n + (f + 1) * T].cpu().numpy()])
        res = g64 + [ws_h, bits(o[b, h])[None, None], lse[b, h].cpu().numpy()[None, None]]
        worst = check_head(x, bits(do[b, h])[None, None], 0, 0, res, True, scale,
                           rows=sampled(T, 100 + f, n=24), keys=sampled(T, 200 + f, n=24),
                           ub=2 * U)
        say(f"    head {f} ({b},{h}): worst error / bound {worst:.3f}")
    del q, k, v, do, o, lse, ws, dq, dk, dv
    free()


def test_decode_over_4gib_cache():
    import torch

    import exact_attention_123_amd as ea
    Bd, Hd, Hkv, Tk = 16, 32, 8, 140000
    assert Bd * Hkv * Tk * D * 2 > 2 ** 32
    say(f"[large decode] B={Bd} H={Hd} H_kv={Hkv} Tk={Tk}: "
        f"{Bd * Hkv * Tk * D * 2 / 1e9:.2f} GB per cache tensor")
    q = draw((Bd, Hd, 1, D), 101)
    kc, vc = draw((Bd, Hkv, Tk, D), 102), draw((Bd, Hkv, Tk, D), 103)
    scale = 1.0 / math.sqrt(D)
    o, lse = ea.decode(q, kc, vc, causal=True, scale=scale)
    torch.cuda.synchronize()
    G = Hd // Hkv
    f64 = lambda t: QKV("bf16", bits(t)[None, None], None, None, 0).q64(0, 0)
    for (b, h) in ((0, 0), (7, 31), (8, 0), (Bd - 1, Hd - 1)):
        ref = oracle.attention_decode_head(f64(q[b, h]), f64(kc[b, h // G]), f64(vc[b, h // G]),
                                           causal=True, scale=scale)
        eo = float(np.abs(o[b, h].float().cpu().numpy() - ref["O"]).max())
        el = float(np.abs(lse[b, h].cpu().numpy() - ref["LSE"]).max())
        say(f"    ({b},{h}) cache byte {(b * Hkv + h // G) * Tk * D * 2}: "
            f"O err {eo:.3e} LSE err {el:.3e}")
        assert eo <= TOL_O and el <= TOL_LSE
    del q, kc, vc, o, lse
    free()


def test_decode_at_the_maximum_cache_length():
    """One head at the longest cache attn_decode accepts at d = 128 (a head of
    2^31 - 1 bytes holds Tk_cap + 64 rows): with Q = 0 every score is 0, so
    the single new query's output is the mean of all V rows and its LSE is
    ln(Tk), checked on the host from V read back in chunks; one key more is
    rejected as a shape error."""
    import torch

    import exact_attention_123_amd as ea
    d = 128
    Tk = (2 ** 31 - 1) // (d * 2) - 64
    say(f"[max decode] Tk={Tk} d={d}: {Tk * d * 2 / 1e9:.2f} GB per cache tensor")
    q = torch.zeros((1, 1, 1, d), dtype=torch.bfloat16, device="cuda")
    kc, vc = draw((1, 1, Tk, d), 111), draw((1, 1, Tk, d), 112)
    o, lse = ea.decode(q, kc, vc, causal=True, scale=1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    mean = np.zeros(d)
    step = 1 << 20
    for t0 in range(0, Tk, step):
        mean += vc[0, 0, t0:t0 + step].double().sum(0).cpu().numpy()
    mean /= Tk
    eo = float(np.abs(o[0, 0, 0].double().cpu().numpy() - mean).max())
    el = abs(float(lse[0, 0, 0]) - math.log(Tk))
    say(f"    O err {eo:.3e} LSE err {el:.3e} (splits {ea.decode_splits(1, 1, 1, 1, Tk)})")
    assert eo <= TOL_O and el <= TOL_LSE
    big = torch.empty((1, 1, Tk + 1, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ea.AttnError) as err:
        ea.decode(q, big, big.clone(), causal=True)
    assert err.value.code == 2  # ATTN_ERR_SHAPE
    del q, kc, vc, o, lse, big
    free()
