"""Concurrent calls of the library (GPU): the C ABI keeps no mutable state
beyond a per-device cache of the architecture check and CU count, so calls
on different streams, and calls from several host threads, must each give
exactly what the same call gives alone (every kernel here is deterministic:
a fixed summation order, no atomics).

  - forward, backward and decode enqueued interleaved on three streams,
    several rounds, against the same calls run one at a time: bitwise;
  - four host threads, each calling forward (and the kernel-name query)
    on its own stream with its own inputs, many times: bitwise against the
    single-threaded result.
"""
import math
import sys
import threading

import pytest

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(seed, B, H, T, d, Hkv=None):
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    Hkv = Hkv or H
    q = torch.randn(B, H, T, d, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hkv, T, d, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, T, d, device="cuda", generator=g).to(torch.bfloat16)
    return q, k, v


def test_three_streams_interleaved():
    import torch

    import exact_attention_123_amd as ea
    say("[concurrency] forward, backward and decode on three streams")
    qf, kf, vf = _inputs(1, 1, 32, 2048, 128)
    qb, kb, vb = _inputs(2, 1, 8, 1500, 64, Hkv=2)
    dob = torch.randn_like(qb)
    ob, lb = ea.forward(qb, kb, vb, causal=True)
    qd = torch.randn(4, 32, 1, 128, device="cuda").to(torch.bfloat16)
    kd = torch.randn(4, 8, 20000, 128, device="cuda").to(torch.bfloat16)
    vd = torch.randn_like(kd)
    torch.cuda.synchronize()
    # alone
    ref_f = ea.forward(qf, kf, vf, causal=True)
    torch.cuda.synchronize()
    ref_b = ea.backward(qb, kb, vb, ob, lb, dob, causal=True)
    torch.cuda.synchronize()
    ref_d = ea.decode(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    for rnd in range(4):
        outs = []
        with torch.cuda.stream(streams[0]):
            f = ea.forward(qf, kf, vf, causal=True)
        with torch.cuda.stream(streams[1]):
            b = ea.backward(qb, kb, vb, ob, lb, dob, causal=True)
        with torch.cuda.stream(streams[2]):
            dd = ea.decode(qd, kd, vd, causal=True)
        # a second forward on the backward's stream, behind it
        with torch.cuda.stream(streams[1]):
            f2 = ea.forward(qf, kf, vf, causal=True)
        torch.cuda.synchronize()
        for got, want in ((f, ref_f), (b, ref_b), (dd, ref_d), (f2, ref_f)):
            for x, y in zip(got, want):
                assert torch.equal(x, y), rnd


def test_host_threads():
    import torch

    import exact_attention_123_amd as ea
    say("[concurrency] four host threads calling forward")
    shapes = [(1, 8, 1024, 64), (1, 4, 3000, 128), (2, 16, 512, 128), (1, 32, 2048, 128)]
    inputs = [_inputs(10 + i, *s) for i, s in enumerate(shapes)]
    refs = []
    for (q, k, v) in inputs:
        refs.append(ea.forward(q, k, v, causal=True))
    torch.cuda.synchronize()
    errors = []

    def work(i):
        try:
            q, k, v = inputs[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(25):
                    B, H, T, d = shapes[i]
                    assert ea.fwd_kernel_name_for(B, H, T, d, True) is not None
                    o, lse = ea.forward(q, k, v, causal=True)
                    s.synchronize()
                    if not (torch.equal(o, refs[i][0]) and torch.equal(lse, refs[i][1])):
                        errors.append(f"thread {i}: result differs")
                        return
        except Exception as e:  # reported below
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
