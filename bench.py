#!/usr/bin/env python3
"""Benchmark of the fused exact-attention passes on one MI355X.

Default (``--pass fwd``): one step = one launch of the fused forward over the
whole batch (every head, every query row): the entire hot path.  Default
workload: B=1, H=32, T=8192, d=128, bf16, causal, Q and K drawn N(0,1) times 4
(scaled-score spread of 16), scale 1/sqrt(128).  FLOPs counted: 4*T*T*d per
head, halved under the causal mask.

``--pass bwd``: one step = one call of the backward (row statistics, dK/dV,
dQ kernels) on the same workload with a seeded upstream gradient dO, after
one untimed forward that provides O and LSE.  FLOPs counted: the five T x T x
d contractions of the gradient, 2.5 times the forward's count.

``--pass decode``: one step = one decode call (split-KV kernel and, with
several splits, the merge kernel) of the new queries over a key/value cache;
default workload B=16 sequences, 32 query heads over 8 key/value heads, one
new query each, 32768 cached keys, d=128.  The path reads the cache once, so
it is HBM-bound: the value is GB/s of algorithmic bytes (the valid cache
rows of K and V, Q, O, LSE) against MI355X's 8 TB/s.

``--pass mat``: one step = one call of the materialised three-kernel forward
(S in fp32 and P in bf16 written to and read back from device memory) on the
default forward workload; same FLOP count as the fused forward.  It is
HBM-bound: the roofline is GB/s of the S and P traffic (plus Q, K, V, O, LSE)
against 8 TB/s, and the fused forward is timed in the same run for the
comparison.

Timing: W untimed warm-up steps, then untimed steps until --settle-ms (default
2 s) of wall time has passed since the warm-up began (the shader clock of a
cold GPU needs a few hundred launches to reach its loaded steady state), then
K steps between two HIP events on the launch stream (none between the steps:
the value and the roofline both come from this region's average step).  After
the region, K more steps, each between its own pair of events, give the
spread of launch durations.  The record carries the settle phase's length,
that spread (minimum, maximum, median, the first and last five launches), and
the shader and memory clocks, socket power and power-limit residency sampled
(amdsmi, host-side) over the settle phase's last 500 ms and over the timed
region.

After the timed region the library's MFMA-only probe measures the bf16
matrix-core rate this GPU sustains with nothing else running
(``mfma_ceiling``: TFLOP/s, its clock, and the pass's fraction of it), a
secondary denominator next to the published dense peak.

Prints one JSON line with the throughput, the roofline position of the pass
(MFMA-bound, against MI355X's dense bf16 peak; for the backward the three
kernels of one call are timed together) and the float64 CPU oracle timed on a
bounded sample of the same workload on this host's cores.

    python bench.py [--pass fwd|bwd|decode|mat] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "bf16_b1h32_t8192_d128_causal_qk4"
DEFAULT_DECODE_WORKLOAD = "bf16_b16h32kv8_tq1_tk32768_d128_causal"
HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
# MI355X published dense peaks (TFLOP/s) by MFMA input type.
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
PROFILES = os.path.join(ROOT, "profiles")
DOUT_SEED_OFFSET = 7000  # dO seed = workload seed + this


def metric_name(pass_: str, causal: bool, dt: str, T: int, d: int) -> str:
    return (f"fused {'causal ' if causal else ''}attn {pass_} TFLOP/s ({dt}, T={T}, d={d}) "
            f"+ % MFMA peak")


def measured_traffic(name: str, workload: str, pass_: str = "fwd"):
    """HBM bytes per call from the committed rocprofv3 counter summary of
    this pass and workload, or None when there is none or the pass's kernel
    code changed since the counters were taken."""
    from exact_attention_123_amd.rocprof_summary import source_sha

    path = os.path.join(PROFILES, f"{name}__{workload}__traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel_code_sha256:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not b or h.group(1) != source_sha(pass_):
        return None
    return float(b.group(1))


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        return int(max((p["num_threads"] for p in blas), default=1))
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(x, causal: bool, scale: float, heads: int, pass_: str, do_bits=None):
    """Time the float64 oracle on the first `heads` heads (all rows)."""
    import oracle
    from seeded_inputs import bf16_bits_to_f32

    B, H, T, d = x.shape
    G = H // x.k.shape[1]  # query heads per key/value head
    t0 = time.perf_counter()
    done = 0
    for i in range(heads):
        b, h = divmod(i, H)
        if pass_ == "fwd":
            oracle.attention_head(x.q64(b, h), x.k64(b, h // G), x.v64(b, h // G),
                                  causal=causal, scale=scale)
        else:
            g = bf16_bits_to_f32(do_bits[b, h]).astype("float64")
            oracle.attention_head_bwd(x.q64(b, h), x.k64(b, h // G), x.v64(b, h // G), g,
                                      causal=causal, scale=scale)
        done += 1
    dt = time.perf_counter() - t0
    fl = 4.0 * T * T * d * done / (2 if causal else 1) * (2.5 if pass_ == "bwd" else 1.0)
    what = ("S and P materialised" if pass_ == "fwd"
            else "forward, P, dP and dS materialised, all of dQ, dK, dV")
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": f"{done} of {B * H} heads, all {T} rows each; float64 numpy, {what}; "
                  f"{dt:.1f} s wall",
        "seconds": dt,
        "host_cpus": len(os.sched_getaffinity(0)),
        "blas": blas_info(),
    }


class GpuMetricsSampler:
    """Samples the GPU's clocks, power and throttle-residency counters
    (amdsmi's gpu_metrics table, host-side reads only) on a background thread
    while the benchmark runs, so that the record shows the clock state the
    timed launches ran at.  Any failure (no amdsmi, no permission) leaves the
    fields None with the reason."""

    KEYS = ("current_gfxclks", "current_gfxclk", "current_uclk", "current_socket_power",
            "accumulation_counter", "ppt_residency_acc",
            "socket_thm_residency_acc", "temperature_hotspot")

    def __init__(self, period_s: float = 0.004):
        self.period = period_s
        self.samples = []
        self.error = None
        self._handle = None
        self._stop = None
        self._thread = None

    def start(self):
        import threading
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if not handles:
                raise RuntimeError("no GPU handle")
            self._handle = handles[0]
            self._amdsmi = amdsmi
            self._read()  # fail here rather than in the thread
        except Exception as e:  # pragma: no cover - depends on the machine
            self.error = f"{type(e).__name__}: {e}"
            return self
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()
        return self

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        return (time.perf_counter(), {k: m.get(k) for k in self.KEYS})

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception as e:  # pragma: no cover
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period)

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            try:
                self.samples.append(self._read())
                self._amdsmi.amdsmi_shut_down()
            except Exception:  # pragma: no cover
                pass

    @staticmethod
    def _num(v):
        return v if isinstance(v, (int, float)) and v not in (65535, 0xFFFFFFFF) else None

    def window(self, t0: float, t1: float):
        """Summary of the samples taken in [t0, t1] (perf_counter seconds):
        median shader clock over the XCDs, memory clock, socket power, and
        from the residency accumulators the fraction of the window spent at
        the package power limit (and at a thermal limit)."""
        if self.error and not self.samples:
            return {"error": self.error}
        sel = [(t, m) for t, m in self.samples if t0 <= t <= t1]
        if not sel:
            return {"samples": 0}

        def med(xs):
            xs = sorted(x for x in xs if x is not None)
            return xs[len(xs) // 2] if xs else None

        def xcd_mean(m):
            v = m.get("current_gfxclks")
            vals = [self._num(x) for x in v] if isinstance(v, (list, tuple)) else []
            vals = [x for x in vals if x]
            return sum(vals) / len(vals) if vals else self._num(m.get("current_gfxclk"))

        out = {"samples": len(sel),
               "sclk_mhz_median": med([xcd_mean(m) for _, m in sel]),
               "sclk_mhz_min": min((x for x in (xcd_mean(m) for _, m in sel) if x),
                                   default=None),
               "mclk_mhz_median": med([self._num(m.get("current_uclk")) for _, m in sel]),
               "socket_power_w_median": med([self._num(m.get("current_socket_power"))
                                             for _, m in sel]),
               "hotspot_c_max": max((self._num(m.get("temperature_hotspot")) or 0
                                     for _, m in sel), default=None)}
        (ta, a), (tb, b) = sel[0], sel[-1]
        try:
            dacc = b["accumulation_counter"] - a["accumulation_counter"]
            if dacc > 0:
                out["ppt_limited_frac"] = round(
                    (b["ppt_residency_acc"] - a["ppt_residency_acc"]) / dacc, 3)
                out["thermal_limited_frac"] = round(
                    (b["socket_thm_residency_acc"] - a["socket_thm_residency_acc"]) / dacc, 3)
        except (TypeError, KeyError):
            pass
        return out


def time_steps(step, stream, steps: int, warmup: int, settle_ms: float = 0.0, sampler=None):
    """W untimed steps, then (untimed) more steps until `settle_ms` of wall
    time has passed since the warm-up began, so that the clocks reach their
    loaded steady state; then the timed region: K steps between one pair of
    HIP events on the launch stream, none between the steps (an event pair
    per step adds several microseconds of device time to each step, half
    again on a 15 us launch); then, after the region, K more steps each
    between its own pair of events, for the spread of launch durations.
    Returns (per-step ms list of that spread pass, region ms, wall s of the
    region, info) with info holding the settle phase's length and, when a
    sampler runs, the clock and power summary of the settle phase's last
    500 ms and of the timed region."""
    import torch

    t_warm = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    settle_steps = 0
    while (time.perf_counter() - t_warm) * 1e3 < settle_ms:
        for _ in range(8):
            step()
        settle_steps += 8
        torch.cuda.synchronize()
    t_settled = time.perf_counter()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for _ in range(steps):
        step()
    r1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    info = {"settle_ms": round((t_settled - t_warm) * 1e3, 1), "settle_steps": settle_steps,
            "warmup_steps": warmup}
    if sampler is not None:
        time.sleep(3 * sampler.period)  # one more sample after the spread pass
        sampler.stop()
        info["clocks_settle_last_500ms"] = sampler.window(t_settled - 0.5, t_settled)
        # the first sample after the region closes it (the accumulators are
        # differenced between the first and last samples of the window)
        info["clocks_timed_region"] = sampler.window(t0, t1 + sampler.period)
    return per, r0.elapsed_time(r1), wall, info


def timing_record(region_ms: float, steps: int, wall: float, per, tinfo) -> dict:
    """The record's timing block: the timed region's average step, and the
    spread pass's average, minimum, maximum, median and first and last five
    launch durations (ms)."""
    return {"avg_launch_ms": round(region_ms / steps, 4), "wall_s": round(wall, 3),
            "spread_pass": {"avg_launch_ms": round(sum(per) / len(per), 4),
                            "min_launch_ms": round(min(per), 4),
                            "max_launch_ms": round(max(per), 4), **launch_spread(per)},
            **tinfo}


def mfma_ceiling(dev, sampler=None, shape: int = 0):
    """The measured matrix-core ceiling: the library's MFMA-only probe
    (independent bf16 accumulation chains on register operands, 4 waves per
    workgroup, 8 workgroups per CU), timed with HIP events on its stream
    after one untimed launch.  Returns TFLOP/s and, with a sampler, the
    shader clock during the probe."""
    import torch

    import exact_attention_123_amd as ea

    lib = ea.load_library()
    wg = 8 * torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 8000
    sink = torch.empty(wg * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream
    if lib.attn_probe_mfma(shape, wg, iters, sink.data_ptr(), s) != 0:
        return {"error": "probe launch failed"}
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(3):
        lib.attn_probe_mfma(shape, wg, iters, sink.data_ptr(), s)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = e0.elapsed_time(e1) / 3
    out = {"tflops": round(lib.attn_probe_mfma_flops(shape, wg, iters) / (ms * 1e-3) / 1e12, 1),
           "instruction": ("v_mfma_f32_32x32x16_bf16" if shape == 0
                           else "v_mfma_f32_16x16x32_bf16"),
           "avg_launch_ms": round(ms, 3)}
    if sampler is not None:
        out["clocks"] = sampler.window(t0, t1)
    return out


def launch_spread(per):
    """Median and the first and last five launch durations (ms) of a pass
    timed launch by launch."""
    srt = sorted(per)
    mid = len(srt) // 2
    median = srt[mid] if len(srt) % 2 else 0.5 * (srt[mid - 1] + srt[mid])
    return {"median_launch_ms": round(median, 4),
            "first5_ms": [round(x, 4) for x in per[:5]],
            "last5_ms": [round(x, 4) for x in per[-5:]]}


def blas_info():
    """The BLAS library numpy uses (name, version, threads) for the CPU
    baseline record."""
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        return [{"library": p.get("internal_api"), "version": p.get("version"),
                 "threads": p.get("num_threads"),
                 "file": os.path.basename(p.get("filepath", ""))} for p in blas]
    except Exception as e:  # pragma: no cover
        return [{"error": str(e)}]


def copy_calibration(mib: int, dev):
    """One plain device-to-device copy of `mib` MiB (counter calibration)."""
    import torch

    if mib:
        n = mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()


def run_decode(args) -> int:
    import numpy as np
    import torch

    import exact_attention_123_amd as ea
    import oracle
    from seeded_inputs import DECODE_WORKLOADS, bf16_bits_to_f32, make_decode

    name = args.workload or DEFAULT_DECODE_WORKLOAD
    w = DECODE_WORKLOADS[name]
    B, H, Hkv, Tq, Tk, d, causal = (w[k] for k in ("B", "H", "H_kv", "Tq", "Tk", "d", "causal"))
    G = H // Hkv
    scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = make_decode(B, H, Hkv, Tq, Tk, d, seed=w["seed"])

    def up(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v = up(x.q), up(x.k), up(x.v)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    need = ea.decode_workspace_bytes(B, H, Hkv, Tq, Tk, d)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    def step():
        ea.decode(q, k, v, Tk=Tk, causal=causal, scale=scale, out=out, lse=lse, ws=ws)

    def ref_head(b, h):
        g = h // G
        return oracle.attention_decode_head(
            bf16_bits_to_f32(x.q[b, h]).astype(np.float64),
            bf16_bits_to_f32(x.k[b, g, :Tk]).astype(np.float64),
            bf16_bits_to_f32(x.v[b, g, :Tk]).astype(np.float64), causal=causal, scale=scale)

    parity = None
    if not args.no_parity:
        step()
        torch.cuda.synchronize()
        O = bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16))
        L = lse.cpu().numpy()
        eo = el = 0.0
        heads = [(0, 0), (0, H - 1), (B - 1, 0), (B - 1, H - 1)]
        for (b, h) in heads:
            r = ref_head(b, h)
            eo = max(eo, float(np.abs(O[b, h] - r["O"]).max()))
            el = max(el, float(np.abs(L[b, h] - r["LSE"]).max()))
        parity = {"heads_checked": len(heads), "max_abs_err_o": eo, "max_abs_err_lse": el,
                  "pass": bool(eo <= 2e-2 and el <= 1e-3)}
        if not parity["pass"]:
            print(json.dumps({"error": "parity failed", "parity": parity}), flush=True)
            return 1

    stream = torch.cuda.current_stream(dev)
    sampler = None if args.no_clock_sampler else GpuMetricsSampler().start()
    per, region_ms, wall, tinfo = time_steps(step, stream, args.steps, args.warmup,
                                             args.settle_ms, sampler)
    copy_calibration(args.copy_calibration_mib, dev)
    ms_per_step = region_ms / args.steps
    nbytes = (2 * B * Hkv * Tk * d * 2      # valid K and V cache rows, read once
              + 2 * B * H * Tq * d * 2      # Q read, O written
              + B * H * Tq * 4)             # LSE written
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = value  # one launch per step, averaged over the timed region
    kname = f"attn_decode_bf16_d{d}_{'causal' if causal else 'full'}_w4_blk32"
    traffic = measured_traffic(kname, name, "decode")
    res = {
        "metric": f"decode attn GB/s (bf16, Tq={Tq}, Tk={Tk}, d={d}) + % HBM peak",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded PCG64 N(0,1) draws rounded to bf16 (RNE)",
        "config": {"workload": name, "pass": "decode", "B": B, "H": H, "H_kv": Hkv, "Tq": Tq,
                   "Tk": Tk, "d": d, "causal": causal, "scale": scale,
                   "splits": ea.decode_splits(B, H, Hkv, Tq, Tk), "bytes_per_step": nbytes,
                   "kernel": kname, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "timing": timing_record(region_ms, args.steps, wall, per, tinfo),
        "parity": parity,
    }
    if not args.no_cpu_baseline:
        seqs = args.cpu_heads if args.cpu_heads is not None else 2
        t0 = time.perf_counter()
        done = 0
        for b in range(min(seqs, B)):
            for h in range(H):
                ref_head(b, h)
            done += 1
        dt = time.perf_counter() - t0
        cb = done * (2 * Hkv * Tk * d * 2 + 2 * H * Tq * d * 2 + H * Tq * 4)
        res["cpu_baseline"] = {
            "value": cb / dt / 1e9, "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} of {B} sequences, all {H} query heads each; float64 numpy, "
                      f"scores and probabilities materialised; {dt:.1f} s wall",
            "seconds": dt, "host_cpus": len(os.sched_getaffinity(0)), "blas": blas_info()}
    print(json.dumps(res), flush=True)
    return 0


def mat_bytes(B: int, H: int, T: int, d: int, causal: bool) -> int:
    """Algorithmic bytes of one materialised forward: S written (fp32) and
    read once over each row's visible part, P written and read (bf16) over
    the tiles the kernels touch, Q, K, V read once, O and LSE written."""
    R = 128  # query rows per block of the scores and P V kernels
    if causal:
        nqb = T // R
        touched = R * R * nqb * (nqb + 1) // 2  # entries of the blocks' key ranges
        visible = T * (T + 1) // 2
    else:
        touched = visible = T * T
    per_head = touched * 4 + visible * 4 + 2 * touched * 2 + 4 * T * d * 2 + T * 4
    return B * H * per_head


def run_mat(args) -> int:
    import numpy as np
    import torch

    import exact_attention_123_amd as ea
    import oracle
    from seeded_inputs import WORKLOADS, bf16_bits_to_f32, make_workload

    name = args.workload or DEFAULT_WORKLOAD
    w = WORKLOADS[name]
    causal = w["causal"][0]
    B, H, T, d = w["B"], w["H"], w["T"], w["d"]
    scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = make_workload(name)

    def up(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v = up(x.q), up(x.k), up(x.v)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    s_buf = torch.empty((B, H, T, T), dtype=torch.float32, device=dev)
    p_buf = torch.empty((B, H, T, T), dtype=torch.bfloat16, device=dev)

    def step():
        ea.forward_materialized(q, k, v, causal=causal, scale=scale, out=out, lse=lse,
                                s_buf=s_buf, p_buf=p_buf)

    parity = None
    if not args.no_parity:
        step()
        torch.cuda.synchronize()
        O = bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16))
        L = lse.cpu().numpy()
        rows = np.unique(np.r_[0, 1, 127, 128, T // 2, T - 1,
                               np.random.Generator(np.random.PCG64(9)).choice(T, 24)])
        eo = el = 0.0
        for (b, h) in ((0, 0), (B - 1, H - 1)):
            ref = oracle.attention_head(x.q64(b, h), x.k64(b, h), x.v64(b, h), causal=causal,
                                        scale=scale, rows=rows)
            eo = max(eo, float(np.abs(O[b, h][rows] - ref["O"]).max()))
            el = max(el, float(np.abs(L[b, h][rows] - ref["LSE"]).max()))
        parity = {"rows_checked": int(2 * len(rows)), "max_abs_err_o": eo,
                  "max_abs_err_lse": el, "pass": bool(eo <= 2e-2 and el <= 1e-3)}
        if not parity["pass"]:
            print(json.dumps({"error": "parity failed", "parity": parity}), flush=True)
            return 1

    stream = torch.cuda.current_stream(dev)
    steps = max(1, args.steps // 10)  # each step moves ~13 GB: a tenth of the steps
    warm = max(1, args.warmup // 10)
    per, region_ms, wall, tinfo = time_steps(step, stream, steps, warm)
    o2 = torch.empty_like(q)
    l2 = torch.empty_like(lse)
    _, fused_region_ms, _, _ = time_steps(lambda: ea.forward(q, k, v, causal=causal, scale=scale,
                                                             out=o2, lse=l2), stream, steps, warm)
    copy_calibration(args.copy_calibration_mib, dev)
    ms_per_step = region_ms / steps
    avg_ms = ms_per_step
    fused_ms = fused_region_ms / steps
    fl = ea.flops(B, H, T, d, causal)
    nbytes = mat_bytes(B, H, T, d, causal)
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    kname = f"attn_mat_bf16_d{d}_{'causal' if causal else 'full'}_3k"
    res = {
        "metric": (f"materialised {'causal ' if causal else ''}attn fwd TFLOP/s (bf16, T={T}, "
                   f"d={d}) + % HBM peak"),
        "value": round(fl / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded PCG64 N(0,1) draws rounded to bf16 (RNE)"
                + (", Q and K multiplied by 4" if w.get("qk_mult", 1.0) != 1.0 else ""),
        "config": {"workload": name, "pass": "mat", "B": B, "H": H, "T": T, "d": d,
                   "causal": causal, "scale": scale, "flops_per_step": fl,
                   "bytes_per_step": nbytes, "s_dtype": "f32", "p_dtype": "bf16",
                   "kernel": kname, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(kname, name, "mat")},
        "timing": timing_record(region_ms, steps, wall, per, tinfo),
        "compare": {"fused_fwd_avg_ms": round(fused_ms, 4),
                    "materialised_over_fused": round(avg_ms / fused_ms, 2)},
        "parity": parity,
    }
    if not args.no_cpu_baseline:
        heads = args.cpu_heads if args.cpu_heads is not None else 32
        res["cpu_baseline"] = cpu_baseline(x, causal, scale, min(heads, B * H), "fwd")
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--pass", dest="pass_", choices=["fwd", "bwd", "decode", "mat"],
                    default="fwd")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--mask", choices=["causal", "full"], default=None,
                    help="forward/backward: which of the workload's masks to run "
                         "(default: its first)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=None,
                    help="heads (fwd, bwd) or sequences (decode) of the workload the CPU "
                         "oracle is timed on (default 32 for fwd, 2 for bwd and decode)")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=2000.0,
                    help="untimed: keep stepping after the warm-up until this much wall "
                         "time has passed since it began, so the clocks settle under load "
                         "before the timed region (reported as timing.settle_ms)")
    ap.add_argument("--no-clock-sampler", action="store_true",
                    help="do not sample clocks and power (amdsmi) around the timed region")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip the MFMA-only probe (the measured ceiling reported next to "
                         "the published peak)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (for counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(heads shard across GPUs with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    if args.pass_ == "decode":
        return run_decode(args)
    if args.pass_ == "mat":
        return run_mat(args)
    args.workload = args.workload or DEFAULT_WORKLOAD

    import numpy as np
    import torch

    import exact_attention_123_amd as ea
    from seeded_inputs import WORKLOADS, bf16_bits_to_f32, make_dout, make_workload

    w = WORKLOADS[args.workload]
    causal = w["causal"][0]
    if args.mask is not None:
        causal = args.mask == "causal"
        if causal not in w["causal"]:
            print(f"workload {args.workload} has no {args.mask} mask", file=sys.stderr)
            return 2
    B, H, T, d, dt = w["B"], w["H"], w["T"], w["d"], w["dtype"]
    bwd = args.pass_ == "bwd"
    Hkv = w.get("H_kv", H)
    if bwd and dt != "bf16":
        print("bench --pass bwd takes bf16 workloads", file=sys.stderr)
        return 2
    scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    x = make_workload(args.workload)

    def up(a):
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    def to64(t):
        if dt == "bf16":
            return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
        return t.cpu().numpy()

    q, k, v = up(x.q), up(x.k), up(x.v)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    if bwd:
        do_bits = make_dout(B, H, T, d, seed=x.seed + DOUT_SEED_OFFSET)
        dout = up(do_bits)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(2 * B * H * T, dtype=torch.float32, device=dev)
        ea.forward(q, k, v, causal=causal, scale=scale, out=out, lse=lse)
        # the instances attn_bwd_gqa launches for these sizes on this device
        kname = ea.bwd_kernel_name_for(B, H, Hkv, T, d, causal, 1)
        knames = [ea.bwd_kernel_name_for(B, H, Hkv, T, d, causal, i) for i in range(3)]
        fl = ea.bwd_flops(B, H, T, d, causal)
    else:
        do_bits = None
        # the instance attn_fwd launches for these sizes on this device
        kname = (ea.fwd_f32_kernel_name_for(B, H, T, d, causal) if dt == "f32"
                 else ea.fwd_kernel_name_for(B, H, T, d, causal))
        knames = [kname]
        fl = ea.flops(B, H, T, d, causal)

    def step():
        if bwd:
            ea.backward(q, k, v, out, lse, dout, causal=causal, scale=scale, dq=dq, dk=dk,
                        dv=dv, ws=ws)
        else:
            ea.forward(q, k, v, causal=causal, scale=scale, out=out, lse=lse)

    # Parity before timing: sampled rows (and keys) of two heads against the
    # oracle.
    parity = None
    if not args.no_parity:
        import oracle
        step()
        torch.cuda.synchronize()
        rng = np.random.Generator(np.random.PCG64(9))
        rows = np.unique(np.r_[0, 1, 63, 64, 127, 128, T // 2, T - 1, rng.choice(T, 24)])
        heads = ((0, 0), (B - 1, H - 1))
        if not bwd:
            O, L = to64(out), lse.cpu().numpy()
            eo = el = 0.0
            G = H // Hkv
            for (b, h) in heads:
                ref = oracle.attention_head(x.q64(b, h), x.k64(b, h // G), x.v64(b, h // G),
                                            causal=causal, scale=scale, rows=rows)
                eo = max(eo, float(np.abs(O[b, h][rows] - ref["O"]).max()))
                el = max(el, float(np.abs(L[b, h][rows] - ref["LSE"]).max()))
            tol = (2e-2, 1e-3) if dt == "bf16" else (1e-5, 1e-5)
            parity = {"rows_checked": int(2 * len(rows)), "max_abs_err_o": eo,
                      "max_abs_err_lse": el, "pass": bool(eo <= tol[0] and el <= tol[1])}
        else:
            # Relative to the largest reference magnitude of each gradient;
            # the parity tests hold the per-element bound.
            # (grouped heads: dQ of query head h against its key/value head
            # h // G; dK, dV of key/value head g sum its G query heads')
            G = [to64(t) for t in (dq, dk, dv)]
            grp = H // Hkv
            worst = 0.0

            def rel(got, want):
                return float(np.abs(got - want).max() / np.abs(want).max())

            for (b, h) in heads:
                g = bf16_bits_to_f32(do_bits[b, h]).astype(np.float64)
                ref = oracle.attention_head_bwd(x.q64(b, h), x.k64(b, h // grp),
                                                x.v64(b, h // grp), g, causal=causal,
                                                scale=scale, rows=rows, keys=rows)
                worst = max(worst, rel(G[0][b, h][rows], ref["dQ"]))
            for (b, kh) in ((0, 0), (B - 1, Hkv - 1)):
                rdk = rdv = 0.0
                for h in range(kh * grp, (kh + 1) * grp):
                    g = bf16_bits_to_f32(do_bits[b, h]).astype(np.float64)
                    ref = oracle.attention_head_bwd(x.q64(b, h), x.k64(b, kh), x.v64(b, kh), g,
                                                    causal=causal, scale=scale, rows=rows,
                                                    keys=rows)
                    rdk = rdk + ref["dK"]
                    rdv = rdv + ref["dV"]
                worst = max(worst, rel(G[1][b, kh][rows], rdk), rel(G[2][b, kh][rows], rdv))
            parity = {"rows_checked": int(2 * len(rows)), "keys_checked": int(2 * len(rows)),
                      "max_err_rel_to_max_ref": worst, "pass": bool(worst <= 2e-2)}
        if not parity["pass"]:
            print(json.dumps({"error": "parity failed", "parity": parity}), flush=True)
            return 1

    stream = torch.cuda.current_stream(dev)  # the launch stream of the binding
    sampler = None if args.no_clock_sampler else GpuMetricsSampler().start()
    per_launch_ms, region_ms, wall, tinfo = time_steps(step, stream, args.steps, args.warmup,
                                                       args.settle_ms, sampler)
    ms_per_step = region_ms / args.steps
    avg_launch_ms = ms_per_step  # one launch (one call) per step
    copy_calibration(args.copy_calibration_mib, dev)

    ceiling = None
    if dt == "bf16" and not args.no_mfma_ceiling:
        psampler = None if args.no_clock_sampler else GpuMetricsSampler().start()
        ceiling = mfma_ceiling(dev, psampler)
        if psampler is not None:
            time.sleep(3 * psampler.period)
            psampler.stop()
            ceiling["clocks"] = psampler.window(0.0, time.perf_counter())

    value = fl / (ms_per_step * 1e-3) / 1e12
    achieved = fl / (avg_launch_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dt]
    if ceiling is not None and ceiling.get("tflops"):
        ceiling["frac"] = round(achieved / ceiling["tflops"], 4)
    traffic = measured_traffic(kname, args.workload, args.pass_)

    config = {"workload": args.workload + (("_causal" if causal else "_full")
                                           if len(w["causal"]) > 1 else ""),
              "pass": args.pass_, "B": B, "H": H, "H_kv": Hkv,
              "T": T, "d": d,
              "causal": causal, "scale": scale, "qk_mult": w.get("qk_mult", 1.0),
              "flops_per_step": fl, "kernel": kname, "parallelism": "single GPU"}
    if causal:
        # the metric counts 4 T^2 d per head halved; the causal mask keeps
        # T (T + 1) / 2 score entries, the diagonal included
        config["flops_exact_causal"] = (4.0 * B * H * d * T * (T + 1) / 2
                                        * (2.5 if bwd else 1.0))
    if bwd:
        config["kernels"] = knames
        config["dout_seed"] = x.seed + DOUT_SEED_OFFSET
    res = {
        "metric": metric_name(args.pass_, causal, dt, T, d),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": ("synthetic: seeded PCG64 N(0,1) draws rounded to bf16 (RNE)" if dt == "bf16"
                 else "synthetic: seeded PCG64 N(0,1) float32 draws")
                + (", Q and K multiplied by 4" if w.get("qk_mult", 1.0) != 1.0 else "")
                + ("; dO N(0,1) rounded to bf16" if bwd else ""),
        "config": config,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic},
        "timing": timing_record(region_ms, args.steps, wall, per_launch_ms, tinfo),
        "parity": parity,
    }
    if ceiling is not None:
        # secondary denominator: the bf16 MFMA rate this GPU sustains with
        # nothing else running (untimed, after the timed region)
        res["mfma_ceiling"] = ceiling
    if not args.no_cpu_baseline:
        heads = args.cpu_heads if args.cpu_heads is not None else (2 if bwd else 32)
        res["cpu_baseline"] = cpu_baseline(x, causal, scale, min(heads, B * H), args.pass_,
                                           do_bits)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
