"""Turn rocprofv3 CSV output into the short text summaries kept under
``profiles/``.

A "pass" is the forward (one kernel per call, symbols containing
``attn_fwd_``), the backward (three kernels per call, ``attn_bwd_``) or the
decode (one or two kernels per call, ``attn_decode_``) or the materialised
forward (three kernels per call, ``attn_mat_``).
Summaries per (name, workload), where name is the forward kernel's instance
name or the backward's dK/dV kernel name:

``<name>__<workload>__kernel_trace.md``
    calls, average / min / max duration of each kernel of the pass from a
    ``rocprofv3 --kernel-trace --stats`` run of ``bench.py``, the sum of the
    averages (one call of the pass) and the TFLOP/s that sum implies.

``<name>__<workload>__mfma_util.md``
    matrix-core busy fraction from one ``rocprofv3 --pmc`` run of
    ``SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_INSTS_MFMA``:
    busy SIMD-cycles over (GPU-active cycles per XCD x 1024 SIMDs), and the
    clock that GPU-active cycles over the traced average duration imply.

``<name>__<workload>__counters.md``
    any other ``rocprofv3 --pmc`` passes (``--counters CSV --counters-cmd
    CMD``, repeatable): each counter's value per call, summed over the
    pass's kernels, and its share of ``SQ_WAVE_CYCLES`` when that counter
    was collected in the same pass.

``<name>__<workload>__traffic.md``
    device-memory bytes per call from two ``rocprofv3 --pmc`` runs
    (``FETCH_SIZE``, then ``WRITE_SIZE``), each scaled by what the same
    counter reads for a plain device-to-device copy of known size
    (``bench.py --copy-calibration-mib N`` launches it after the timed
    region), summed over the pass's kernels.  It records the SHA-256 of the
    pass's kernel code the counters were taken on; ``bench.py`` reports the
    traffic only while that code is unchanged.

    python -m exact_attention_123_amd.rocprof_summary --pass fwd \
        --workload bf16_b1h32_t8192_d128_causal_qk4 --name <kernel> \
        --flops F --alg-bytes A \
        --stats prof/kt/kt_kernel_stats.csv \
        --fetch prof/pmc_fetch/f_counter_collection.csv \
        --write prof/pmc_write/w_counter_collection.csv \
        --copy-mib 1024 --kt-cmd '...' --fetch-cmd '...' --write-cmd '...'
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
_CSRC = os.path.join(PKG, "csrc")
# the kernel code of each pass: its source and the headers it includes
SOURCES = {"fwd": [os.path.join(_CSRC, "attn_fwd.hip"), os.path.join(_CSRC, "rows.h"),
                   os.path.join(_CSRC, "tiles.h"), os.path.join(_CSRC, "fwd_cache.h")],
           "bwd": [os.path.join(_CSRC, "attn_bwd.hip"), os.path.join(_CSRC, "tiles.h")],
           "decode": [os.path.join(_CSRC, "attn_decode.hip"), os.path.join(_CSRC, "rows.h"),
                      os.path.join(_CSRC, "tiles.h"), os.path.join(_CSRC, "fwd_cache.h")],
           "mat": [os.path.join(_CSRC, "attn_materialized.hip"), os.path.join(_CSRC, "tiles.h")]}
# substring of the pass's kernel symbols
MARKS = {"fwd": "attn_fwd_", "bwd": "attn_bwd_", "decode": "attn_decode_", "mat": "attn_mat_"}
COPY_MARK = "copyBuffer"   # the runtime's device-to-device copy kernel


def code_sha(text: str) -> str:
    """SHA-256 (first 16 hex digits) of kernel source text with its ``//``
    comments and blank lines removed: a summary stays valid across edits of
    comments, and any change of code invalidates it."""
    lines = []
    for line in text.splitlines():
        code = re.sub(r"//.*", "", line).rstrip()
        if code.strip():
            lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def source_sha(pass_: str = "fwd") -> str:
    """code_sha of the pass's sources, each followed by the compiler options
    the library build gives that file alone (build.FILE_FLAGS), so that a
    change of those options also invalidates the pass's summaries."""
    from .build import FILE_FLAGS

    text = ""
    for path in SOURCES[pass_]:
        with open(path) as f:
            text += f.read() + "\n"
        flags = FILE_FLAGS.get(os.path.basename(path))
        if flags:
            text += "compiler options: " + " ".join(flags) + "\n"
    return code_sha(text)


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def kernel_stats(path: str, mark: str):
    """[(symbol, calls, avg_ns, min_ns, max_ns)] of the pass's kernels."""
    out = [(r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
            float(r["MaxNs"])) for r in _rows(path) if mark in r["Name"]]
    if not out:
        raise ValueError(f"no kernel matching {mark!r} in {path}")
    return out


def counter_per_call(path: str, counter: str, mark: str):
    """(KiB per call summed over the pass's kernels -- each kernel's mean per
    dispatch --, dispatches per kernel, KiB of the copy kernel)."""
    per, copy = {}, []
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        if mark in r["Kernel_Name"]:
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        elif COPY_MARK in r["Kernel_Name"]:
            copy.append(float(r["Counter_Value"]))
    if not per or not copy:
        raise ValueError(f"{path}: need {counter} for the pass's kernels and the copy kernel")
    return (sum(statistics.mean(v) for v in per.values()),
            min(len(v) for v in per.values()), copy[-1])


def counters_mean(path: str, mark: str):
    """{counter: value per call} summed over the pass's kernels (each
    kernel's mean per dispatch), and dispatches per kernel."""
    agg = {}
    for r in _rows(path):
        if mark in r["Kernel_Name"]:
            agg.setdefault((r["Counter_Name"], r["Kernel_Name"]), []).append(
                float(r["Counter_Value"]))
    out = {}
    for (cname, _), v in agg.items():
        out[cname] = out.get(cname, 0.0) + statistics.mean(v)
    return out, min(len(v) for v in agg.values())


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--pass", dest="pass_", choices=sorted(SOURCES), default="fwd")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--name", "--kernel", dest="name", required=True,
                    help="file name stem: the forward kernel's or the backward dK/dV "
                         "kernel's instance name")
    ap.add_argument("--flops", type=float, required=True, help="counted FLOPs per call")
    ap.add_argument("--alg-bytes", type=float, required=True,
                    help="algorithmic bytes per call (inputs read once, outputs written once)")
    ap.add_argument("--stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--kt-cmd", default="")
    ap.add_argument("--fetch-cmd", default="")
    ap.add_argument("--write-cmd", default="")
    ap.add_argument("--util", help="counter CSV of the MFMA utilisation pass")
    ap.add_argument("--util-cmd", default="")
    ap.add_argument("--counters", action="append", default=[],
                    help="counter CSV of another --pmc pass (repeatable)")
    ap.add_argument("--counters-cmd", action="append", default=[])
    ap.add_argument("--out", default=PROFILES)
    a = ap.parse_args()
    os.makedirs(a.out, exist_ok=True)
    mark = MARKS[a.pass_]
    sha = source_sha(a.pass_)
    base = os.path.join(a.out, f"{a.name}__{a.workload}")

    avg_call = None
    if a.stats:
        ks = kernel_stats(a.stats, mark)
        avg_call = sum(k[2] for k in ks)
        rows = "".join(f"| `{s}` | {c} | {av / 1e3:.1f} | {mn / 1e3:.1f} | {mx / 1e3:.1f} |\n"
                       for s, c, av, mn, mx in ks)
        with open(base + "__kernel_trace.md", "w") as f:
            f.write(f"# {a.name} on {a.workload}: rocprofv3 kernel trace\n\n"
                    f"command: `{a.kt_cmd}`\n\n"
                    f"kernel_code_sha256: {sha}\n\n"
                    f"| symbol | calls | avg us | min us | max us |\n"
                    f"|---|---|---|---|---|\n" + rows +
                    f"\nsum of averages (one call of the pass): {avg_call / 1e3:.1f} us\n\n"
                    f"TFLOP/s at that duration: {a.flops / (avg_call * 1e-9) / 1e12:.1f}\n")
        print("wrote", base + "__kernel_trace.md")

    if a.util:
        m, n = counters_mean(a.util, mark)
        xcd_cycles = m["GRBM_GUI_ACTIVE"] / 8  # the counter sums the 8 XCDs
        util = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd_cycles * 1024)
        other = (m["SQ_INSTS_VALU"] - m["SQ_INSTS_MFMA"]) / m["SQ_INSTS_MFMA"]
        clock = ""
        if avg_call:
            clock = (f"clock implied by GPU-active cycles over the traced average duration: "
                     f"{xcd_cycles / avg_call:.2f} GHz\n\n")
        with open(base + "__mfma_util.md", "w") as f:
            f.write(f"# {a.name} on {a.workload}: matrix-core utilisation\n\n"
                    f"command: `{a.util_cmd}`\n\n"
                    f"kernel_code_sha256: {sha}\n\n"
                    f"| counter | per call, summed over the pass's kernels ({n} calls) |\n"
                    f"|---|---|\n"
                    + "".join(f"| {k} | {v:.6g} |\n" for k, v in sorted(m.items()))
                    + f"\nMFMA busy fraction: {util:.3f}\n\n"
                    f"non-MFMA VALU instructions per MFMA: {other:.2f}\n\n" + clock)
        print("wrote", base + "__mfma_util.md")

    if a.counters:
        parts = []
        for i, path in enumerate(a.counters):
            m, n = counters_mean(path, mark)
            cmd = a.counters_cmd[i] if i < len(a.counters_cmd) else ""
            wc = m.get("SQ_WAVE_CYCLES")
            rows = "".join(
                f"| {k} | {v:.6g} | " + (f"{v / wc:.3f}" if wc else "") + " |\n"
                for k, v in sorted(m.items()))
            parts.append(f"command: `{cmd}`\n\n| counter | per call ({n} calls) | "
                         f"share of SQ_WAVE_CYCLES |\n|---|---|---|\n{rows}\n")
        with open(base + "__counters.md", "w") as f:
            f.write(f"# {a.name} on {a.workload}: SQ counters\n\n"
                    f"kernel_code_sha256: {sha}\n\n" + "".join(parts))
        print("wrote", base + "__counters.md")

    if a.fetch and a.write:
        copy_bytes = a.copy_mib * (1 << 20)
        fk, fn, fcopy = counter_per_call(a.fetch, "FETCH_SIZE", mark)
        wk, wn, wcopy = counter_per_call(a.write, "WRITE_SIZE", mark)
        ff = copy_bytes / (fcopy * 1024)  # bytes per counted byte
        wf = copy_bytes / (wcopy * 1024)
        fb, wb = fk * 1024 * ff, wk * 1024 * wf
        with open(base + "__traffic.md", "w") as f:
            f.write(f"# {a.name} on {a.workload}: device-memory traffic per call\n\n"
                    f"fetch command: `{a.fetch_cmd}`\n\n"
                    f"write command: `{a.write_cmd}`\n\n"
                    f"kernel_code_sha256: {sha}\n\n"
                    f"| counter | KiB per call (mean of {fn}/{wn}) | copy of {a.copy_mib} "
                    f"MiB reads as KiB | scale | bytes per call |\n|---|---|---|---|---|\n"
                    f"| FETCH_SIZE | {fk:.1f} | {fcopy:.1f} | {ff:.3f} | {fb:.4g} |\n"
                    f"| WRITE_SIZE | {wk:.1f} | {wcopy:.1f} | {wf:.3f} | {wb:.4g} |\n\n"
                    f"algorithmic bytes per call: {a.alg_bytes:.4g}\n\n"
                    f"hbm_bytes_per_launch: {fb + wb:.6g}\n\n"
                    f"ratio to algorithmic: {(fb + wb) / a.alg_bytes:.2f}\n")
        print("wrote", base + "__traffic.md")
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
