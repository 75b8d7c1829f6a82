"""Turn rocprofv3 CSV output into the short text summaries kept under
``profiles/``.

Two summaries per (kernel, workload):

``<kernel>__<workload>__kernel_trace.md``
    calls, average / min / max duration of the attention kernel from a
    ``rocprofv3 --kernel-trace --stats`` run of ``bench.py``, and the
    TFLOP/s that average implies.

``<kernel>__<workload>__mfma_util.md``
    matrix-core busy fraction from one ``rocprofv3 --pmc`` run of
    ``SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_INSTS_MFMA``:
    busy SIMD-cycles over (GPU-active cycles per XCD x 1024 SIMDs), and the
    clock that GPU-active cycles over the traced average duration imply.

``<kernel>__<workload>__traffic.md``
    device-memory bytes per launch from two ``rocprofv3 --pmc`` runs
    (``FETCH_SIZE``, then ``WRITE_SIZE``), each scaled by what the same
    counter reads for a plain device-to-device copy of known size
    (``bench.py --copy-calibration-mib N`` launches it after the timed
    region).  It records the SHA-256 of the kernel source the counters were
    taken on; ``bench.py`` reports the traffic only while that source is
    unchanged.

    python -m exact_attention_123_amd.rocprof_summary \
        --workload bf16_b1h32_t8192_d128_causal_qk4 \
        --stats gpurun_out/kt/kt_kernel_stats.csv \
        --fetch gpurun_out/pmc_fetch/f_counter_collection.csv \
        --write gpurun_out/pmc_write/w_counter_collection.csv \
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
KERNEL_SRC = os.path.join(PKG, "csrc", "attn_fwd.hip")
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_MARK = "attn_fwd_"  # substring of every attention kernel's symbol
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


def source_sha() -> str:
    with open(KERNEL_SRC) as f:
        return code_sha(f.read())


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def kernel_stats(path: str):
    """(symbol, calls, avg_ns, min_ns, max_ns) of the attention kernel."""
    for r in _rows(path):
        if KERNEL_MARK in r["Name"]:
            return (r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                    float(r["MaxNs"]))
    raise ValueError(f"no attention kernel in {path}")


def counter_per_dispatch(path: str, counter: str):
    """(mean KiB per attention dispatch, dispatches, KiB of the copy kernel)."""
    att, copy = [], []
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        if KERNEL_MARK in r["Kernel_Name"]:
            att.append(float(r["Counter_Value"]))
        elif COPY_MARK in r["Kernel_Name"]:
            copy.append(float(r["Counter_Value"]))
    if not att or not copy:
        raise ValueError(f"{path}: need {counter} for the attention and the copy kernel")
    return statistics.mean(att), len(att), copy[-1]


def counters_mean(path: str):
    """{counter: mean value per attention dispatch} of a counter CSV."""
    agg = {}
    for r in _rows(path):
        if KERNEL_MARK in r["Kernel_Name"]:
            agg.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: statistics.mean(v) for k, v in agg.items()}, max(len(v) for v in agg.values())


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--kernel", required=True, help="instance name (attn_kernel_name)")
    ap.add_argument("--flops", type=float, required=True, help="counted FLOPs per launch")
    ap.add_argument("--alg-bytes", type=float, required=True,
                    help="algorithmic bytes per launch (Q, K, V read, O, LSE written)")
    ap.add_argument("--stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--kt-cmd", default="")
    ap.add_argument("--fetch-cmd", default="")
    ap.add_argument("--write-cmd", default="")
    ap.add_argument("--util", help="counter CSV of the MFMA utilisation pass")
    ap.add_argument("--util-cmd", default="")
    ap.add_argument("--out", default=PROFILES)
    a = ap.parse_args()
    os.makedirs(a.out, exist_ok=True)
    sha = source_sha()
    base = os.path.join(a.out, f"{a.kernel}__{a.workload}")

    if a.stats:
        sym, calls, avg, mn, mx = kernel_stats(a.stats)
        with open(base + "__kernel_trace.md", "w") as f:
            f.write(f"# {a.kernel} on {a.workload}: rocprofv3 kernel trace\n\n"
                    f"command: `{a.kt_cmd}`\n\n"
                    f"kernel_code_sha256: {sha}\n\n"
                    f"| symbol | calls | avg us | min us | max us | TFLOP/s at avg |\n"
                    f"|---|---|---|---|---|---|\n"
                    f"| `{sym}` | {calls} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | "
                    f"{mx / 1e3:.1f} | {a.flops / (avg * 1e-9) / 1e12:.1f} |\n")
        print("wrote", base + "__kernel_trace.md")

    if a.util:
        m, n = counters_mean(a.util)
        xcd_cycles = m["GRBM_GUI_ACTIVE"] / 8  # the counter sums the 8 XCDs
        util = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd_cycles * 1024)
        other = (m["SQ_INSTS_VALU"] - m["SQ_INSTS_MFMA"]) / m["SQ_INSTS_MFMA"]
        clock = ""
        if a.stats:
            clock = (f"clock implied by GPU-active cycles over the traced average duration: "
                     f"{xcd_cycles / avg:.2f} GHz\n\n")
        with open(base + "__mfma_util.md", "w") as f:
            f.write(f"# {a.kernel} on {a.workload}: matrix-core utilisation\n\n"
                    f"command: `{a.util_cmd}`\n\n"
                    f"kernel_code_sha256: {sha}\n\n"
                    f"| counter | mean per dispatch ({n}) |\n|---|---|\n"
                    + "".join(f"| {k} | {v:.6g} |\n" for k, v in sorted(m.items()))
                    + f"\nMFMA busy fraction: {util:.3f}\n\n"
                    f"non-MFMA VALU instructions per MFMA: {other:.2f}\n\n" + clock)
        print("wrote", base + "__mfma_util.md")

    if a.fetch and a.write:
        copy_bytes = a.copy_mib * (1 << 20)
        fk, fn, fcopy = counter_per_dispatch(a.fetch, "FETCH_SIZE")
        wk, wn, wcopy = counter_per_dispatch(a.write, "WRITE_SIZE")
        ff = copy_bytes / (fcopy * 1024)  # bytes per counted byte
        wf = copy_bytes / (wcopy * 1024)
        fb, wb = fk * 1024 * ff, wk * 1024 * wf
        with open(base + "__traffic.md", "w") as f:
            f.write(f"# {a.kernel} on {a.workload}: device-memory traffic per launch\n\n"
                    f"fetch command: `{a.fetch_cmd}`\n\n"
                    f"write command: `{a.write_cmd}`\n\n"
                    f"kernel_code_sha256: {sha}\n\n"
                    f"| counter | KiB per dispatch (mean of {fn}/{wn}) | copy of {a.copy_mib} "
                    f"MiB reads as KiB | scale | bytes per launch |\n|---|---|---|---|---|\n"
                    f"| FETCH_SIZE | {fk:.1f} | {fcopy:.1f} | {ff:.3f} | {fb:.4g} |\n"
                    f"| WRITE_SIZE | {wk:.1f} | {wcopy:.1f} | {wf:.3f} | {wb:.4g} |\n\n"
                    f"algorithmic bytes per launch: {a.alg_bytes:.4g}\n\n"
                    f"hbm_bytes_per_launch: {fb + wb:.6g}\n\n"
                    f"ratio to algorithmic: {(fb + wb) / a.alg_bytes:.2f}\n")
        print("wrote", base + "__traffic.md")
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
