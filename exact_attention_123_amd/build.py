"""Build the HIP library ``libattn.so`` in-tree for gfx950.

    python -m exact_attention_123_amd.build

compiles ``csrc/attn_fwd.hip`` (forward), ``csrc/attn_bwd.hip`` (backward),
``csrc/attn_decode.hip`` (decode over a key/value cache),
``csrc/attn_materialized.hip`` (the unfused three-kernel forward),
``csrc/mfma_probe.hip`` (the matrix-core throughput probe) and
``csrc/device.hip`` (the host-side device checks they share) with hipcc into
``exact_attention_123_amd/libattn.so``, the same sources with
``-DATTN_DEBUG_BARRIERS`` into ``libattn_debug_barriers.so`` (race check),
and the plain C caller of the ABI used by a GPU test
(``tests/c_abi/libattn_c_caller.so``).
The library exports the C ABI of ``include/attn.h``; the Python binding loads
it with ctypes.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", n)
        for n in ("attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip", "attn_materialized.hip",
                  "mfma_probe.hip", "device.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
# The same library built with -DATTN_DEBUG_BARRIERS (extra workgroup barriers
# at every key/value tile, for the bitwise race check of the GPU tests).
DEBUG_LIB = os.path.join(PKG, "libattn_debug_barriers.so")

ARCH = "gfx950"
# Compiler options of single sources, on top of HIPCC_FLAGS (A/B in one
# process on MI355X at B H = 32, T = 8192, d = 128, causal; bit-identical
# outputs):
#  - the forward kernels are scheduled with LLVM's memory-clause strategy:
#    525.0 against 527.6 us per call (twice); the same strategy makes the
#    backward's dK/dV kernel spill (1899 against 1681 us), and the ILP
#    strategy is slower for both;
#  - the backward's scheduler uses the AMDGPU register-pressure trackers:
#    1649.5 against 1665.6 and 1686.4 against 1699.4 us per call (two
#    boxes); for the forward they change nothing measurable, nor does the
#    occupancy / latency bias of the scheduler for either.
FILE_FLAGS = {
    "attn_fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
    "attn_bwd.hip": ["-mllvm", "-amdgpu-use-amdgpu-trackers"],
}
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep hipcc from emitting packed fp32 VALU ops (v_pk_fma/mul/add_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # device code only: no NaN inputs are supported, so float max needs no
    # NaN-quieting (the host keeps IEEE semantics for argument validation)
    "-Xarch_device", "-fno-honor-nans",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd, verbose):
    """Start one hipcc command; returns the process."""
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _finish(proc, verbose):
    """Wait for a hipcc process; raises with its messages on failure."""
    out, _ = proc.communicate()
    # hipcc's host pass does not know the GPU-only target feature above and
    # says so; that line is expected and not shown.
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in out.splitlines() if noise not in ln]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)


def build(verbose: bool = False, out: str = LIB, debug_barriers: bool = False) -> str:
    """Compile the library (with debug_barriers: the race-check build);
    returns its path.  Each source is compiled to an object with its own
    FILE_FLAGS (in parallel), then the objects are linked.  Raises on
    compiler errors."""
    extra = ["-DATTN_DEBUG_BARRIERS"] if debug_barriers else []
    with tempfile.TemporaryDirectory(prefix="attn_build_") as tmpdir:
        objs, procs = [], []
        for src in SRCS:
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            flags = FILE_FLAGS.get(os.path.basename(src), [])
            cmd = [hipcc(), *HIPCC_FLAGS, *flags, *extra, "-I", INCLUDE, "-c", src, "-o", obj]
            objs.append(obj)
            procs.append(_run(cmd, verbose))
        for proc in procs:
            _finish(proc, verbose)
        tmp = out + ".tmp"
        _finish(_run([hipcc(), *HIPCC_FLAGS, *objs, "-o", tmp], verbose), verbose)
    os.replace(tmp, out)
    return out


# A plain C99 caller of the C ABI (tests/c_abi/c_caller.c), built next to its
# source and linked against libattn.so; a GPU test loads it.
C_CALLER_SRC = os.path.join(ROOT, "tests", "c_abi", "c_caller.c")
C_CALLER_LIB = os.path.join(ROOT, "tests", "c_abi", "libattn_c_caller.so")


def build_c_caller(verbose: bool = False) -> str:
    """Compile the C caller with the host C compiler (after build()); returns
    its path.  Raises on compiler errors."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler (gcc) found")
    tmp = C_CALLER_LIB + ".tmp"
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"), "-I", INCLUDE,
           C_CALLER_SRC, "-o", tmp, "-L", PKG, "-lattn", "-L", os.path.join(rocm, "lib"),
           "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN/../../exact_attention_123_amd"]
    _finish(_run(cmd, verbose), verbose)
    os.replace(tmp, C_CALLER_LIB)
    return C_CALLER_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build(verbose="-v" in sys.argv, out=DEBUG_LIB, debug_barriers=True))
    print(build_c_caller(verbose="-v" in sys.argv))
