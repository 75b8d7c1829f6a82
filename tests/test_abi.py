"""The C-ABI library on the host (CPU only): it loads, exports every function
include/attn.h declares, and rejects bad arguments before any HIP call.

No call here reaches a kernel launch: every argument set is invalid (or
empty), and validation returns before the library touches the HIP runtime.
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

import exact_attention_123_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ea.LIB_PATH),
                                reason="libattn.so not built")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# The argument sets below use fake device addresses and are all invalid, so
# validation rejects them before any launch.  They are still kept off
# machines with a GPU: a validation bug there would launch a kernel on fake
# addresses.
no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer checks run GPU-less")


def declared_functions():
    """Every function the headers under include/ declare."""
    names = set()
    for h in sorted(os.listdir(os.path.dirname(HEADER))):
        if h.endswith(".h"):
            text = open(os.path.join(os.path.dirname(HEADER), h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_exports():
    assert declared_functions() == sorted(ea.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ea.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ea.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (attn_\w+)", out))
    assert set(declared_functions()) <= exported


def test_status_strings_and_kernel_names():
    for code in range(9):
        assert ea.status_string(code)
    assert ea.status_string(99) == "unknown status"
    assert ea.kernel_name(False, 128, True).startswith("attn_fwd_bf16_d128_causal")
    assert ea.kernel_name(False, 64, False).startswith("attn_fwd_bf16_d64_full")
    assert ea.kernel_name(True, 64, True).startswith("attn_fwd_f32_d64_causal")
    assert ea.kernel_name(False, 96, True) is None


A = 0x10000  # 16-byte aligned fake addresses, never dereferenced


def call(fn, q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=1, T=8, d=64, causal=1,
         scale=0.125):
    return fn(q, k, v, o, lse, B, H, T, d, causal, scale)


@no_gpu_only
@pytest.mark.parametrize("fn", [ea.attn_fwd, ea.attn_fwd_f32], ids=["bf16", "f32"])
def test_validation_errors(fn):
    assert call(fn, q=0) == 1
    assert call(fn, lse=0) == 1
    assert call(fn, B=-1) == 2
    assert call(fn, T=-5) == 2
    assert call(fn, T=(1 << 30) + 1) == 2
    assert call(fn, B=1 << 20, H=1 << 20) == 2
    # one head of q (or k, v, o) must stay under 2 GiB
    assert call(fn, T=(1 << 31) // 256, d=128) == 2
    for d in (0, 32, 96, 127, 256):
        assert call(fn, d=d) == 3
    for s in (math.nan, math.inf, -math.inf):
        assert call(fn, scale=s) == 4
    assert call(fn, q=A + 2) == 5
    assert call(fn, o=4 * A + 8) == 5
    assert call(fn, lse=5 * A + 2) == 5
    assert call(fn, causal=2) == 6
    assert call(fn, causal=-1) == 6
    assert call(fn, o=A) == 6          # output aliases q
    assert call(fn, lse=4 * A) == 6    # lse overlaps o


@pytest.mark.parametrize("fn", [ea.attn_fwd, ea.attn_fwd_f32], ids=["bf16", "f32"])
def test_empty_problem_is_a_no_op(fn):
    for kw in (dict(B=0), dict(H=0), dict(T=0)):
        assert call(fn, q=0, k=0, v=0, o=0, lse=0, **kw) == 0


@no_gpu_only
def test_error_precedence_shape_before_pointers():
    # a negative size is reported even when pointers are also bad
    assert call(ea.attn_fwd, q=0, B=-1) == 2


def test_flops_convention():
    # 4*T^2*d per head, halved under a causal mask
    assert ea.flops(1, 32, 8192, 128, True) == pytest.approx(549.755813888e9)
    assert ea.flops(4, 16, 4096, 128, False) == pytest.approx(549.755813888e9)
    assert ea.flops(1, 1, 256, 64, True) == 2 * 256 * 256 * 64


def call_bwd(q=A, k=2 * A, v=3 * A, o=4 * A, do=5 * A, lse=6 * A, dq=7 * A, dk=8 * A,
             dv=9 * A, ws=10 * A, B=1, H=1, T=8, d=64, causal=1, scale=0.125):
    return ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, B, H, T, d, causal, scale)


@no_gpu_only
def test_bwd_validation_errors():
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws"):
        assert call_bwd(**{name: 0}) == 1, name
    assert call_bwd(B=-1) == 2
    assert call_bwd(T=(1 << 31) // 256, d=128) == 2
    for d in (0, 32, 96, 256):
        assert call_bwd(d=d) == 3
    for s in (math.nan, math.inf):
        assert call_bwd(scale=s) == 4
    assert call_bwd(dq=7 * A + 8) == 5
    assert call_bwd(do=5 * A + 4) == 5
    assert call_bwd(ws=10 * A + 2) == 5
    assert call_bwd(causal=3) == 6
    assert call_bwd(dq=A) == 6           # dq aliases q
    assert call_bwd(dk=9 * A) == 6       # dk aliases dv
    assert call_bwd(ws=6 * A) == 6       # ws overlaps lse


def test_bwd_empty_problem_is_a_no_op():
    for kw in (dict(B=0), dict(H=0), dict(T=0)):
        assert call_bwd(q=0, k=0, v=0, o=0, do=0, lse=0, dq=0, dk=0, dv=0, ws=0, **kw) == 0


def test_bwd_kernel_names_and_flops():
    assert ea.bwd_kernel_name(128, True, 1).startswith("attn_bwd_dkdv_bf16_d128_causal")
    assert ea.bwd_kernel_name(64, False, 2).startswith("attn_bwd_dq_bf16_d64_full")
    assert ea.bwd_kernel_name(128, True, 0) == "attn_bwd_prep_d128"
    assert ea.bwd_kernel_name(96, True, 1) is None
    assert ea.bwd_kernel_name(128, True, 3) is None
    # five T x T x d contractions: 2.5 times the forward
    assert ea.bwd_flops(1, 32, 8192, 128, True) == pytest.approx(2.5 * 549.755813888e9)


@no_gpu_only
def test_gqa_validation_errors():
    def fwd(**kw):
        a = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=8, Hkv=2, T=8, d=64,
                 causal=1, scale=0.125)
        a.update(kw)
        return ea.attn_fwd_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                               a["Hkv"], a["T"], a["d"], a["causal"], a["scale"])
    assert fwd(Hkv=3) == 2          # H not a multiple of H_kv
    assert fwd(Hkv=0) == 2
    assert fwd(Hkv=-1) == 2
    assert fwd(Hkv=16) == 2
    assert fwd(q=0) == 1
    assert fwd(d=96) == 3
    assert fwd(B=0, q=0, k=0, v=0, o=0, lse=0) == 0
    assert fwd(H=0, Hkv=0, q=0, k=0, v=0, o=0, lse=0) == 0

    def bwd(**kw):
        a = dict(B=1, H=8, Hkv=2, T=8, d=64)
        a.update(kw)
        return ea.attn_bwd_gqa(A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, 7 * A, 8 * A, 9 * A,
                               10 * A, a["B"], a["H"], a["Hkv"], a["T"], a["d"], 1, 0.125)
    assert bwd(Hkv=3) == 2
    assert bwd(Hkv=0) == 2
    assert bwd(d=32) == 3


@no_gpu_only
def test_decode_validation_errors():
    def dec(**kw):
        a = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, ws=6 * A, wsb=1 << 30, B=1, H=8,
                 Hkv=2, Tq=1, Tk=100, Tcap=100, d=128, causal=1, scale=0.1)
        a.update(kw)
        return ea.attn_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], a["wsb"],
                              a["B"], a["H"], a["Hkv"], a["Tq"], a["Tk"], a["Tcap"], a["d"],
                              a["causal"], a["scale"])
    assert dec(Hkv=3) == 2                 # H not a multiple of H_kv
    assert dec(Tk=0) == 2                  # a query needs a key
    assert dec(Tq=3, Tk=2, Tcap=2) == 2    # causal: the queries are cache positions
    assert dec(Tcap=50) == 2               # valid length beyond capacity
    assert dec(Tq=1 << 29, Tk=1 << 29, Tcap=1 << 29) == 2  # 2^31 rows per key/value head
    assert dec(d=96) == 3
    assert dec(q=0) == 1
    assert dec(causal=2) == 6
    assert dec(o=A) == 6
    assert dec(Tq=0) == 0                  # nothing to do
    # the split needs a workspace here
    assert ea.decode_workspace_bytes(1, 8, 2, 1, 100000, 128) > 0  # 25 splits
    far = dict(Tk=100000, Tcap=100000, q=1 << 36, k=2 << 36, v=3 << 36, o=4 << 36,
               lse=5 << 36)
    assert dec(ws=0, wsb=0, **far) == 9
    assert dec(ws=6 << 36, wsb=16, **far) == 9


@no_gpu_only
def test_decode_many_query_rows_pass_validation():
    # 4096 new queries x 4 query heads per key/value head: a prefill in
    # chunks; validation accepts it and only the device check (no GPU) stops
    # it
    r = ea.attn_decode(1 << 36, 2 << 36, 3 << 36, 4 << 36, 5 << 36, 6 << 36, 1 << 30, 1, 8, 2,
                       4096, 8192, 8192, 128, 1, 0.1)
    assert r == 7


def test_decode_split_sizes():
    # about 512 workgroups, each split at least 4096 keys
    assert ea.decode_splits(1, 32, 8, 1, 131072) == 32
    assert ea.decode_splits(16, 32, 8, 1, 32768) == 4
    assert ea.decode_splits(1, 1, 1, 1, 100) == 1
    assert ea.decode_splits(1, 8, 1, 2, 40000) == 10
    assert ea.decode_splits(2048, 32, 8, 1, 4096) == 1
    # 64 query rows per key/value head: two row chunks, half the splits
    assert ea.decode_splits(1, 32, 8, 1, 262144) == 64
    assert ea.decode_splits(1, 32, 8, 16, 262144) == 32
    assert ea.decode_workspace_bytes(2048, 32, 8, 1, 4096, 128) == 0
    # a prefill in chunks: 512 row chunks over the two key/value heads, one split
    assert ea.decode_splits(1, 8, 2, 2048, 8192) == 1
    assert ea.decode_workspace_bytes(1, 8, 2, 2048, 8192, 128) == 0
    assert ea.decode_workspace_bytes(1, 32, 8, 1, 131072, 128) == 32 * 32 * 129 * 4


@no_gpu_only
def test_materialized_validation_errors():
    def mat(**kw):
        a = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, s=1 << 36, p=2 << 36, B=1, H=1,
                 T=256, d=64, causal=1, scale=0.1)
        a.update(kw)
        return ea.attn_fwd_materialized(a["q"], a["k"], a["v"], a["o"], a["lse"], a["s"],
                                        a["p"], a["B"], a["H"], a["T"], a["d"], a["causal"],
                                        a["scale"])
    assert mat(T=200) == 3          # T must be a multiple of 128
    assert mat(T=65536) == 2        # a head's scores must stay under 4 GiB
    assert mat(d=96) == 3
    assert mat(s=0) == 1
    assert mat(p=A) == 6            # scratch overlaps q
    assert mat(T=0) == 0


def test_binding_buffer_checks():
    """The binding checks caller-supplied outputs and scratch buffers
    (shape, dtype, contiguity, device) before it passes their addresses to
    the C ABI, which cannot check sizes (CPU tensors stand in for device
    ones here)."""
    import torch
    cpu = torch.device("cpu")
    good = torch.empty((2, 3, 5, 64), dtype=torch.bfloat16)
    ea._check_buffer(good, "out", (2, 3, 5, 64), torch.bfloat16, cpu)
    with pytest.raises(ValueError, match="shape"):
        ea._check_buffer(good, "out", (2, 3, 6, 64), torch.bfloat16, cpu)
    with pytest.raises(ValueError, match="float32"):
        ea._check_buffer(good, "lse", (2, 3, 5, 64), torch.float32, cpu)
    with pytest.raises(ValueError, match="contiguous"):
        ea._check_buffer(good.transpose(2, 3).contiguous().transpose(2, 3), "out",
                         (2, 3, 5, 64), torch.bfloat16, cpu)
    with pytest.raises(ValueError, match="must be on"):
        ea._check_buffer(good.to("meta"), "s_buf", (2, 3, 5, 64), torch.bfloat16, cpu)
    with pytest.raises(ValueError, match="same device"):
        ea._check_same_device((good, good.to("meta")), "q, k")


def test_library_shares_torchs_hip_runtime():
    """Loading the library in a fresh process maps exactly one libamdhip64:
    torch's (the binding imports torch before it loads the library)."""
    code = ("import re, sys; sys.path.insert(0, %r); import exact_attention_123_amd as ea; "
            "ea.load_library(); maps = open('/proc/self/maps').read(); "
            "print(sorted(set(re.findall(r'/\\S*libamdhip64\\S*', maps))))" % ROOT)
    out = subprocess.run([__import__("sys").executable, "-c", code], capture_output=True,
                         text=True, check=True, timeout=300).stdout.strip()
    libs = eval(out)
    assert len(libs) == 1 and "/torch/lib/" in libs[0], libs


@no_gpu_only
def test_decode_noalloc_validation_errors():
    """The allocation-free decode validates like attn_decode and rejects a
    problem whose split results exceed its device scratch before any HIP
    call."""
    def dec(**kw):
        a = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=8, Hkv=2, Tq=1, Tk=100,
                 Tcap=100, d=128, causal=1, scale=0.1)
        a.update(kw)
        return ea.attn_decode_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                                      a["H"], a["Hkv"], a["Tq"], a["Tk"], a["Tcap"], a["d"],
                                      a["causal"], a["scale"])
    assert dec(Hkv=3) == 2
    assert dec(d=96) == 3
    assert dec(q=0) == 1
    assert dec(causal=2) == 6
    assert dec(Tq=0) == 0
    # 300 heads x 32 queries, 2 splits: 2 * 9600 rows * 129 * 4 B = 9.9 MB > 8 MiB
    big = dict(B=1, H=300, Hkv=300, Tq=32, Tk=8192, Tcap=8192, q=1 << 36, k=2 << 36,
               v=3 << 36, o=4 << 36, lse=5 << 36)
    assert ea.decode_workspace_bytes(1, 300, 300, 32, 8192, 128) > ea.DECODE_NOALLOC_MAX_BYTES
    assert dec(**big) == 9
    header = open(HEADER).read()
    assert re.search(r"#define ATTN_DECODE_NOALLOC_MAX_BYTES \(8 << 20\)", header)
    assert ea.DECODE_NOALLOC_MAX_BYTES == 8 << 20


def test_debug_barriers_build_exports_the_same_symbols():
    """The race-check build (-DATTN_DEBUG_BARRIERS) exists next to the
    library and exports every declared function."""
    path = os.path.join(os.path.dirname(ea.LIB_PATH), "libattn_debug_barriers.so")
    assert os.path.exists(path), "build() compiles the race-check library too"
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (attn_\w+)", out))
    assert set(declared_functions()) <= exported


@no_gpu_only
def test_probe_validation_and_flop_count():
    assert ea.load_library().attn_probe_mfma(2, 1, 1, A, None) == 6
    assert ea.load_library().attn_probe_mfma(0, 0, 1, A, None) == 2
    assert ea.load_library().attn_probe_mfma(0, 1, 0, A, None) == 2
    assert ea.load_library().attn_probe_mfma(0, 1, 1, None, None) == 1
    assert ea.load_library().attn_probe_mfma(0, 1, 1, A + 2, None) == 5
    f = ea.load_library().attn_probe_mfma_flops
    # 4 waves x iters x (16 MFMAs of 32x32x16 | 32 of 16x16x32) x 2 m n k
    assert f(0, 3, 10) == 3 * 4 * 10 * 16 * 2 * 32 * 32 * 16
    assert f(1, 3, 10) == 3 * 4 * 10 * 32 * 2 * 16 * 16 * 32
    assert f(5, 3, 10) == 0.0


def test_c_caller_built():
    """The plain C caller of the ABI (tests/c_abi/c_caller.c) is built by the
    library build and runs its checks or, without a GPU, reports the HIP call
    that failed (no crash)."""
    from exact_attention_123_amd.build import C_CALLER_LIB
    assert os.path.exists(C_CALLER_LIB), "build it with python -m exact_attention_123_amd.build"
    lib = ctypes.CDLL(C_CALLER_LIB)
    lib.attn_c_caller_check.restype = ctypes.c_int
    lib.attn_c_caller_check.argtypes = [ctypes.c_char_p, ctypes.c_int]
    msg = ctypes.create_string_buffer(256)
    rc = lib.attn_c_caller_check(msg, len(msg))
    text = msg.value.decode()
    assert (rc == 0 and "passed" in text) or (rc != 0 and "failed" in text), (rc, text)
