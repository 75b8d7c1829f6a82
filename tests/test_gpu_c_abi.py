"""The C ABI from plain C on the GPU: tests/c_abi/c_caller.c (built into
tests/c_abi/libattn_c_caller.so by the library build) allocates its buffers
with hipMalloc, calls attn_fwd and attn_decode on the default stream and
checks the results against closed forms (Q = 0: every score equal, O the
mean of the visible V rows, LSE = ln of their count), with no Python
between it and the library.  The test loads it in this process and runs
its checks."""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "libattn_c_caller.so")


def test_c_caller():
    import exact_attention_123_amd as ea
    ea.load_library()  # torch's HIP runtime first, then the attention library
    assert os.path.exists(LIB), f"{LIB} missing: python -m exact_attention_123_amd.build"
    lib = ctypes.CDLL(LIB)
    lib.attn_c_caller_check.restype = ctypes.c_int
    lib.attn_c_caller_check.argtypes = [ctypes.c_char_p, ctypes.c_int]
    msg = ctypes.create_string_buffer(512)
    rc = lib.attn_c_caller_check(msg, len(msg))
    print(f"[c caller] rc={rc}: {msg.value.decode()}", flush=True)
    assert rc == 0, msg.value.decode()
