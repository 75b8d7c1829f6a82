"""Python binding of the fused exact-attention forward for MI355X (gfx950).

The computation runs entirely in the HIP library ``libattn.so`` (C ABI in
``include/attn.h``); this module only marshals arguments.  PyTorch provides
device memory and the current stream.

    from exact_attention_123_amd import forward
    o, lse = forward(q, k, v, causal=True)        # q, k, v: [B, H, T, d] on cuda

The raw entry points ``attn_fwd`` / ``attn_fwd_f32`` take integer device
addresses and sizes exactly as the C functions do.  If the library has not
been built, importing works but every call raises ``LibraryNotBuilt``: there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "forward", "backward", "attn_fwd", "attn_fwd_f32", "attn_bwd", "attn_fwd_gqa",
    "attn_bwd_gqa", "attn_decode", "attn_decode_noalloc", "DECODE_NOALLOC_MAX_BYTES", "decode",
    "decode_workspace_bytes", "decode_splits",
    "attn_fwd_materialized", "forward_materialized",
    "kernel_name", "fwd_kernel_name_for", "fwd_f32_kernel_name_for", "decode_kernel_name_for",
    "bwd_kernel_name", "bwd_kernel_name_for", "status_string", "AttnError", "LibraryNotBuilt", "load_library",
    "LIB_PATH", "STATUS", "flops", "bwd_flops",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_SCALE", 5: "ATTN_ERR_ALIGN", 6: "ATTN_ERR_ARG", 7: "ATTN_ERR_DEVICE",
    8: "ATTN_ERR_LAUNCH", 9: "ATTN_ERR_WORKSPACE",
}

# The C prototypes from include/attn.h and include/attn_probe.h.
EXPORTS = {
    "attn_fwd": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4
                 + [ctypes.c_int, ctypes.c_float, ctypes.c_void_p]),
    "attn_fwd_f32": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4
                     + [ctypes.c_int, ctypes.c_float, ctypes.c_void_p]),
    "attn_bwd": (ctypes.c_int, [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 4
                 + [ctypes.c_int, ctypes.c_float, ctypes.c_void_p]),
    "attn_fwd_gqa": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5
                     + [ctypes.c_int, ctypes.c_float, ctypes.c_void_p]),
    "attn_bwd_gqa": (ctypes.c_int, [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 5
                     + [ctypes.c_int, ctypes.c_float, ctypes.c_void_p]),
    "attn_decode": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int64] * 8
                    + [ctypes.c_int, ctypes.c_float, ctypes.c_void_p]),
    "attn_decode_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 7
                            + [ctypes.c_int, ctypes.c_float, ctypes.c_void_p]),
    "attn_decode_workspace_bytes": (ctypes.c_int64, [ctypes.c_int64] * 6),
    "attn_decode_splits": (ctypes.c_int64, [ctypes.c_int64] * 5),
    "attn_fwd_materialized": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 4
                              + [ctypes.c_int, ctypes.c_float, ctypes.c_void_p]),
    "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_kernel_name": (ctypes.c_char_p, [ctypes.c_int, ctypes.c_int64, ctypes.c_int]),
    "attn_fwd_kernel_name_for": (ctypes.c_char_p, [ctypes.c_int64] * 4 + [ctypes.c_int]),
    "attn_fwd_f32_kernel_name_for": (ctypes.c_char_p, [ctypes.c_int64] * 4 + [ctypes.c_int]),
    "attn_bwd_kernel_name": (ctypes.c_char_p, [ctypes.c_int64, ctypes.c_int, ctypes.c_int]),
    "attn_bwd_kernel_name_for": (ctypes.c_char_p, [ctypes.c_int64] * 5 + [ctypes.c_int] * 2),
    "attn_decode_kernel_name_for": (ctypes.c_char_p, [ctypes.c_int64] * 6 + [ctypes.c_int]),
    # include/attn_probe.h
    "attn_probe_mfma": (ctypes.c_int, [ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_void_p]),
    "attn_probe_mfma_flops": (ctypes.c_double, [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]),
}


class LibraryNotBuilt(RuntimeError):
    pass


class AttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so once and attach the prototypes."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise LibraryNotBuilt(
            f"{path} is missing; build it with `python -m exact_attention_123_amd.build`")
    # One HIP runtime per process: torch ships its own libamdhip64 with the
    # same soname as the system one the library links, and whichever loads
    # first serves both.  Loading the library first would bind torch to the
    # system runtime, and torch's device initialisation then fails; so torch
    # loads first, and the library shares torch's runtime (and its streams).
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - torch is part of the environment
        pass
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().attn_status_string(code).decode()


def kernel_name(is_f32: bool, d: int, causal: bool):
    n = load_library().attn_kernel_name(int(bool(is_f32)), int(d), int(bool(causal)))
    return None if n is None else n.decode()


def fwd_kernel_name_for(B: int, H: int, T: int, d: int, causal: bool):
    """The bf16 forward instance attn_fwd launches for these sizes on the
    current device (needs a GPU)."""
    n = load_library().attn_fwd_kernel_name_for(B, H, T, d, int(bool(causal)))
    return None if n is None else n.decode()


def fwd_f32_kernel_name_for(B: int, H: int, T: int, d: int, causal: bool):
    """The fp32 forward instance attn_fwd_f32 launches for these sizes on
    the current device (needs a GPU)."""
    n = load_library().attn_fwd_f32_kernel_name_for(B, H, T, d, int(bool(causal)))
    return None if n is None else n.decode()


def decode_kernel_name_for(B: int, H: int, H_kv: int, Tq: int, Tk: int, d: int, causal: bool):
    """The kernel attn_decode launches first for these sizes on the current
    device: the split-key decode kernel or the forward instance that runs
    over the cache (needs a GPU)."""
    n = load_library().attn_decode_kernel_name_for(B, H, H_kv, Tq, Tk, d, int(bool(causal)))
    return None if n is None else n.decode()


def bwd_kernel_name(d: int, causal: bool, which: int):
    """Name of backward kernel ``which`` (0 row statistics, 1 dK/dV, 2 dQ)."""
    n = load_library().attn_bwd_kernel_name(int(d), int(bool(causal)), int(which))
    return None if n is None else n.decode()


def bwd_kernel_name_for(B: int, H: int, H_kv: int, T: int, d: int, causal: bool, which: int):
    """Name of backward kernel ``which`` that attn_bwd_gqa launches for these
    sizes on the current device (needs a GPU)."""
    n = load_library().attn_bwd_kernel_name_for(B, H, H_kv, T, d, int(bool(causal)), int(which))
    return None if n is None else n.decode()


def attn_fwd(q, k, v, o, lse, B, H, T, d, causal, scale, stream=0) -> int:
    """Raw bf16 entry point: integer device addresses, returns the status."""
    return load_library().attn_fwd(q, k, v, o, lse, B, H, T, d, int(causal), float(scale),
                                   stream or None)


def attn_fwd_f32(q, k, v, o, lse, B, H, T, d, causal, scale, stream=0) -> int:
    """Raw fp32 entry point: integer device addresses, returns the status."""
    return load_library().attn_fwd_f32(q, k, v, o, lse, B, H, T, d, int(causal),
                                       float(scale), stream or None)


def attn_fwd_gqa(q, k, v, o, lse, B, H, H_kv, T, d, causal, scale, stream=0) -> int:
    """Raw grouped-query bf16 forward: integer device addresses."""
    return load_library().attn_fwd_gqa(q, k, v, o, lse, B, H, H_kv, T, d, int(causal),
                                       float(scale), stream or None)


def attn_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, H_kv, T, d, causal, scale,
                 stream=0) -> int:
    """Raw grouped-query bf16 backward: integer device addresses."""
    return load_library().attn_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, H_kv, T, d,
                                       int(causal), float(scale), stream or None)


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, T, d, causal, scale,
             stream=0) -> int:
    """Raw bf16 backward entry point: integer device addresses, returns the
    status."""
    return load_library().attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, T, d,
                                   int(causal), float(scale), stream or None)


def attn_decode(q, k, v, o, lse, ws, ws_bytes, B, H, H_kv, Tq, Tk, Tk_cap, d, causal, scale,
                stream=0) -> int:
    """Raw decode entry point: integer device addresses, returns the status."""
    return load_library().attn_decode(q, k, v, o, lse, ws or None, ws_bytes, B, H, H_kv, Tq, Tk,
                                      Tk_cap, d, int(causal), float(scale), stream or None)


def attn_decode_noalloc(q, k, v, o, lse, B, H, H_kv, Tq, Tk, Tk_cap, d, causal, scale,
                        stream=0) -> int:
    """Raw decode entry point that allocates nothing (the library's own
    device scratch of DECODE_NOALLOC_MAX_BYTES holds the split results):
    integer device addresses, returns the status."""
    return load_library().attn_decode_noalloc(q, k, v, o, lse, B, H, H_kv, Tq, Tk, Tk_cap, d,
                                              int(causal), float(scale), stream or None)


# Size of the device scratch of attn_decode_noalloc (ATTN_DECODE_NOALLOC_MAX_BYTES).
DECODE_NOALLOC_MAX_BYTES = 8 << 20


def decode_workspace_bytes(B: int, H: int, H_kv: int, Tq: int, Tk: int, d: int) -> int:
    return int(load_library().attn_decode_workspace_bytes(B, H, H_kv, Tq, Tk, d))


def decode_splits(B: int, H: int, H_kv: int, Tq: int, Tk: int) -> int:
    return int(load_library().attn_decode_splits(B, H, H_kv, Tq, Tk))


def attn_fwd_materialized(q, k, v, o, lse, s_buf, p_buf, B, H, T, d, causal, scale,
                          stream=0) -> int:
    """Raw materialised (three-kernel) forward: integer device addresses."""
    return load_library().attn_fwd_materialized(q, k, v, o, lse, s_buf, p_buf, B, H, T, d,
                                                int(causal), float(scale), stream or None)


def _check_buffer(t, name: str, shape, dtype, device) -> None:
    """A caller-supplied output or scratch tensor must match exactly: the C
    ABI receives only its address and cannot check its size."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be a {dtype} tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _check_same_device(ts, names: str) -> None:
    dev = ts[0].device
    if any(t.device != dev for t in ts):
        raise ValueError(f"{names} must all be on the same device")


_raw_stream = None
_get_device = None


def _launch(dev, stream, entry, *args) -> int:
    """Calls the raw entry point ``entry(*args, stream_handle)`` with ``dev``
    as the current device (the library launches on the current device) and
    the handle of ``stream``, else of dev's current stream.  The handle and
    the current device are read through torch's direct accessors where it
    has them (a few hundred ns, against microseconds for a Stream object and
    a device guard), so that the host keeps ahead of kernels of tens of
    microseconds."""
    global _raw_stream, _get_device
    import torch

    if _raw_stream is None:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream",
                              lambda i: torch.cuda.current_stream(i).cuda_stream)
        _get_device = getattr(torch._C, "_cuda_getDevice", torch.cuda.current_device)
    idx = dev.index
    s = stream.cuda_stream if stream is not None else _raw_stream(idx)
    if _get_device() == idx:
        return entry(*args, s)
    with torch.cuda.device(dev):
        return entry(*args, s)


def flops(B: int, H: int, T: int, d: int, causal: bool) -> float:
    """Counted FLOPs of one forward: the two T x T x d contractions,
    4*T*T*d per head, halved under a causal mask."""
    f = 4.0 * B * H * T * T * d
    return f / 2 if causal else f


def bwd_flops(B: int, H: int, T: int, d: int, causal: bool) -> float:
    """Counted FLOPs of one backward: the five T x T x d contractions of the
    gradient (S recomputed, dP, dV, dQ, dK), 2.5 times the forward's.  The
    kernels recompute S and dP once more for dQ; that work is not counted."""
    return 2.5 * flops(B, H, T, d, causal)


def forward(q, k, v, causal: bool = True, scale: float | None = None, out=None, lse=None,
            stream=None):
    """Fused attention forward on torch tensors (bf16 or fp32).

    q: [B, H, T, d]; k, v: [B, H_kv, T, d] with H_kv dividing H (grouped
    query heads, bf16 only, when H_kv < H).  Returns (o, lse): o has q's
    dtype and shape; lse is float32 [B, H, T].  Runs on ``stream`` (a
    torch.cuda.Stream) or the current stream.
    """
    import torch

    if q.dim() != 4 or k.shape != v.shape or k.dim() != 4:
        raise ValueError("q must be [B, H, T, d] and k, v [B, H_kv, T, d]")
    B, H, T, d = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2:] != q.shape[2:] or Hkv < 1 or H % Hkv:
        raise ValueError("k, v must be [B, H_kv, T, d] with H_kv dividing H")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    if q.dtype == torch.float32 and Hkv != H:
        raise ValueError("grouped key/value heads are supported in bfloat16 only")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous CUDA tensors")
    _check_same_device((q, k, v), "q, k, v")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    _check_buffer(out, "out", q.shape, q.dtype, q.device)
    _check_buffer(lse, "lse", (B, H, T), torch.float32, q.device)
    if q.dtype == torch.float32:
        st = _launch(q.device, stream, attn_fwd_f32, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                     out.data_ptr(), lse.data_ptr(), B, H, T, d, causal, scale)
    else:
        st = _launch(q.device, stream, attn_fwd_gqa, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                     out.data_ptr(), lse.data_ptr(), B, H, Hkv, T, d, causal, scale)
    if st != 0:
        raise AttnError(st, status_string(st))
    return out, lse


def backward(q, k, v, o, lse, dout, causal: bool = True, scale: float | None = None,
             dq=None, dk=None, dv=None, ws=None, stream=None):
    """Gradients of the attention forward on bf16 torch tensors.

    q, o, dout: [B, H, T, d]; k, v: [B, H_kv, T, d] (H_kv dividing H).  ``o``
    and ``lse`` are what :func:`forward` returned for the same q, k, v,
    causal and scale; ``dout`` is the gradient of o.  Returns (dq, dk, dv)
    shaped like q, k, v.  ``ws`` is an optional float32 workspace of 2*B*H*T
    elements (allocated when None); after the call it holds -Delta, then
    -lse/scale (-lse*log2(e) when |scale| < 2^-32), each [B, H, T].
    """
    import torch

    if q.dim() != 4 or o.shape != q.shape or dout.shape != q.shape or k.shape != v.shape:
        raise ValueError("q, o, dout must be [B, H, T, d] and k, v [B, H_kv, T, d]")
    B, H, T, d = q.shape
    Hkv = k.shape[1]
    if k.dim() != 4 or k.shape[0] != B or k.shape[2:] != q.shape[2:] or Hkv < 1 or H % Hkv:
        raise ValueError("k, v must be [B, H_kv, T, d] with H_kv dividing H")
    ts = (q, k, v, o, dout)
    if any(t.dtype != torch.bfloat16 for t in ts):
        raise ValueError("the backward takes bfloat16 q, k, v, o, dout")
    for t in ts + (lse,):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous CUDA tensors")
    _check_same_device(ts + (lse,), "q, k, v, o, dout, lse")
    if lse.shape != (B, H, T) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [B, H, T] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if ws is None:
        ws = torch.empty(2 * B * H * T, dtype=torch.float32, device=q.device)
    for t, like, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _check_buffer(t, name, like.shape, torch.bfloat16, q.device)
    if ws.numel() < 2 * B * H * T or ws.dtype != torch.float32 or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous float32 tensor of 2*B*H*T elements")
    if ws.device != q.device:
        raise ValueError(f"ws must be on {q.device}")
    st = _launch(q.device, stream, attn_bwd_gqa, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                 o.data_ptr(), dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                 dv.data_ptr(), ws.data_ptr(), B, H, Hkv, T, d, causal, scale)
    if st != 0:
        raise AttnError(st, status_string(st))
    return dq, dk, dv


def decode(q, k_cache, v_cache, Tk: int | None = None, causal: bool = True,
           scale: float | None = None, out=None, lse=None, ws=None, stream=None):
    """Decode on bf16 torch tensors: q [B, H, Tq, d] (the last Tq positions),
    k_cache, v_cache [B, H_kv, Tk_cap, d] with the first ``Tk`` rows valid
    (default all).  Returns (o [B, H, Tq, d] bf16, lse [B, H, Tq] float32).
    ``ws`` is an optional uint8/any-dtype device buffer of at least
    decode_workspace_bytes(...) bytes (allocated when None and needed)."""
    import torch

    if q.dim() != 4 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B, H, Tq, d] and the caches [B, H_kv, Tk_cap, d]")
    B, H, Tq, d = q.shape
    Hkv, Tcap = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError("cache batch and head dimension must match q")
    if any(t.dtype != torch.bfloat16 for t in (q, k_cache, v_cache)):
        raise ValueError("decode takes bfloat16 tensors")
    for t in (q, k_cache, v_cache):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q and the caches must be contiguous CUDA tensors")
    _check_same_device((q, k_cache, v_cache), "q, k_cache, v_cache")
    Tk = Tcap if Tk is None else int(Tk)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_buffer(out, "out", q.shape, torch.bfloat16, q.device)
    _check_buffer(lse, "lse", (B, H, Tq), torch.float32, q.device)
    need = decode_workspace_bytes(B, H, Hkv, Tq, Tk, d) if Hkv and Tk else 0
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    if ws is not None and (not ws.is_contiguous() or ws.device != q.device):
        raise ValueError(f"ws must be a contiguous tensor on {q.device}")
    ws_ptr = ws.data_ptr() if ws is not None else 0
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    st = _launch(q.device, stream, attn_decode, q.data_ptr(), k_cache.data_ptr(),
                 v_cache.data_ptr(), out.data_ptr(), lse.data_ptr(), ws_ptr, ws_bytes, B, H, Hkv,
                 Tq, Tk, Tcap, d, causal, scale)
    if st != 0:
        raise AttnError(st, status_string(st))
    return out, lse


def forward_materialized(q, k, v, causal: bool = True, scale: float | None = None, out=None,
                         lse=None, s_buf=None, p_buf=None, stream=None):
    """The unfused three-kernel forward on bf16 tensors [B, H, T, d] (T a
    multiple of 128): S (fp32) and P (bf16) go through device memory.
    Returns (o, lse) like :func:`forward`."""
    import torch

    if q.dim() != 4 or not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must all have shape [B, H, T, d]")
    if any(t.dtype != torch.bfloat16 for t in (q, k, v)):
        raise ValueError("the materialised forward takes bfloat16 tensors")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous CUDA tensors")
    _check_same_device((q, k, v), "q, k, v")
    B, H, T, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if lse is None else lse
    if s_buf is None:
        s_buf = torch.empty((B, H, T, T), dtype=torch.float32, device=q.device)
    if p_buf is None:
        p_buf = torch.empty((B, H, T, T), dtype=torch.bfloat16, device=q.device)
    _check_buffer(out, "out", q.shape, torch.bfloat16, q.device)
    _check_buffer(lse, "lse", (B, H, T), torch.float32, q.device)
    _check_buffer(s_buf, "s_buf", (B, H, T, T), torch.float32, q.device)
    _check_buffer(p_buf, "p_buf", (B, H, T, T), torch.bfloat16, q.device)
    st = _launch(q.device, stream, attn_fwd_materialized, q.data_ptr(), k.data_ptr(),
                 v.data_ptr(), out.data_ptr(), lse.data_ptr(), s_buf.data_ptr(),
                 p_buf.data_ptr(), B, H, T, d, causal, scale)
    if st != 0:
        raise AttnError(st, status_string(st))
    return out, lse
