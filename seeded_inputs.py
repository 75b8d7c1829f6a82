"""Seeded synthetic inputs for the attention forward: the only module that the
GPU path's tests and the CPU oracle's tests both use.

It holds no attention arithmetic.  It draws Q, K and V from a seeded numpy
generator (PCG64), rounds them to the storage type the kernel
reads (bfloat16, round-to-nearest-even, written from the IEEE-754 bit layout,
or float32 as drawn) and hands out two views of the same numbers: the raw
storage (what is uploaded to the device) and an exact float64 upcast (what the
oracle reads).  Both sides therefore see bit-identical inputs.

Workloads (shapes, dtypes, value distributions) follow the single-head and
multi-head settings of exact attention with a per-head T x d layout; see
``WORKLOADS``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "QKV",
    "make_qkv",
    "WORKLOADS",
    "sample_rows",
    "make_workload",
    "make_dout",
    "make_decode",
    "DECODE_WORKLOADS",
]


# ---------------------------------------------------------------------------
# bfloat16 storage: the upper 16 bits of an IEEE-754 binary32 word.
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bfloat16, nearest with ties to even.

    bfloat16 keeps the sign, the 8 exponent bits and the top 7 fraction bits
    of binary32.  Rounding adds 0x7FFF plus the lowest kept bit to the 32-bit
    word and truncates: below half an ulp truncates, above half rounds up, and
    an exact half rounds to the even neighbour.  NaN maps to the canonical
    quiet NaN 0x7FC0 (no inputs here are NaN).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    keep_lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + (np.uint32(0x7FFF) + keep_lsb)) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 storage to binary32 (append 16 zero bits)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Q, K, V draws
# ---------------------------------------------------------------------------

@dataclass
class QKV:
    """One seeded draw of Q, K, V in [B, H, T, d] layout (d innermost).

    ``q``, ``k``, ``v`` hold device storage: uint16 bfloat16 bit patterns when
    ``dtype == "bf16"``, float32 values when ``dtype == "f32"``.
    """

    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    seed: int
    qk_mult: float = 1.0
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        return self.q.shape

    def _f64(self, a: np.ndarray, b: int | None, h: int | None) -> np.ndarray:
        if b is not None:
            a = a[b, h]
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    def q64(self, b=None, h=None):
        """Exact float64 upcast of Q (one head if b, h are given)."""
        return self._f64(self.q, b, h)

    def k64(self, b=None, h=None):
        return self._f64(self.k, b, h)

    def v64(self, b=None, h=None):
        return self._f64(self.v, b, h)


def make_qkv(B: int, H: int, T: int, d: int, *, dtype: str = "bf16",
             seed: int = 0, qk_mult: float = 1.0, H_kv: int | None = None) -> QKV:
    """Draw Q, K, V i.i.d. standard normal (float32) from PCG64(seed).

    Draw order is Q, then K, then V.  Q is [B, H, T, d]; K and V are
    [B, H_kv, T, d] (H_kv = H unless given: grouped key/value heads).  Q and
    K are multiplied by ``qk_mult`` before rounding to bfloat16 (a power of
    two such as 4 commutes with the rounding, so the order does not matter
    for it).
    """
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    H_kv = H if H_kv is None else H_kv
    rng = np.random.Generator(np.random.PCG64(seed))
    arrs = []
    for name in ("q", "k", "v"):
        shape = (B, H if name == "q" else H_kv, T, d)
        a = rng.standard_normal(shape, dtype=np.float32)
        if name in ("q", "k") and qk_mult != 1.0:
            a *= np.float32(qk_mult)
        arrs.append(f32_to_bf16_bits(a) if dtype == "bf16" else a)
    return QKV(dtype=dtype, q=arrs[0], k=arrs[1], v=arrs[2], seed=seed,
               qk_mult=qk_mult)


def make_dout(B: int, H: int, T: int, d: int, *, seed: int) -> np.ndarray:
    """Upstream gradient dO of the output for the backward pass: i.i.d.
    standard normal (float32) from PCG64(seed), rounded to bfloat16; returns
    the uint16 bit patterns, [B, H, T, d]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return f32_to_bf16_bits(rng.standard_normal((B, H, T, d), dtype=np.float32))


def sample_rows(T: int, n: int, seed: int, heads: int) -> np.ndarray:
    """Per head, ``n`` distinct query rows drawn uniformly without replacement
    from PCG64(seed), plus rows 0 and T-1; shape [heads, n'] sorted."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(heads):
        r = rng.choice(T, size=min(n, T), replace=False)
        r = np.union1d(r, [0, T - 1])
        out.append(np.sort(r))
    width = max(len(r) for r in out)
    return np.stack([np.pad(r, (0, width - len(r)), mode="edge") for r in out])


# Workloads: the single-GPU sizes exercised by tests and the benchmark.
# Scale is 1/sqrt(d) throughout.
WORKLOADS = {
    "f32_b1h1_t256_d64_causal": dict(
        B=1, H=1, T=256, d=64, dtype="f32", causal=(True,), seed=1),
    "bf16_b1h8_t2048_d64_causal": dict(
        B=1, H=8, T=2048, d=64, dtype="bf16", causal=(True,), seed=2),
    "bf16_b4h16_t4096_d128": dict(
        B=4, H=16, T=4096, d=128, dtype="bf16", causal=(True, False), seed=3),
    "bf16_b1h32_t8192_d128_causal_qk4": dict(
        B=1, H=32, T=8192, d=128, dtype="bf16", causal=(True,), seed=4,
        qk_mult=4.0),
    # grouped key/value heads: 32 query heads over 8 key/value heads
    "bf16_b1h32kv8_t8192_d128_causal": dict(
        B=1, H=32, H_kv=8, T=8192, d=128, dtype="bf16", causal=(True,), seed=6),
    "bf16_b1h8_t65536_d128_causal": dict(
        B=1, H=8, T=65536, d=128, dtype="bf16", causal=(True,), seed=5,
        sample_rows=512, row_seed=1005),
}


def make_workload(name: str) -> QKV:
    w = WORKLOADS[name]
    x = make_qkv(w["B"], w["H"], w["T"], w["d"], dtype=w["dtype"],
                 seed=w["seed"], qk_mult=w.get("qk_mult", 1.0), H_kv=w.get("H_kv"))
    x.meta = dict(w, name=name)
    return x


# ---------------------------------------------------------------------------
# Decode: new queries over a key/value cache
# ---------------------------------------------------------------------------

def make_decode(B: int, H: int, H_kv: int, Tq: int, Tk: int, d: int, *, seed: int,
                Tk_cap: int | None = None, qk_mult: float = 1.0) -> QKV:
    """Draw the Tq new queries [B, H, Tq, d] and caches [B, H_kv, Tk_cap, d]
    i.i.d. standard normal (float32) from PCG64(seed), in the order Q, K, V,
    rounded to bfloat16.  Cache rows >= Tk (capacity beyond the valid
    length) hold the bit pattern 0x7FC0 (a NaN), which no correct reader
    touches."""
    Tk_cap = Tk if Tk_cap is None else Tk_cap
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, H, Tq, d), dtype=np.float32)
    k = rng.standard_normal((B, H_kv, Tk, d), dtype=np.float32)
    v = rng.standard_normal((B, H_kv, Tk, d), dtype=np.float32)
    if qk_mult != 1.0:
        q *= np.float32(qk_mult)
        k *= np.float32(qk_mult)
    arrs = [f32_to_bf16_bits(q)]
    for a in (k, v):
        full = np.full((B, H_kv, Tk_cap, d), 0x7FC0, dtype=np.uint16)
        full[:, :, :Tk] = f32_to_bf16_bits(a)
        arrs.append(full)
    return QKV(dtype="bf16", q=arrs[0], k=arrs[1], v=arrs[2], seed=seed, qk_mult=qk_mult,
               meta=dict(B=B, H=H, H_kv=H_kv, Tq=Tq, Tk=Tk, Tk_cap=Tk_cap, d=d))


# Decode workloads: one new token per sequence over a long cache, grouped
# key/value heads (32 query heads over 8 key/value heads).
DECODE_WORKLOADS = {
    "bf16_b16h32kv8_tq1_tk32768_d128_causal": dict(
        B=16, H=32, H_kv=8, Tq=1, Tk=32768, d=128, causal=True, seed=8),
    "bf16_b1h32kv8_tq1_tk131072_d128_causal": dict(
        B=1, H=32, H_kv=8, Tq=1, Tk=131072, d=128, causal=True, seed=9),
}
