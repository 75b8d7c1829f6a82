"""Grouped-query attention in float64 (oracle of the grouped-key/value
variants of the forward and the backward).

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may import it.

"FlashAttention -- avoid writing the giant intermediate" closes by naming
grouped-query attention as the way a model's head structure shrinks the
stored keys and values; it does not spell the structure out.  The plainest
reading, taken here: H query heads and H_kv key/value heads, H_kv dividing
H, and query head h attends with key/value head h // (H / H_kv), so each run
of G = H / H_kv consecutive query heads shares one key/value head.  Each
query head is then ordinary exact attention (``attention.attention_head``)
against its group's keys and values.  The gradient with respect to a shared
key/value head is the sum of what its G query heads send back
(``backward.attention_head_bwd`` per query head), since the loss depends on
that head through each of them.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_head
from .backward import attention_head_bwd

__all__ = ["kv_head", "attention_gqa", "attention_gqa_bwd"]


def kv_head(h: int, H: int, H_kv: int) -> int:
    """Key/value head read by query head h."""
    if H_kv < 1 or H % H_kv:
        raise ValueError("H_kv must divide H")
    return h // (H // H_kv)


def attention_gqa(q, k, v, *, causal: bool, scale: float, rows=None):
    """q [B, H, T, d]; k, v [B, H_kv, T, d].  Returns (O [B, H, R, d],
    LSE [B, H, R]) in float64; ``rows`` as for ``oracle.attention``."""
    q, k, v = (np.asarray(x) for x in (q, k, v))
    B, H, T, d = q.shape
    H_kv = k.shape[1]
    Os, Ls = [], []
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, H_kv)
            r = attention_head(q[b, h], k[b, g], v[b, g], causal=causal, scale=scale,
                               rows=rows)
            Os.append(r["O"])
            Ls.append(r["LSE"])
    R = Os[0].shape[0]
    return np.stack(Os).reshape(B, H, R, d), np.stack(Ls).reshape(B, H, R)


def attention_gqa_bwd(q, k, v, do, *, causal: bool, scale: float):
    """Gradients for an upstream gradient dO [B, H, T, d]: returns dQ
    [B, H, T, d] and dK, dV [B, H_kv, T, d] in float64."""
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    B, H, T, d = q.shape
    H_kv = k.shape[1]
    dQ = np.zeros((B, H, T, d))
    dK = np.zeros((B, H_kv, T, d))
    dV = np.zeros((B, H_kv, T, d))
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, H_kv)
            r = attention_head_bwd(q[b, h], k[b, g], v[b, g], do[b, h], causal=causal,
                                   scale=scale)
            dQ[b, h] = r["dQ"]
            dK[b, g] += r["dK"]
            dV[b, g] += r["dV"]
    return dQ, dK, dV
