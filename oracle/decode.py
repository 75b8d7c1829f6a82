"""Attention of a few new queries over a cached sequence of keys and values
(decode), in float64: the oracle of the split-key/value decode path.

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may import it.

"FlashAttention -- avoid writing the giant intermediate" separates long-input
prefill from short-input decode and stresses the key/value state kept across
steps; it does not define decode further.  The plainest reading, taken here:
the cache holds keys and values of Tk positions 0 .. Tk-1, the Tq new queries
are the last Tq of those positions (query i sits at position Tk - Tq + i, its
own key and value already appended), and the causal mask is the one of the
square forward at those positions: query i may see key j iff
j <= Tk - Tq + i.  Without the mask every query sees all Tk keys.  Each query
row is then the ordinary computation of ``attention.attention_head``: scaled
scores, mask, row softmax, P V, and the natural-log sum of exponentials.
"""
from __future__ import annotations

import numpy as np

__all__ = ["attention_decode_head", "attention_decode"]


def attention_decode_head(q, k, v, *, causal: bool, scale: float):
    """q [Tq, d]; k, v [Tk, d] (Tk >= Tq under the causal mask).  Returns dict
    O [Tq, d], LSE [Tq], P [Tq, Tk] (float64)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, Tk = q.shape[0], k.shape[0]
    if causal and Tk < Tq:
        raise ValueError("the cache must hold at least the new queries' positions")
    S = scale * (q @ k.T)
    if causal:
        pos = Tk - Tq + np.arange(Tq)
        S = np.where(np.arange(Tk)[None, :] > pos[:, None], -np.inf, S)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    return {"O": P @ v, "LSE": m[:, 0] + np.log(l[:, 0]), "P": P}


def attention_decode(q, k, v, *, causal: bool, scale: float):
    """q [B, H, Tq, d]; k, v [B, H_kv, Tk, d], H_kv dividing H (query head h
    reads key/value head h // (H / H_kv), as in ``gqa``).  Returns
    (O [B, H, Tq, d], LSE [B, H, Tq])."""
    q, k, v = (np.asarray(x) for x in (q, k, v))
    B, H, Tq, d = q.shape
    G = H // k.shape[1]
    O = np.zeros((B, H, Tq, d))
    L = np.zeros((B, H, Tq))
    for b in range(B):
        for h in range(H):
            r = attention_decode_head(q[b, h], k[b, h // G], v[b, h // G], causal=causal,
                                      scale=scale)
            O[b, h], L[b, h] = r["O"], r["LSE"]
    return O, L
