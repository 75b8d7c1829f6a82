"""Materialised exact attention in float64 (the oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may import it.

For one head with queries Q, keys K and values V, each T x d:

  1. scores      S = scale * Q K^T, a T x T matrix, rows = queries and
                 columns = keys.                       [P1 "The Attention
                 Computation Flow"; P2 section 1, the attention equation and
                 step 1 "Score Calculation"]
  2. scaling     ``scale`` is a plain multiplier; the usual choice is
                 1/sqrt(d).  Scaling comes before masking.   [P1 Figure 1
                 discussion; P2 section 1 step 2]
  3. causal mask a key j later than the query i (j > i) gets score -inf, so
                 its probability is exactly zero; the diagonal is kept.
                 [P1 "The Attention Computation Flow", Figure 1]
  4. softmax     each row: exp of every unmasked score divided by the row's
                 "exponential sum".  The row maximum m_i is subtracted before
                 exp (softmax is unchanged by a per-row shift; this only keeps
                 float64 in range).    [P1 "From a Score Tile to
                 Probabilities"; P2 section 1 step 2]
  5. output      O = P V.              [P1 "The Attention Computation Flow";
                 P2 section 1 step 3]
  6. LSE         LSE_i = m_i + ln(l_i) with l_i = sum_j exp(S_ij - m_i), the
                 natural log of the exponential sum of the scaled, masked
                 scores.  The pages do not define this side output; this is
                 the plainest reading of "log-sum-exp" of the row.

Everything is materialised (S and P exist in full), as in the "materialized
attention" path of [P3 "Watch the decision"]; this module never tiles.
"""
from __future__ import annotations

import numpy as np

__all__ = ["attention_head", "attention", "attention_heads"]


def attention_head(q, k, v, *, causal: bool, scale: float, rows=None):
    """Exact attention for one head, float64, materialised.

    Parameters
    ----------
    q, k, v : array_like, shape [T, d]
        Queries, keys, values (converted to float64).
    causal : bool
        Apply the causal mask (key j permitted for query i iff j <= i).
    scale : float
        Multiplier applied to every dot product before masking.
    rows : array_like of int, optional
        Compute only these query rows (each still against all T keys).

    Returns
    -------
    dict with
      ``S``   [R, T] scaled, masked scores (-inf where masked),
      ``P``   [R, T] probabilities,
      ``O``   [R, d] outputs,
      ``LSE`` [R]    log of the exponential sum (natural log),
      ``rows`` [R]   the query indices the rows correspond to.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T = k.shape[0]
    if q.shape[0] != T or v.shape[0] != T:
        raise ValueError("Q, K and V must have the same number of rows")
    r = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)

    # 1-2. scaled scores: query rows against every key.
    S = scale * (q[r] @ k.T)
    # 3. causal mask: future keys (column index greater than the query's
    # index) are set to -inf after scaling.
    if causal:
        future = np.arange(T)[None, :] > r[:, None]
        S = np.where(future, -np.inf, S)
    # 4. row softmax with the exponential sum as denominator.
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    # 5. output and 6. log-sum-exp.
    O = P @ v
    LSE = m[:, 0] + np.log(l[:, 0])
    return {"S": S, "P": P, "O": O, "LSE": LSE, "rows": r}


def attention(q, k, v, *, causal: bool, scale: float, rows=None):
    """Exact attention over a [B, H, T, d] batch, one head at a time.

    ``q``, ``k``, ``v`` are arrays of shape [B, H, T, d] (see
    :func:`attention_heads` for per-head accessors).  ``rows`` is None (all rows), a 1-D index array used for every
    head, or a [B*H, R] array giving the rows per head (flattened b*H + h).

    Returns (O, LSE) with shapes [B, H, R, d] and [B, H, R] in float64.
    """
    q = np.asarray(q)
    B, H, T, d = q.shape
    return attention_heads(lambda b, h: q[b, h], lambda b, h: k[b, h],
                           lambda b, h: v[b, h], B=B, H=H, causal=causal,
                           scale=scale, rows=rows)


def attention_heads(qf, kf, vf, *, B: int, H: int, causal: bool, scale: float,
                    rows=None):
    """Same as :func:`attention`, with callables ``f(b, h) -> [T, d]`` in
    place of the arrays, so that large inputs are upcast one head at a
    time."""
    Os, Ls = [], []
    for b in range(B):
        for h in range(H):
            if rows is None:
                rr = None
            else:
                rows_a = np.asarray(rows)
                rr = rows_a if rows_a.ndim == 1 else rows_a[b * H + h]
            res = attention_head(qf(b, h), kf(b, h), vf(b, h), causal=causal,
                                 scale=scale, rows=rr)
            Os.append(res["O"])
            Ls.append(res["LSE"])
    R = Os[0].shape[0]
    d = Os[0].shape[1]
    return (np.stack(Os).reshape(B, H, R, d), np.stack(Ls).reshape(B, H, R))
