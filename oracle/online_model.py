"""Float64 CPU models of the tiled ("online") softmax, used to check the
method itself against the materialised oracle.

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may import it.

``online_attention_head`` walks the keys in blocks and carries, per query
row, a running maximum, a running normaliser (the exponential sum, expressed
relative to the running maximum) and an output accumulator.  Whenever a block
raises the maximum, the normaliser and the accumulator gathered so far are
rescaled by exp(old max - new max) before the block's own terms are added.
After the last block the accumulator is divided by the normaliser.
[P2 section 3, "Online Softmax"; P3 "Tiling and an incremental
normalization"; the control flow is the "Tiled attention" path of P3 "Watch
the decision": load a tile, update the running normalisation and output,
repeat while tiles remain, then write the output.]

The pages describe the recurrence in words only; the formulas below are the
plainest ones that match that description.

``tile_local_softmax_head`` is the wrong method the pages warn about: each key
block normalises its own scores with its own denominator and the per-block
probabilities are concatenated.  [P1 "How the Remaining Scores Change a
Probability", Figure 4; P3 "Tiling and an incremental normalization"]  It is
kept only as a negative control.
"""
from __future__ import annotations

import numpy as np

__all__ = ["online_attention_head", "tile_local_softmax_head"]


def _scaled_masked_block(q, kb, scale, causal, row_idx, col_idx):
    s = scale * (q @ kb.T)
    if causal:
        s = np.where(col_idx[None, :] > row_idx[:, None], -np.inf, s)
    return s


def online_attention_head(q, k, v, *, causal: bool, scale: float,
                          block: int):
    """Tiled forward with the running-max / running-sum recurrence.

    Returns dict(O=[T, d], LSE=[T]) in float64.  ``block`` is the number of
    keys per tile (any value from 1 to T).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, d = q.shape
    rows = np.arange(T)
    m = np.full(T, -np.inf)          # running maximum of the row's scores
    l = np.zeros(T)                  # running exponential sum, relative to m
    acc = np.zeros((T, v.shape[1]))  # running weighted sum of values, rel. m
    for start in range(0, T, block):
        cols = np.arange(start, min(start + block, T))
        s = _scaled_masked_block(q, k[cols], scale, causal, rows, cols)
        m_new = np.maximum(m, s.max(axis=1))
        # Rows with no permitted key so far keep m = -inf; use 0 as their
        # base so that the exponentials below are exp(-inf) = 0, not NaN.
        base = np.where(np.isneginf(m_new), 0.0, m_new)
        alpha = np.exp(m - base)                      # rescale old terms
        p = np.exp(s - base[:, None])                 # this block's terms
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[cols]
        m = m_new
    O = acc / l[:, None]
    LSE = m + np.log(l)
    return {"O": O, "LSE": LSE}


def tile_local_softmax_head(q, k, v, *, causal: bool, scale: float,
                            block: int):
    """Negative control: softmax applied to each key block on its own.

    Each block's probabilities sum to one over that block, so a row spread
    over n blocks gets total weight n.  Returns dict(P=[T, T], O=[T, d]).
    Blocks in which a row has no permitted key contribute zero weight.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T = q.shape[0]
    rows = np.arange(T)
    P = np.zeros((T, T))
    for start in range(0, T, block):
        cols = np.arange(start, min(start + block, T))
        s = _scaled_masked_block(q, k[cols], scale, causal, rows, cols)
        mb = s.max(axis=1, keepdims=True)
        ok = np.isfinite(mb[:, 0])
        e = np.zeros_like(s)
        e[ok] = np.exp(s[ok] - mb[ok])
        denom = e.sum(axis=1, keepdims=True)
        denom[~ok] = 1.0
        P[:, cols] = e / denom
    return {"P": P, "O": P @ v}
