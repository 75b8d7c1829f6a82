"""Gradients of exact attention in float64 (the oracle of the backward pass).

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may import it.

The pages state that the fused method's backward pass recomputes the
attention scores, which the forward never stored, instead of reading them
back ("Attention Mechanism: Computation & Memory Patterns", section 4,
"Computational Pattern", and its conclusion).  They do not write the
gradient out.  The plainest reading, taken here: the gradient of the forward
of ``attention.py`` with respect to Q, K and V, for an upstream gradient dO
of the output (equivalently, of the scalar L = sum_ic dO_ic O_ic).  The chain
rule through the forward's steps, one head, T x d operands:

  5. O = P V             ->  dV = P^T dO,   dP = dO V^T
  4. P = rowsoftmax(S)   ->  dS_ij = P_ij (dP_ij - Delta_i),
                             Delta_i = sum_k P_ik dP_ik
                             (the Jacobian of a row softmax; a masked entry
                             has P_ij = 0 and so dS_ij = 0: the causal mask
                             passes no gradient)
  1-2. S = scale Q K^T   ->  dQ = scale dS K,   dK = scale dS^T Q

Delta_i also equals sum_c dO_ic O_ic, since O_i = sum_k P_ik V_k; the
function returns it because the fused backward computes it that way.

Everything is materialised from the forward oracle's P; nothing is tiled or
recomputed from a saved log-sum-exp (that is the fused kernel's business, and
the tests compare it against this).
"""
from __future__ import annotations

import numpy as np

from .attention import attention_head

__all__ = ["attention_head_bwd"]


def attention_head_bwd(q, k, v, do, *, causal: bool, scale: float, rows=None, keys=None):
    """Gradients of exact attention for one head, float64, materialised.

    Parameters
    ----------
    q, k, v, do : array_like, shape [T, d]
        Queries, keys, values and the upstream gradient of the output.
    causal, scale :
        As for :func:`oracle.attention_head`.
    rows : array_like of int, optional
        Query rows whose dQ (and Delta) to return; default all.
    keys : array_like of int, optional
        Key rows whose dK and dV to return; default all.

    Returns
    -------
    dict with
      ``dQ`` [R, d], ``Delta`` [R]   for the selected query rows,
      ``dK`` [J, d], ``dV`` [J, d]   for the selected key rows,
      ``P``, ``dS`` [T, T]           the full probability and score-gradient
                                     matrices (rows = queries),
      ``O``, ``LSE``                 the forward's output rows and
                                     log-sum-exp, all T rows,
      ``rows``, ``keys``             the selected indices.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    T = k.shape[0]
    if do.shape != q.shape:
        raise ValueError("dO must have the shape of Q")
    r = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(T) if keys is None else np.asarray(keys, dtype=np.int64)

    fwd = attention_head(q, k, v, causal=causal, scale=scale)
    P = fwd["P"]
    # through O = P V
    dP = do @ v.T
    dV = P[:, j].T @ do
    # through the row softmax
    Delta = (P * dP).sum(axis=1)
    dS = P * (dP - Delta[:, None])
    # through S = scale Q K^T
    dQ = scale * (dS[r] @ k)
    dK = scale * (dS[:, j].T @ q)
    return {"dQ": dQ, "dK": dK, "dV": dV, "Delta": Delta[r], "P": P, "dS": dS,
            "O": fwd["O"], "LSE": fwd["LSE"], "rows": r, "keys": j}
