"""Pins for the attention oracle: checks against values the pages print,
closed forms, invariants, a library routine on a reducing special case and an
independent brute force on tiny inputs.

Every pin takes the function under test as its argument (same signature and
return value as ``oracle.attention_head``) so that the mutation tests can run
the same pins against deliberately broken copies of the oracle and show that
each plausible mistake is caught.  A pin raises AssertionError on failure.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _ok(res):
    for key in ("O", "LSE"):
        assert np.all(np.isfinite(res[key])), f"non-finite {key}"


# ---------------------------------------------------------------------------
# Values printed by the pages
# ---------------------------------------------------------------------------

def pin_two_score_exercise(attn):
    """Scores {0, ln 3} give weights {1/4, 3/4}.  [P3 "Tiling and an
    incremental normalization", normalization exercise]

    T = 2, causal, scale 1, d = 2: k0 = 0, k1 = (ln 3, 0), q1 = (1, 0) so
    that row 1's scores are (0, ln 3); V = identity so O row 1 equals P row 1.
    Row 0 sees only key 0, so O[0] = V[0] and LSE[0] = q0.k0 = 0.
    """
    g = _golden("two_score_exercise.json")
    w = np.array(g["correct_weights"])
    q = np.array([[0.3, -0.7], [1.0, 0.0]])
    k = np.array([[0.0, 0.0], [math.log(3.0), 0.0]])
    v = np.eye(2)
    res = attn(q, k, v, causal=True, scale=1.0)
    _ok(res)
    np.testing.assert_allclose(res["P"][1], w, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["O"][1], w, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["LSE"][1], math.log(4.0), rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["O"][0], [1.0, 0.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(res["P"][0], [1.0, 0.0], rtol=0, atol=0)
    assert abs(res["LSE"][0]) <= 1e-15


def pin_fig4_rows(attn):
    """Figure 4 rows: [0,0,0,0] -> 25 % each; [0,0,2,2] -> first probability
    about 6 %, exponential sum about 16.78.  [P1 "How the Remaining Scores
    Change a Probability", Figure 4]

    d = 1, scale 1, non-causal: query 1 and keys equal to the printed scores.
    The exponential sum is exp(LSE).  The printed values are checked at the
    page's two decimals and the closed forms 1/4 and 1/(2 + 2 e^2) tightly.
    """
    g = _golden("fig4_row_probabilities.json")
    for case in g["cases"]:
        s = np.array(case["scores"])
        q = np.ones((4, 1))
        k = s[:, None]
        v = np.arange(4.0)[:, None] + 1.0
        res = attn(q, k, v, causal=False, scale=1.0)
        _ok(res)
        p0 = res["P"][0, 0]
        z = math.exp(res["LSE"][0])
        dec = case["printed_decimals"]
        assert round(p0, dec) == case["printed_first_probability"], p0
        assert round(z, dec) == case["printed_exp_sum"], z
        closed = 1.0 / sum(math.exp(x) for x in case["scores"])
        assert abs(p0 - closed) <= 1e-12
        # every row of this input is identical
        np.testing.assert_allclose(res["P"], np.tile(res["P"][0], (4, 1)),
                                   rtol=0, atol=1e-15)
    # the right-hand row's first weight, tightly: 1 / (2 + 2 e^2)
    res = attn(np.ones((4, 1)), np.array([[0.0], [0.0], [2.0], [2.0]]),
               np.ones((4, 1)), causal=False, scale=1.0)
    assert abs(res["P"][0, 0] - 1.0 / (2.0 + 2.0 * math.exp(2.0))) <= 1e-12
    assert abs(res["P"][0, 2] - math.exp(2.0) / (2.0 + 2.0 * math.exp(2.0))) <= 1e-12


# ---------------------------------------------------------------------------
# Invariants the pages state
# ---------------------------------------------------------------------------

def pin_rows_sum_to_one_masked_zero(attn):
    """Each row of P sums to 1 and masked (future) keys get probability
    exactly 0.  [P1 "The Attention Computation Flow"]"""
    rng = _rng(11)
    for causal in (True, False):
        T, d = 37, 8
        q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
        res = attn(q, k, v, causal=causal, scale=0.7)
        _ok(res)
        P = res["P"]
        assert np.all(P >= 0)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        if causal:
            iu = np.triu_indices(T, k=1)
            assert np.all(P[iu] == 0.0)
            assert np.all(np.isneginf(res["S"][iu]))
            il = np.tril_indices(T)
            assert np.all(P[il] > 0.0)
        else:
            assert np.all(P > 0.0)


def pin_causal_row0(attn):
    """Causal row 0 may attend only to key 0: O[0] = V[0] and LSE[0] =
    scale * q0.k0.  [P1 "The Attention Computation Flow": a token attends
    to itself and earlier tokens]"""
    rng = _rng(12)
    T, d = 19, 6
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    res = attn(q, k, v, causal=True, scale=0.45)
    _ok(res)
    np.testing.assert_allclose(res["O"][0], v[0], rtol=0, atol=1e-15)
    assert abs(res["LSE"][0] - 0.45 * float(q[0] @ k[0])) <= 1e-14


def pin_equal_scores(attn):
    """Equal scores give each permitted key the same weight (Figure 4's
    uniform row): with scale 0, causal row i is the mean of V[0..i] and
    LSE = ln(i+1); non-causal rows are the mean of V and LSE = ln T.  Same
    for Q = 0 at any scale.  [P1 Figure 4, left case]"""
    rng = _rng(13)
    T, d = 23, 5
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    for qq, sc in ((q, 0.0), (np.zeros_like(q), 1.3)):
        rc = attn(qq, k, v, causal=True, scale=sc)
        _ok(rc)
        prefix = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None]
        np.testing.assert_allclose(rc["O"], prefix, rtol=0, atol=1e-13)
        np.testing.assert_allclose(rc["LSE"], np.log(np.arange(1, T + 1)),
                                   rtol=0, atol=1e-13)
        rn = attn(qq, k, v, causal=False, scale=sc)
        _ok(rn)
        np.testing.assert_allclose(rn["O"], np.tile(v.mean(axis=0), (T, 1)),
                                   rtol=0, atol=1e-13)
        np.testing.assert_allclose(rn["LSE"], math.log(T), rtol=0, atol=1e-13)


def pin_future_keys_do_not_matter(attn):
    """A causal row depends only on the keys it may attend to: changing K
    and V rows after i0 leaves rows 0..i0 unchanged.  [P1 "From a Score Tile
    to Probabilities": the dependency spans the permitted key positions]"""
    rng = _rng(14)
    T, d, i0 = 29, 7, 11
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    a = attn(q, k, v, causal=True, scale=0.5)
    k2, v2 = k.copy(), v.copy()
    k2[i0 + 1:] = 50.0 * rng.standard_normal((T - i0 - 1, d))
    v2[i0 + 1:] = 50.0 * rng.standard_normal((T - i0 - 1, d))
    b = attn(q, k2, v2, causal=True, scale=0.5)
    _ok(a), _ok(b)
    np.testing.assert_allclose(a["O"][:i0 + 1], b["O"][:i0 + 1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(a["LSE"][:i0 + 1], b["LSE"][:i0 + 1], rtol=0, atol=1e-13)
    assert np.abs(a["O"][i0 + 1:] - b["O"][i0 + 1:]).max() > 1e-3


def pin_query_rows_independent(attn):
    """Changing query row r changes only output row r.  [P1 "From a Score
    Tile to Probabilities": scores from other query rows are not needed]"""
    rng = _rng(15)
    T, d, r = 21, 6, 9
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    for causal in (True, False):
        a = attn(q, k, v, causal=causal, scale=0.8)
        q2 = q.copy()
        q2[r] = rng.standard_normal(d) * 3.0
        b = attn(q2, k, v, causal=causal, scale=0.8)
        keep = np.arange(T) != r
        np.testing.assert_allclose(a["O"][keep], b["O"][keep], rtol=0, atol=1e-13)
        np.testing.assert_allclose(a["LSE"][keep], b["LSE"][keep], rtol=0, atol=1e-13)
        assert np.abs(a["O"][r] - b["O"][r]).max() > 1e-3


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def pin_single_token(attn):
    """T = 1: the only weight is 1, so O = V and LSE = scale * q.k."""
    rng = _rng(16)
    for d in (1, 4, 64):
        q, k, v = (rng.standard_normal((1, d)) for _ in range(3))
        for causal in (True, False):
            res = attn(q, k, v, causal=causal, scale=0.3)
            np.testing.assert_allclose(res["O"], v, rtol=0, atol=1e-15)
            assert abs(res["LSE"][0] - 0.3 * float(q[0] @ k[0])) <= 1e-13


def pin_key_shift(attn):
    """Adding a vector u to every key adds scale*q_i.u to every permitted
    score of row i: P and O are unchanged and LSE_i grows by scale*q_i.u
    (softmax is invariant to a per-row shift)."""
    rng = _rng(17)
    T, d, sc = 17, 5, 0.6
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    u = rng.standard_normal(d)
    for causal in (True, False):
        a = attn(q, k, v, causal=causal, scale=sc)
        b = attn(q, k + u, v, causal=causal, scale=sc)
        np.testing.assert_allclose(b["O"], a["O"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(b["LSE"], a["LSE"] + sc * (q @ u),
                                   rtol=0, atol=1e-12)


def pin_linear_in_values(attn):
    """O = P V is linear in V: O(aV + bW) = a O(V) + b O(W).  [P1 "The
    Attention Computation Flow": a probability-weighted sum of values]"""
    rng = _rng(18)
    T, d = 15, 4
    q, k, v, w = (rng.standard_normal((T, d)) for _ in range(4))
    for causal in (True, False):
        a = attn(q, k, v, causal=causal, scale=0.9)["O"]
        b = attn(q, k, w, causal=causal, scale=0.9)["O"]
        c = attn(q, k, 2.5 * v - 1.5 * w, causal=causal, scale=0.9)["O"]
        np.testing.assert_allclose(c, 2.5 * a - 1.5 * b, rtol=0, atol=1e-12)


def pin_values_identity(attn):
    """With V = I (T = d) the output rows are the probability rows."""
    rng = _rng(19)
    T = 12
    q, k = (rng.standard_normal((T, 3)) for _ in range(2))
    for causal in (True, False):
        res = attn(q, k, np.eye(T), causal=causal, scale=1.1)
        np.testing.assert_allclose(res["O"], res["P"], rtol=0, atol=1e-15)


def pin_rows_subset(attn):
    """Computing a subset of query rows gives exactly those rows of the full
    result (rows are independent)."""
    rng = _rng(20)
    T, d = 33, 6
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    rows = np.array([0, 5, 17, 32])
    for causal in (True, False):
        full = attn(q, k, v, causal=causal, scale=0.4)
        sub = attn(q, k, v, causal=causal, scale=0.4, rows=rows)
        np.testing.assert_allclose(sub["O"], full["O"][rows], rtol=0, atol=1e-14)
        np.testing.assert_allclose(sub["LSE"], full["LSE"][rows], rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# A library routine on a case that reduces to it
# ---------------------------------------------------------------------------

def pin_scipy_softmax(attn):
    """Row softmax and log-sum-exp agree with scipy.special.softmax /
    logsumexp applied to the scaled, masked score matrix built here by an
    explicit double loop."""
    from scipy.special import logsumexp, softmax
    rng = _rng(21)
    T, d, sc = 14, 3, -0.75
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    for causal in (True, False):
        S = np.empty((T, T))
        for i in range(T):
            for j in range(T):
                S[i, j] = -np.inf if (causal and j > i) else sc * math.fsum(
                    q[i, t] * k[j, t] for t in range(d))
        res = attn(q, k, v, causal=causal, scale=sc)
        np.testing.assert_allclose(res["P"], softmax(S, axis=1), rtol=0, atol=1e-13)
        np.testing.assert_allclose(res["LSE"], logsumexp(S, axis=1), rtol=0, atol=1e-13)
        np.testing.assert_allclose(res["O"], softmax(S, axis=1) @ v, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# Brute force on tiny inputs
# ---------------------------------------------------------------------------

def brute_force_head(q, k, v, causal, scale):
    """Direct scalar evaluation of the definition: weight_ij =
    exp(s_ij) / sum over permitted j' of exp(s_ij'), with no shift, in pure
    Python with compensated sums (valid for the small scores used here)."""
    T = len(q)
    dv = len(v[0])
    O, L = [], []
    for i in range(T):
        perm = [j for j in range(T) if not (causal and j > i)]
        e = [math.exp(scale * math.fsum(a * b for a, b in zip(q[i], k[j])))
             for j in perm]
        z = math.fsum(e)
        O.append([math.fsum(e[n] * v[j][c] for n, j in enumerate(perm)) / z
                  for c in range(dv)])
        L.append(math.log(z))
    return np.array(O), np.array(L)


def pin_brute_force(attn):
    """Agreement with the scalar brute force for T = 1..12, several d, both
    mask settings and random (also negative) scales."""
    rng = _rng(22)
    for T in range(1, 13):
        for d in (1, 2, 3, 5, 8):
            q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
            sc = float(rng.uniform(-1.5, 1.5))
            for causal in (True, False):
                res = attn(q, k, v, causal=causal, scale=sc)
                O, L = brute_force_head(q.tolist(), k.tolist(), v.tolist(),
                                        causal, sc)
                np.testing.assert_allclose(res["O"], O, rtol=0, atol=1e-12)
                np.testing.assert_allclose(res["LSE"], L, rtol=0, atol=1e-12)


ALL_PINS = [
    pin_two_score_exercise,
    pin_fig4_rows,
    pin_rows_sum_to_one_masked_zero,
    pin_causal_row0,
    pin_equal_scores,
    pin_future_keys_do_not_matter,
    pin_query_rows_independent,
    pin_single_token,
    pin_key_shift,
    pin_linear_in_values,
    pin_values_identity,
    pin_rows_subset,
    pin_scipy_softmax,
    pin_brute_force,
]
