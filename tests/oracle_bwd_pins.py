"""Pins of the backward oracle: what the mathematics fixes about the gradient
of exact attention, independently of the oracle's own formulas.

Each pin takes a backward function with the signature of
``oracle.attention_head_bwd`` and raises AssertionError when it is wrong.
The strongest pin is the finite-difference one: it differentiates the
(separately pinned) forward oracle numerically, so it shares no formula with
the chain rule written out in ``oracle/backward.py``.  The others are exact
identities that hold for any inputs:

- softmax rows are invariant to a shift of every score in the row, so adding
  one vector to every key changes nothing: the key gradients sum to zero;
- rows of P sum to one, so the value gradients sum to the summed dO;
- a single key (or the first query under a causal mask) sees P = 1,
  independent of Q and K: no gradient reaches Q or K there;
- with all value rows equal, O does not depend on P at all;
- Delta_i = sum_c dO_ic O_ic;
- the gradient is linear in dO.
"""
import numpy as np

from oracle import attention_head


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _loss(q, k, v, do, causal, scale):
    return float((attention_head(q, k, v, causal=causal, scale=scale)["O"] * do).sum())


def pin_finite_differences(bwd):
    """Central differences of L = sum(dO * O(Q, K, V)) through the forward
    oracle, every entry of Q, K and V."""
    rng = _rng(11)
    h = 1e-5
    for T, d, causal, scale in ((1, 3, True, 0.8), (3, 2, False, -0.6), (5, 3, True, 0.7),
                                (6, 4, False, 1.3), (7, 2, True, 2.1)):
        q, k, v, do = (rng.standard_normal((T, d)) for _ in range(4))
        g = bwd(q, k, v, do, causal=causal, scale=scale)
        for name, x, ref in (("dQ", q, g["dQ"]), ("dK", k, g["dK"]), ("dV", v, g["dV"])):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"dQ": (xp, k, v), "dK": (q, xp, v), "dV": (q, k, xp)}[name]
                args_m = {"dQ": (xm, k, v), "dK": (q, xm, v), "dV": (q, k, xm)}[name]
                num[idx] = (_loss(*args_p, do, causal, scale)
                            - _loss(*args_m, do, causal, scale)) / (2 * h)
            np.testing.assert_allclose(ref, num, rtol=1e-6, atol=1e-8,
                                       err_msg=f"{name} T={T} causal={causal}")


def pin_single_key(bwd):
    """T = 1: O = V, so dV = dO and nothing reaches Q or K."""
    rng = _rng(12)
    for causal in (True, False):
        q, k, v, do = (rng.standard_normal((1, 5)) for _ in range(4))
        g = bwd(q, k, v, do, causal=causal, scale=0.9)
        np.testing.assert_allclose(g["dV"], do, rtol=0, atol=1e-15)
        np.testing.assert_allclose(g["dQ"], 0.0, rtol=0, atol=1e-15)
        np.testing.assert_allclose(g["dK"], 0.0, rtol=0, atol=1e-15)


def pin_equal_values(bwd):
    """All value rows equal: O = that row whatever P is, so dQ = dK = 0,
    while dV_j = sum_i P_ij dO_i still sums to sum_i dO_i."""
    rng = _rng(13)
    for causal in (True, False):
        T, d = 7, 4
        q, k, do = (rng.standard_normal((T, d)) for _ in range(3))
        v = np.tile(rng.standard_normal((1, d)), (T, 1))
        g = bwd(q, k, v, do, causal=causal, scale=1.1)
        np.testing.assert_allclose(g["dQ"], 0.0, rtol=0, atol=1e-13)
        np.testing.assert_allclose(g["dK"], 0.0, rtol=0, atol=1e-13)
        np.testing.assert_allclose(g["dV"].sum(0), do.sum(0), rtol=0, atol=1e-12)


def pin_key_shift_invariance(bwd):
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i, for any inputs."""
    rng = _rng(14)
    for T, causal in ((9, True), (9, False), (16, True)):
        q, k, v, do = (rng.standard_normal((T, 4)) * 1.5 for _ in range(4))
        g = bwd(q, k, v, do, causal=causal, scale=0.6)
        np.testing.assert_allclose(g["dK"].sum(0), 0.0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(g["dV"].sum(0), do.sum(0), rtol=0, atol=1e-12)


def pin_causal_ends(bwd):
    """Causal: query 0 sees only key 0 (P = 1), so dQ_0 = 0; the last key is
    seen only by the last query, so dV_{T-1} = P_{T-1,T-1} dO_{T-1} and
    dK_{T-1} = scale dS_{T-1,T-1} Q_{T-1}, with P from the forward oracle and
    dS_{T-1,T-1} = P (dO_{T-1} . (V_{T-1} - O_{T-1}))."""
    rng = _rng(15)
    T, d, scale = 8, 3, 0.75
    q, k, v, do = (rng.standard_normal((T, d)) for _ in range(4))
    g = bwd(q, k, v, do, causal=True, scale=scale)
    f = attention_head(q, k, v, causal=True, scale=scale)
    p_last = f["P"][T - 1, T - 1]
    np.testing.assert_allclose(g["dQ"][0], 0.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(g["dV"][T - 1], p_last * do[T - 1], rtol=1e-13, atol=1e-15)
    ds = p_last * float(do[T - 1] @ (v[T - 1] - f["O"][T - 1]))
    np.testing.assert_allclose(g["dK"][T - 1], scale * ds * q[T - 1], rtol=1e-12, atol=1e-15)


def pin_delta(bwd):
    """Delta_i = sum_c dO_ic O_ic with O from the forward oracle."""
    rng = _rng(16)
    for causal in (True, False):
        q, k, v, do = (rng.standard_normal((10, 5)) for _ in range(4))
        g = bwd(q, k, v, do, causal=causal, scale=0.5)
        O = attention_head(q, k, v, causal=causal, scale=0.5)["O"]
        np.testing.assert_allclose(g["Delta"], (do * O).sum(1), rtol=1e-13, atol=1e-14)


def pin_linear_in_do(bwd):
    """grad(dO1 + 2 dO2) = grad(dO1) + 2 grad(dO2)."""
    rng = _rng(17)
    q, k, v, d1, d2 = (rng.standard_normal((6, 3)) for _ in range(5))
    g1 = bwd(q, k, v, d1, causal=True, scale=0.9)
    g2 = bwd(q, k, v, d2, causal=True, scale=0.9)
    g3 = bwd(q, k, v, d1 + 2 * d2, causal=True, scale=0.9)
    for n in ("dQ", "dK", "dV"):
        np.testing.assert_allclose(g3[n], g1[n] + 2 * g2[n], rtol=1e-12, atol=1e-13)


def pin_selection(bwd):
    """rows / keys select rows of the full result."""
    rng = _rng(18)
    q, k, v, do = (rng.standard_normal((9, 3)) for _ in range(4))
    full = bwd(q, k, v, do, causal=True, scale=0.7)
    rows, keys = np.array([8, 0, 3]), np.array([2, 7])
    part = bwd(q, k, v, do, causal=True, scale=0.7, rows=rows, keys=keys)
    np.testing.assert_allclose(part["dQ"], full["dQ"][rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(part["Delta"], full["Delta"][rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(part["dK"], full["dK"][keys], rtol=0, atol=1e-14)
    np.testing.assert_allclose(part["dV"], full["dV"][keys], rtol=0, atol=1e-14)


ALL_BWD_PINS = [pin_finite_differences, pin_single_key, pin_equal_values,
                pin_key_shift_invariance, pin_causal_ends, pin_delta, pin_linear_in_do,
                pin_selection]
