"""Property tests of the oracle over generated shapes, scales and inputs
(Hypothesis): the invariants the source pages fix, checked on many random
cases instead of a few fixed ones.

- rows of P are probability distributions, masked entries exactly zero
  ("Why Attention Is Difficult to Optimize", Figure 1 and "From a Score Tile
  to Probabilities");
- the tiled online recurrence gives the materialised result for any tile
  size ("Attention Mechanism: Computation & Memory Patterns", section 3;
  "FlashAttention -- avoid writing the giant intermediate", "Tiling and an
  incremental normalization");
- a query row depends only on the keys it may see and on no other query row
  ("Why Attention...", "Tile the problem");
- a scalar brute force (math.exp, math.fsum) agrees on tiny problems;
- textbook facts of the softmax: shift of the keys, linearity in V;
- decode rows are the last rows of the square forward, grouped heads are
  ordinary heads over their group's keys and values.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from oracle.decode import attention_decode_head
from oracle.gqa import attention_gqa
from oracle.online_model import online_attention_head

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

SETTINGS = settings(max_examples=60, deadline=None)


@st.composite
def problems(draw, max_t=24, max_d=8):
    T = draw(st.integers(1, max_t))
    d = draw(st.integers(1, max_d))
    causal = draw(st.booleans())
    scale = draw(st.floats(-2.0, 2.0, allow_nan=False, allow_infinity=False))
    amp = draw(st.sampled_from([0.1, 1.0, 5.0]))
    seed = draw(st.integers(0, 2**32 - 1))
    rng = np.random.Generator(np.random.PCG64(seed))
    q, k, v = (amp * rng.standard_normal((T, d)) for _ in range(3))
    return q, k, v, causal, scale


@SETTINGS
@given(problems())
def test_rows_are_distributions(prob):
    q, k, v, causal, scale = prob
    T = q.shape[0]
    P = oracle.attention_head(q, k, v, causal=causal, scale=scale)["P"]
    assert (P >= 0).all()
    assert np.abs(P.sum(axis=1) - 1.0).max() <= 1e-12
    if causal:
        assert (P[np.triu_indices(T, 1)] == 0.0).all()


@SETTINGS
@given(problems(), st.integers(1, 24))
def test_online_recurrence_any_tile(prob, block):
    q, k, v, causal, scale = prob
    T = q.shape[0]
    ref = oracle.attention_head(q, k, v, causal=causal, scale=scale)
    got = online_attention_head(q, k, v, causal=causal, scale=scale, block=min(block, T))
    assert np.abs(got["O"] - ref["O"]).max() <= 1e-10 * (1 + np.abs(v).max())
    assert np.abs(got["LSE"] - ref["LSE"]).max() <= 1e-10 * (1 + np.abs(ref["LSE"]).max())


@settings(max_examples=40, deadline=None)
@given(problems(max_t=7, max_d=4))
def test_scalar_brute_force(prob):
    q, k, v, causal, scale = prob
    T, d = q.shape
    ref = oracle.attention_head(q, k, v, causal=causal, scale=scale)
    for i in range(T):
        keys = range(i + 1) if causal else range(T)
        s = [scale * math.fsum(q[i, c] * k[j, c] for c in range(d)) for j in keys]
        top = max(s)
        w = [math.exp(x - top) for x in s]
        total = math.fsum(w)
        assert abs(top + math.log(total) - ref["LSE"][i]) <= 1e-11 * (1 + abs(ref["LSE"][i]))
        for c in range(d):
            o = math.fsum(wj * v[j, c] for wj, j in zip(w, keys)) / total
            assert abs(o - ref["O"][i, c]) <= 1e-11 * (1 + np.abs(v).max())


@SETTINGS
@given(problems(), st.data())
def test_future_keys_and_other_queries_do_not_matter(prob, data):
    q, k, v, causal, scale = prob
    T, d = q.shape
    ref = oracle.attention_head(q, k, v, causal=causal, scale=scale)
    i0 = data.draw(st.integers(0, T - 1))
    rng = np.random.Generator(np.random.PCG64(data.draw(st.integers(0, 2**32 - 1))))
    # another query row changed: row i0 unchanged
    q2 = q.copy()
    others = [i for i in range(T) if i != i0]
    if others:
        q2[others] += rng.standard_normal((len(others), d))
        got = oracle.attention_head(q2, k, v, causal=causal, scale=scale)
        assert np.abs(got["O"][i0] - ref["O"][i0]).max() <= 1e-12 * (1 + np.abs(v).max())
        assert abs(got["LSE"][i0] - ref["LSE"][i0]) <= 1e-12 * (1 + abs(ref["LSE"][i0]))
    # causal: keys and values after i0 changed: rows <= i0 unchanged
    if causal and i0 + 1 < T:
        k2, v2 = k.copy(), v.copy()
        k2[i0 + 1:] += 3.0 * rng.standard_normal((T - i0 - 1, d))
        v2[i0 + 1:] += 3.0 * rng.standard_normal((T - i0 - 1, d))
        got = oracle.attention_head(q, k2, v2, causal=True, scale=scale)
        assert np.abs(got["O"][: i0 + 1] - ref["O"][: i0 + 1]).max() <= 1e-12 * (
            1 + np.abs(v).max())
        assert np.abs(got["LSE"][: i0 + 1] - ref["LSE"][: i0 + 1]).max() <= 1e-12 * (
            1 + np.abs(ref["LSE"]).max())


@SETTINGS
@given(problems(), st.data())
def test_key_shift_and_value_linearity(prob, data):
    q, k, v, causal, scale = prob
    T, d = q.shape
    rng = np.random.Generator(np.random.PCG64(data.draw(st.integers(0, 2**32 - 1))))
    ref = oracle.attention_head(q, k, v, causal=causal, scale=scale)
    # the same vector added to every key: O unchanged, LSE_i + scale q_i . u
    u = rng.standard_normal(d)
    got = oracle.attention_head(q, k + u, v, causal=causal, scale=scale)
    tol = 1e-9 * (1 + np.abs(ref["LSE"]).max() + np.abs(scale * q @ u).max())
    assert np.abs(got["O"] - ref["O"]).max() <= 1e-9 * (1 + np.abs(v).max())
    assert np.abs(got["LSE"] - (ref["LSE"] + scale * (q @ u))).max() <= tol
    # O is linear in V for fixed Q and K
    w = rng.standard_normal((T, d))
    a, b = data.draw(st.floats(-3, 3)), data.draw(st.floats(-3, 3))
    lin = oracle.attention_head(q, k, a * v + b * w, causal=causal, scale=scale)["O"]
    ow = oracle.attention_head(q, k, w, causal=causal, scale=scale)["O"]
    assert np.abs(lin - (a * ref["O"] + b * ow)).max() <= 1e-10 * (
        1 + abs(a) * np.abs(v).max() + abs(b) * np.abs(w).max())


@SETTINGS
@given(problems(), st.data())
def test_decode_is_the_tail_of_the_square_forward(prob, data):
    q, k, v, causal, scale = prob
    T = q.shape[0]
    tq = data.draw(st.integers(1, T))
    ref = oracle.attention_head(q, k, v, causal=causal, scale=scale)
    got = attention_decode_head(q[T - tq:], k, v, causal=causal, scale=scale)
    assert np.abs(got["O"] - ref["O"][T - tq:]).max() <= 1e-12 * (1 + np.abs(v).max())
    assert np.abs(got["LSE"] - ref["LSE"][T - tq:]).max() <= 1e-12 * (
        1 + np.abs(ref["LSE"]).max())


@SETTINGS
@given(st.integers(1, 12), st.integers(1, 6), st.sampled_from([(2, 1), (4, 2), (6, 3), (3, 3)]),
       st.booleans(), st.integers(0, 2**32 - 1))
def test_grouped_heads_are_ordinary_heads(T, d, heads, causal, seed):
    H, H_kv = heads
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((1, H, T, d))
    k = rng.standard_normal((1, H_kv, T, d))
    v = rng.standard_normal((1, H_kv, T, d))
    scale = 1.0 / math.sqrt(d)
    O, L = attention_gqa(q, k, v, causal=causal, scale=scale)
    G = H // H_kv
    for h in range(H):
        ref = oracle.attention_head(q[0, h], k[0, h // G], v[0, h // G], causal=causal,
                                    scale=scale)
        assert np.abs(O[0, h] - ref["O"]).max() <= 1e-12 * (1 + np.abs(v).max())
        assert np.abs(L[0, h] - ref["LSE"]).max() <= 1e-12 * (1 + np.abs(ref["LSE"]).max())
