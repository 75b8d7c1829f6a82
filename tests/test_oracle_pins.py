"""The oracle against what the pages and the mathematics fix (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from oracle import attention_head, online_attention_head, tile_local_softmax_head
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(attention_head)


def test_batched_wrapper_matches_heads():
    rng = np.random.Generator(np.random.PCG64(3))
    B, H, T, d = 2, 3, 9, 4
    q, k, v = (rng.standard_normal((B, H, T, d)) for _ in range(3))
    O, L = oracle.attention(q, k, v, causal=True, scale=0.5)
    rows = np.array([[0, 4], [1, 8], [2, 3], [5, 6], [7, 8], [0, 0]])
    Os, Ls = oracle.attention(q, k, v, causal=True, scale=0.5, rows=rows)
    for b in range(B):
        for h in range(H):
            r = attention_head(q[b, h], k[b, h], v[b, h], causal=True, scale=0.5)
            np.testing.assert_array_equal(O[b, h], r["O"])
            np.testing.assert_array_equal(L[b, h], r["LSE"])
            sel = rows[b * H + h]
            np.testing.assert_allclose(Os[b, h], r["O"][sel], rtol=0, atol=1e-14)
            np.testing.assert_allclose(Ls[b, h], r["LSE"][sel], rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# The method: the online recurrence reaches the materialised result for every
# tiling, while per-tile normalisation does not.
# [P2 section 3; P3 "Tiling and an incremental normalization"; P1 Figure 4]
# ---------------------------------------------------------------------------

def test_online_model_matches_oracle_every_tiling():
    rng = np.random.Generator(np.random.PCG64(7))
    for T in (1, 2, 5, 11, 16):
        for causal in (True, False):
            q, k, v = (rng.standard_normal((T, 4)) * 2.0 for _ in range(3))
            ref = attention_head(q, k, v, causal=causal, scale=0.9)
            for block in range(1, T + 1):
                got = online_attention_head(q, k, v, causal=causal, scale=0.9,
                                            block=block)
                np.testing.assert_allclose(got["O"], ref["O"], rtol=0, atol=1e-12)
                np.testing.assert_allclose(got["LSE"], ref["LSE"], rtol=0, atol=1e-12)


def test_online_model_large_scores():
    # scores spread over hundreds of units: the running max must rescale
    rng = np.random.Generator(np.random.PCG64(8))
    T = 16
    q, k, v = (rng.standard_normal((T, 8)) * 6.0 for _ in range(3))
    ref = attention_head(q, k, v, causal=True, scale=1.0)
    assert np.ptp(ref["S"][np.isfinite(ref["S"])]) > 200
    for block in (1, 3, 4, 7):
        got = online_attention_head(q, k, v, causal=True, scale=1.0, block=block)
        np.testing.assert_allclose(got["O"], ref["O"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(got["LSE"], ref["LSE"], rtol=0, atol=1e-10)


def test_tile_local_softmax_fails_two_score_exercise():
    # P3: independent one-element softmaxes give 1 and 1 instead of 1/4, 3/4.
    q = np.array([[0.3, -0.7], [1.0, 0.0]])
    k = np.array([[0.0, 0.0], [math.log(3.0), 0.0]])
    v = np.eye(2)
    bad = tile_local_softmax_head(q, k, v, causal=True, scale=1.0, block=1)
    np.testing.assert_allclose(bad["P"][1], [1.0, 1.0], rtol=0, atol=1e-15)
    good = online_attention_head(q, k, v, causal=True, scale=1.0, block=1)
    np.testing.assert_allclose(good["O"][1], [0.25, 0.75], rtol=0, atol=1e-12)


def test_tile_local_softmax_fails_fig4():
    # P1 Figure 4: normalising [0, 0] alone gives 50 % each, not 6 %.
    q = np.ones((4, 1))
    k = np.array([[0.0], [0.0], [2.0], [2.0]])
    v = np.eye(4)
    bad = tile_local_softmax_head(q, k, v, causal=False, scale=1.0, block=2)
    ref = attention_head(q, k, v, causal=False, scale=1.0)
    assert bad["P"][0, 0] == pytest.approx(0.5, abs=1e-15)
    assert ref["P"][0, 0] == pytest.approx(1 / (2 + 2 * math.e ** 2), abs=1e-12)
    assert np.abs(bad["O"] - ref["O"]).max() > 0.4


def test_tile_local_softmax_fails_random():
    rng = np.random.Generator(np.random.PCG64(9))
    T = 16
    q, k, v = (rng.standard_normal((T, 4)) for _ in range(3))
    ref = attention_head(q, k, v, causal=False, scale=1.0)
    for block in (1, 2, 4, 8):
        bad = tile_local_softmax_head(q, k, v, causal=False, scale=1.0, block=block)
        # a row spread over n tiles gets total weight n instead of 1
        np.testing.assert_allclose(bad["P"].sum(axis=1), T // block, atol=1e-12)
        assert np.abs(bad["O"] - ref["O"]).max() > 0.4
    same = tile_local_softmax_head(q, k, v, causal=False, scale=1.0, block=T)
    np.testing.assert_allclose(same["O"], ref["O"], rtol=0, atol=1e-12)
