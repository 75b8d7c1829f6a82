"""Pins of the decode oracle (CPU only), and mutants it must reject.

- the new queries are the last rows of the square causal forward over the
  same keys and values (whatever the earlier queries were);
- one new query under the causal mask sees the whole cache, so it equals
  the unmasked result;
- the first key is always visible and masked keys carry zero weight;
- splitting the keys into consecutive chunks and merging the chunks' (O, LSE)
  by LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s reproduces the
  whole (the algebra a split-key decode relies on, checked on the oracle's
  own chunk results).
"""
import numpy as np
import pytest

from oracle import attention_decode_head, attention_head


def _rng(s):
    return np.random.Generator(np.random.PCG64(s))


def pin_last_rows_of_square(fn):
    rng = _rng(41)
    for Tq, Tk in ((1, 1), (1, 9), (3, 9), (9, 9), (4, 17)):
        k, v = (rng.standard_normal((Tk, 4)) for _ in range(2))
        qfull = rng.standard_normal((Tk, 4))
        for causal in (True, False):
            sq = attention_head(qfull, k, v, causal=causal, scale=0.8)
            r = fn(qfull[Tk - Tq:], k, v, causal=causal, scale=0.8)
            np.testing.assert_allclose(r["O"], sq["O"][Tk - Tq:], rtol=0, atol=1e-14)
            np.testing.assert_allclose(r["LSE"], sq["LSE"][Tk - Tq:], rtol=0, atol=1e-14)


def pin_single_query_sees_all(fn):
    rng = _rng(42)
    q = rng.standard_normal((1, 5))
    k, v = (rng.standard_normal((23, 5)) for _ in range(2))
    a = fn(q, k, v, causal=True, scale=0.6)
    b = fn(q, k, v, causal=False, scale=0.6)
    np.testing.assert_allclose(a["O"], b["O"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(a["LSE"], b["LSE"], rtol=0, atol=1e-15)


def pin_visibility(fn):
    rng = _rng(43)
    Tq, Tk = 4, 10
    q = rng.standard_normal((Tq, 3))
    k, v = (rng.standard_normal((Tk, 3)) for _ in range(2))
    r = fn(q, k, v, causal=True, scale=1.0)
    P = r["P"]
    for i in range(Tq):
        assert np.all(P[i, Tk - Tq + i + 1:] == 0.0)
        assert np.all(P[i, :Tk - Tq + i + 1] > 0.0)
    np.testing.assert_allclose(P.sum(1), 1.0, rtol=0, atol=1e-14)


def pin_chunk_merge(fn):
    rng = _rng(44)
    Tq, Tk, d = 3, 40, 4
    q = rng.standard_normal((Tq, d)) * 2
    k, v = (rng.standard_normal((Tk, d)) * 2 for _ in range(2))
    whole = fn(q, k, v, causal=False, scale=0.9)
    for cuts in ([0, 40], [0, 13, 40], [0, 1, 2, 39, 40], list(range(0, 41, 8))):
        parts = [fn(q, k[a:b], v[a:b], causal=False, scale=0.9)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        Ls = np.stack([p["LSE"] for p in parts])
        L = np.log(np.exp(Ls - Ls.max(0)).sum(0)) + Ls.max(0)
        O = sum(np.exp(p["LSE"] - L)[:, None] * p["O"] for p in parts)
        np.testing.assert_allclose(O, whole["O"], rtol=0, atol=1e-13)
        np.testing.assert_allclose(L, whole["LSE"], rtol=0, atol=1e-13)


ALL_DECODE_PINS = [pin_last_rows_of_square, pin_single_query_sees_all, pin_visibility,
                   pin_chunk_merge]


@pytest.mark.parametrize("pin", ALL_DECODE_PINS, ids=lambda p: p.__name__)
def test_decode_oracle_pin(pin):
    pin(attention_decode_head)


def _mutant(mutation):
    def fn(q, k, v, *, causal, scale):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        Tq, Tk = q.shape[0], k.shape[0]
        S = scale * (q @ k.T)
        if causal:
            if mutation == "top_left_mask":
                pos = np.arange(Tq)
            elif mutation == "off_by_one":
                pos = Tk - Tq + np.arange(Tq) - 1
            else:
                pos = Tk - Tq + np.arange(Tq)
            S = np.where(np.arange(Tk)[None, :] > pos[:, None], -np.inf, S)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        l = E.sum(axis=1, keepdims=True)
        P = E / l
        L = m[:, 0] + np.log(l[:, 0])
        if mutation == "lse_without_max":
            L = np.log(l[:, 0])
        return {"O": P @ v, "LSE": L, "P": P}
    return fn


@pytest.mark.parametrize("mutation", ["top_left_mask", "off_by_one", "lse_without_max"])
def test_decode_pins_reject_mutant(mutation):
    failed = []
    for pin in ALL_DECODE_PINS:
        try:
            pin(_mutant(mutation))
        except (AssertionError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, mutation


def test_unmutated_scaffold_passes():
    for pin in ALL_DECODE_PINS:
        pin(_mutant(None))
