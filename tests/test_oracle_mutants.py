"""Mutation tests for the oracle's pins (CPU only).

Each mutant is a copy of the materialised oracle with one plausible mistake
planted in it (a dropped term, a wrong sign or index, a transposed operand).
The pins in ``oracle_pins`` must reject every one of them; a mutant that
passes all pins would mean the pins could not tell that mistake from the
correct oracle.
"""
import numpy as np
import pytest

from oracle import attention_head
from oracle_pins import ALL_PINS


def _variant(q, k, v, *, causal, scale, rows=None, mutation=None):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T = k.shape[0]
    r = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    if mutation == "rows_ignored":
        r = np.arange(T)
    raw = q[r] @ k.T
    if mutation == "transpose_scores":
        raw = (k @ q.T)[r]
    if mutation == "drop_last_key":
        raw = raw.copy()
        raw[:, -1] = -np.inf if T > 1 else raw[:, -1]
    if mutation == "no_scale":
        S = raw
    elif mutation == "divide_scale":
        with np.errstate(divide="ignore", invalid="ignore"):
            S = raw / scale
    elif mutation == "mask_before_scale":
        S = raw
    else:
        S = scale * raw
    if causal:
        cols = np.arange(T)[None, :]
        if mutation == "mask_past":
            masked = cols < r[:, None]
        elif mutation == "mask_diagonal":
            masked = cols >= r[:, None]
        else:
            masked = cols > r[:, None]
        S = np.where(masked, -np.inf, S)
    if mutation == "mask_before_scale":
        with np.errstate(invalid="ignore"):
            S = scale * S
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        m = S.max(axis=1, keepdims=True)
        if mutation == "no_exp":
            E = np.where(np.isfinite(S), S - m, 0.0)
        elif mutation == "max_added":
            E = np.exp(S + m)
        else:
            E = np.exp(S - m)
        if mutation == "softmax_cols":
            l = E.sum(axis=0, keepdims=True)
        else:
            l = E.sum(axis=1, keepdims=True)
        P = E if mutation == "no_normalise" else E / l
        vv = np.roll(v, 1, axis=0) if mutation == "value_rows_shifted" else v
        O = P.T @ vv if mutation == "pv_transposed" else P @ vv
        if mutation == "softmax_cols":
            l = l.T
        if mutation == "lse_no_max":
            LSE = np.log(l[:, 0])
        elif mutation == "lse_log2":
            LSE = m[:, 0] + np.log2(l[:, 0])
        elif mutation == "lse_of_mean":
            LSE = m[:, 0] + np.log(l[:, 0] / T)
        else:
            LSE = m[:, 0] + np.log(l[:, 0])
    return {"S": S, "P": P, "O": O, "LSE": LSE, "rows": r}


MUTATIONS = [
    "transpose_scores", "drop_last_key", "no_scale", "divide_scale",
    "mask_before_scale", "mask_past", "mask_diagonal", "no_exp", "max_added",
    "softmax_cols", "no_normalise", "value_rows_shifted", "pv_transposed",
    "lse_no_max", "lse_log2", "lse_of_mean", "rows_ignored",
]


def _failures(fn):
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


def test_unmutated_copy_passes_all_pins():
    assert _failures(lambda *a, **kw: _variant(*a, **kw, mutation=None)) == []
    assert _failures(attention_head) == []


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_pins_catch_mutation(mutation):
    failed = _failures(lambda *a, **kw: _variant(*a, **kw, mutation=mutation))
    assert failed, f"no pin catches the planted mistake {mutation!r}"


# ---------------------------------------------------------------------------
# Planted mistakes in the online recurrence are caught by comparing it with
# the materialised oracle over every tiling.
# ---------------------------------------------------------------------------

def _online_variant(q, k, v, causal, scale, block, mutation):
    T = q.shape[0]
    rows = np.arange(T)
    m = np.full(T, -np.inf)
    l = np.zeros(T)
    acc = np.zeros((T, v.shape[1]))
    for start in range(0, T, block):
        cols = np.arange(start, min(start + block, T))
        s = scale * (q @ k[cols].T)
        if causal:
            s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
        m_new = np.maximum(m, s.max(axis=1))
        base = np.where(np.isneginf(m_new), 0.0, m_new)
        alpha = np.exp(m - base)
        if mutation == "alpha_inverted":
            alpha = np.exp(base - m)
        p = np.exp(s - base[:, None])
        l = (l if mutation == "no_alpha_l" else alpha * l) + p.sum(axis=1)
        acc = (acc if mutation == "no_alpha_acc" else alpha[:, None] * acc) + p @ v[cols]
        if mutation != "max_not_carried":
            m = m_new
    return acc / l[:, None], m + np.log(l)


@pytest.mark.parametrize("mutation", ["alpha_inverted", "no_alpha_l",
                                      "no_alpha_acc", "max_not_carried"])
def test_online_mutations_detected(mutation):
    rng = np.random.Generator(np.random.PCG64(5))
    T = 12
    q, k, v = (rng.standard_normal((T, 4)) * 2.0 for _ in range(3))
    ref = attention_head(q, k, v, causal=True, scale=1.0)
    worst = 0.0
    with np.errstate(all="ignore"):
        for block in range(1, T):
            O, L = _online_variant(q, k, v, True, 1.0, block, mutation)
            diff = np.concatenate([O.ravel() - ref["O"].ravel(), L - ref["LSE"]])
            err = np.inf if np.isnan(diff).all() else np.nanmax(np.abs(diff))
            if not np.all(np.isfinite(O)):
                err = np.inf
            worst = max(worst, err)
    assert worst > 1e-3
