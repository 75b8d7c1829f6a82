"""The backward oracle against its pins, and mutants of it against the same
pins (CPU only).

Each mutant repeats the backward with one plausible mistake planted (a
dropped term, a wrong sign, a transposed operand, a missing or wrong scale,
a wrong reduction axis); every one must fail at least one pin.
"""
import numpy as np
import pytest

from oracle import attention_head, attention_head_bwd
from oracle_bwd_pins import ALL_BWD_PINS


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=lambda p: p.__name__)
def test_bwd_oracle_pin(pin):
    pin(attention_head_bwd)


def _mutant(mutation):
    def bwd(q, k, v, do, *, causal, scale, rows=None, keys=None):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        T = k.shape[0]
        r = np.arange(T) if rows is None else np.asarray(rows)
        j = np.arange(T) if keys is None else np.asarray(keys)
        P = attention_head(q, k, v, causal=causal, scale=scale)["P"]
        dP = do @ v.T
        dV = (P @ do) if mutation == "dv_untransposed" else P.T @ do
        if mutation == "delta_axis":
            Delta = (P * dP).sum(axis=0)
        else:
            Delta = (P * dP).sum(axis=1)
        if mutation == "drop_delta":
            dS = P * dP
        elif mutation == "delta_sign":
            dS = P * (Delta[:, None] - dP)
        elif mutation == "no_p_factor":
            dS = dP - Delta[:, None]
        else:
            dS = P * (dP - Delta[:, None])
        sq = 1.0 if mutation == "dq_no_scale" else scale
        dQ = sq * ((dS.T if mutation == "dq_transposed" else dS) @ k)
        xk = k if mutation == "dk_uses_k" else q
        dK = scale * (dS.T @ xk)
        return {"dQ": dQ[r], "dK": dK[j], "dV": dV[j], "Delta": Delta[r]}
    return bwd


MUTATIONS = ["dv_untransposed", "delta_axis", "drop_delta", "delta_sign", "no_p_factor",
             "dq_no_scale", "dq_transposed", "dk_uses_k"]


def test_unmutated_copy_passes():
    # the mutant scaffold itself is correct when nothing is planted
    for pin in ALL_BWD_PINS:
        pin(_mutant(None))


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_pins_reject_mutant(mutation):
    failed = []
    for pin in ALL_BWD_PINS:
        try:
            pin(_mutant(mutation))
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin rejects the mutant {mutation}"
