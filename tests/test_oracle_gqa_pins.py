"""Pins of the grouped-query oracle (CPU only), and mutants it must reject.

- H_kv = H is ordinary attention head by head;
- query heads of one group that carry equal queries give equal outputs, and
  the same queries in another group (other keys) do not: this fixes which
  query heads share a key/value head;
- H_kv = 1 (one key/value head) with equal queries gives equal outputs in
  every head;
- the key/value gradients equal central differences of sum(dO * O) through
  the grouped forward, so they sum over the whole group.
"""
import numpy as np
import pytest

from oracle import attention, attention_gqa, attention_gqa_bwd, attention_head


def _rng(s):
    return np.random.Generator(np.random.PCG64(s))


def pin_reduces_to_mha(fwd, bwd):
    rng = _rng(31)
    q, k, v = (rng.standard_normal((2, 3, 6, 4)) for _ in range(3))
    O, L = fwd(q, k, v, causal=True, scale=0.8)
    O2, L2 = attention(q, k, v, causal=True, scale=0.8)
    np.testing.assert_allclose(O, O2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(L, L2, rtol=0, atol=1e-14)


def pin_group_membership(fwd, bwd):
    rng = _rng(32)
    B, H, Hkv, T, d = 1, 6, 2, 7, 3     # groups {0,1,2} and {3,4,5}
    k, v = (rng.standard_normal((B, Hkv, T, d)) for _ in range(2))
    q = rng.standard_normal((B, H, T, d))
    q[:, 1] = q[:, 0]
    q[:, 2] = q[:, 0]
    q[:, 3] = q[:, 0]
    O, _ = fwd(q, k, v, causal=False, scale=0.9)
    np.testing.assert_allclose(O[:, 1], O[:, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(O[:, 2], O[:, 0], rtol=0, atol=1e-15)
    assert np.abs(O[:, 3] - O[:, 0]).max() > 1e-3  # other group, other keys
    # and head 0 is plain attention against key/value head 0
    r = attention_head(q[0, 0], k[0, 0], v[0, 0], causal=False, scale=0.9)
    np.testing.assert_allclose(O[0, 0], r["O"], rtol=0, atol=1e-15)
    r = attention_head(q[0, 5], k[0, 1], v[0, 1], causal=False, scale=0.9)
    np.testing.assert_allclose(O[0, 5], r["O"], rtol=0, atol=1e-15)


def pin_single_kv_head(fwd, bwd):
    rng = _rng(33)
    k, v = (rng.standard_normal((1, 1, 5, 3)) for _ in range(2))
    q = np.repeat(rng.standard_normal((1, 1, 5, 3)), 4, axis=1)
    O, _ = fwd(q, k, v, causal=True, scale=1.2)
    for h in range(1, 4):
        np.testing.assert_allclose(O[:, h], O[:, 0], rtol=0, atol=1e-15)


def pin_finite_differences(fwd, bwd):
    rng = _rng(34)
    B, H, Hkv, T, d = 1, 4, 2, 3, 2
    q, do = (rng.standard_normal((B, H, T, d)) for _ in range(2))
    k, v = (rng.standard_normal((B, Hkv, T, d)) for _ in range(2))
    for causal in (True, False):
        dQ, dK, dV = bwd(q, k, v, do, causal=causal, scale=0.7)

        def loss(qq, kk, vv):
            return float((fwd(qq, kk, vv, causal=causal, scale=0.7)[0] * do).sum())

        h = 1e-5
        for name, x, g in (("dQ", q, dQ), ("dK", k, dK), ("dV", v, dV)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args = {"dQ": lambda z: (z, k, v), "dK": lambda z: (q, z, v),
                        "dV": lambda z: (q, k, z)}[name]
                num[idx] = (loss(*args(xp)) - loss(*args(xm))) / (2 * h)
            np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


ALL_GQA_PINS = [pin_reduces_to_mha, pin_group_membership, pin_single_kv_head,
                pin_finite_differences]


@pytest.mark.parametrize("pin", ALL_GQA_PINS, ids=lambda p: p.__name__)
def test_gqa_oracle_pin(pin):
    pin(attention_gqa, attention_gqa_bwd)


def _mutant(mutation):
    def kvh(h, H, Hkv):
        return h % Hkv if mutation == "modulo_map" else h // (H // Hkv)

    def fwd(q, k, v, *, causal, scale, rows=None):
        B, H, T, d = q.shape
        res = [[attention_head(q[b, h], k[b, kvh(h, H, k.shape[1])],
                               v[b, kvh(h, H, k.shape[1])], causal=causal, scale=scale)
                for h in range(H)] for b in range(B)]
        return (np.stack([[r["O"] for r in rb] for rb in res]),
                np.stack([[r["LSE"] for r in rb] for rb in res]))

    def bwd(q, k, v, do, *, causal, scale):
        from oracle import attention_head_bwd
        B, H, T, d = q.shape
        Hkv = k.shape[1]
        dQ, dK, dV = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
        for b in range(B):
            for h in range(H):
                g = kvh(h, H, Hkv)
                r = attention_head_bwd(q[b, h], k[b, g], v[b, g], do[b, h], causal=causal,
                                       scale=scale)
                dQ[b, h] = r["dQ"]
                if mutation == "first_member_only":
                    if h % (H // Hkv) == 0:
                        dK[b, g], dV[b, g] = r["dK"], r["dV"]
                elif mutation == "last_member_overwrites":
                    dK[b, g], dV[b, g] = r["dK"], r["dV"]
                else:
                    dK[b, g] += r["dK"]
                    dV[b, g] += r["dV"]
        return dQ, dK, dV
    return fwd, bwd


@pytest.mark.parametrize("mutation", ["modulo_map", "first_member_only",
                                      "last_member_overwrites"])
def test_gqa_pins_reject_mutant(mutation):
    fwd, bwd = _mutant(mutation)
    failed = []
    for pin in ALL_GQA_PINS:
        try:
            pin(fwd, bwd)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, mutation


def test_unmutated_scaffold_passes():
    fwd, bwd = _mutant(None)
    for pin in ALL_GQA_PINS:
        pin(fwd, bwd)
