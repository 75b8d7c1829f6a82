"""The seeded input generator (CPU only)."""
import numpy as np
import pytest

from seeded_inputs import (WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits,
                           make_qkv, sample_rows)


def test_bf16_round_nearest_even_known_values():
    # exact, halfway-to-even and above/below-halfway cases, by bit pattern
    cases = {
        0x3F800000: 0x3F80,  # 1.0 exact
        0x3F808000: 0x3F80,  # halfway, kept lsb even -> down
        0x3F818000: 0x3F82,  # halfway, kept lsb odd -> up
        0x3F808001: 0x3F81,  # just above halfway -> up
        0x3F807FFF: 0x3F80,  # just below halfway -> down
        0xBF808001: 0xBF81,  # negative, above halfway
        0x7F7FFFFF: 0x7F80,  # max finite float rounds to +inf
        0x00000001: 0x0000,  # smallest subnormal -> +0
        0x80000000: 0x8000,  # -0
    }
    x = np.array(list(cases), dtype=np.uint32).view(np.float32)
    got = f32_to_bf16_bits(x)
    np.testing.assert_array_equal(got, np.array(list(cases.values()), dtype=np.uint16))


def test_bf16_matches_torch_rounding():
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(0))
    x = rng.standard_normal(200_000, dtype=np.float32) * np.float32(37.0)
    ours = f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)


def test_bf16_widening_is_exact():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(bits)
    finite = np.isfinite(f)
    np.testing.assert_array_equal(f32_to_bf16_bits(f[finite]), bits[finite])


def test_draws_are_seeded_and_ordered():
    a = make_qkv(1, 2, 8, 4, dtype="bf16", seed=4, qk_mult=4.0)
    b = make_qkv(1, 2, 8, 4, dtype="bf16", seed=4, qk_mult=4.0)
    c = make_qkv(1, 2, 8, 4, dtype="bf16", seed=4, qk_mult=1.0)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        np.testing.assert_array_equal(x, y)
    # Q and K scaled by 4 exactly (a power of two commutes with rounding); V not
    np.testing.assert_array_equal(a.q64(), 4.0 * c.q64())
    np.testing.assert_array_equal(a.k64(), 4.0 * c.k64())
    np.testing.assert_array_equal(a.v64(), c.v64())
    f = make_qkv(1, 2, 8, 4, dtype="f32", seed=4)
    assert f.q.dtype == np.float32
    np.testing.assert_array_equal(f32_to_bf16_bits(f.q), c.q)


def test_sample_rows_distinct_and_bounded():
    r = sample_rows(65536, 512, seed=1005, heads=8)
    assert r.shape[0] == 8
    for row in r:
        assert row[0] == 0 and row[-1] == 65535
        assert np.all(np.diff(row) >= 0)
        assert len(np.unique(row)) >= 512


def test_workload_table():
    for name, w in WORKLOADS.items():
        assert w["dtype"] in ("bf16", "f32")
        assert w["d"] in (64, 128)
        assert name.startswith(w["dtype"])
