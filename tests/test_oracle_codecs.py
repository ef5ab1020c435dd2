"""Pins of the oracle's number-format codecs against things other than itself:
the formats' closed-form definitions, torch's float8_e4m3fn / bfloat16 casts
(library routines), an independent threshold-form encoder, and exhaustive
sweeps of the fp32 ranges the quantizer reaches."""
import numpy as np
import pytest
import torch

import oracle as O


def _f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


# ---------------------------------------------------------------- E2M1 ----

def test_e2m1_decode_matches_format_definition():
    # E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
    # subnormal: m * 2^(1 - bias) * 1/2.
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        want = -mag if s else mag
        got = O.lib().ora_e2m1_decode(c)
        assert got == want and np.signbit(got) == bool(s), (c, got, want)
    assert sorted({abs(O.lib().ora_e2m1_decode(c)) for c in range(16)}) == [0, .5, 1, 1.5, 2, 3, 4, 6]


def test_e2m1_roundtrip_all_codes():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(O.e2m1_encode(O.e2m1_decode(codes)), codes)


def test_e2m1_ties_go_to_even_code_and_saturate():
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 6.0: 7, 7.0: 7, 1e30: 7,
             np.inf: 7, 0.0: 0, 1e-45: 0}
    for y, want in cases.items():
        assert O.lib().ora_e2m1_encode(y) == want, y
        assert O.lib().ora_e2m1_encode(-y) == want | 8, -y


def _e2m1_threshold(y):
    """The same rounding rule written as comparisons against the midpoints
    between neighbouring magnitudes; at a midpoint the even code wins."""
    a = np.abs(y.astype(np.float64))
    m = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5)
         + (a > 5.0)).astype(np.uint8)
    return m | (np.signbit(y).astype(np.uint8) << 3)


def test_e2m1_exhaustive_sweep_vs_threshold_form():
    # Every fp32 pattern with 2^-7 <= |y| < 16 (both signs): all rounding
    # boundaries of E2M1 and the saturation region lie inside.
    lo, hi = 0x3C000000, 0x41800000
    step = 1 << 24
    for sign in (0, 0x80000000):
        for start in range(lo, hi, step):
            bits = np.arange(start, min(start + step, hi), dtype=np.uint32) | np.uint32(sign)
            y = bits.view(np.float32)
            assert np.array_equal(O.e2m1_encode(y), _e2m1_threshold(y)), hex(start)


def test_e2m1_sampled_sweep_outside_dense_range():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    y = bits.view(np.float32)
    y = y[~np.isnan(y)]
    assert np.array_equal(O.e2m1_encode(y), _e2m1_threshold(y))


def test_e2m1_is_nearest_by_brute_force():
    rng = np.random.default_rng(8)
    y = (rng.standard_normal(200_000) * 3).astype(np.float32)
    q = O.e2m1_encode(y)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    d = np.abs(np.abs(y.astype(np.float64))[:, None] - grid[None, :])
    best = d.min(axis=1)
    assert np.all(d[np.arange(y.size), q & 7] == best)


# ---------------------------------------------------------------- E4M3 ----

def _e4m3_formula(b):
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        return np.nan
    mag = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -mag if s else mag


def test_e4m3_decode_all_bytes_vs_formula_and_torch():
    b = np.arange(256, dtype=np.uint8)
    got = O.e4m3_decode(b)
    lib_vals = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for i in range(256):
        want = _e4m3_formula(i)
        if np.isnan(want):
            assert np.isnan(got[i]) and np.isnan(lib_vals[i])
        else:
            assert got[i] == want == lib_vals[i], i
            assert np.signbit(got[i]) == np.signbit(lib_vals[i])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def _torch_e4m3(r):
    return torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_exhaustive_vs_torch_cast():
    # torch's float8_e4m3fn cast rounds to nearest even and keeps subnormals;
    # it does not saturate, so the sweep stops below 464 (448 + half a step),
    # which is the quantizer's whole domain: every non-negative fp32 pattern
    # from 2^-12 (everything smaller encodes to 0) up to 464.
    lo, hi = 0x39800000, 0x43E80000
    step = 1 << 24
    for start in range(lo, hi, step):
        r = np.arange(start, min(start + step, hi), dtype=np.uint32).view(np.float32)
        assert np.array_equal(O.e4m3_encode(r), _torch_e4m3(r)), hex(start)


def test_e4m3_encode_small_values_and_saturation():
    rng = np.random.default_rng(9)
    small = rng.integers(0, 0x39800000, size=2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    assert not O.e4m3_encode(small).any()
    assert np.array_equal(O.e4m3_encode(small), _torch_e4m3(small))
    big = np.array([448.0, 463.99997, 464.0, 500.0, 1e10], np.float32)
    assert list(O.e4m3_encode(big)) == [0x7E] * 5
    # sign symmetry
    r = rng.uniform(0, 460, 100_000).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(-r), O.e4m3_encode(r) | 0x80)


# ---------------------------------------------------------------- bf16 ----

def test_bf16_round_vs_torch_cast():
    rng = np.random.default_rng(10)
    bits = rng.integers(0, 1 << 32, size=8_000_000, dtype=np.uint64).astype(np.uint32)
    # add exact ties (low half 0x8000) and their neighbours around both parities
    hi = rng.integers(0, 1 << 16, size=200_000, dtype=np.uint64).astype(np.uint32) << 16
    bits = np.concatenate([bits, hi | 0x8000, hi | 0x7FFF, hi | 0x8001, hi,
                           np.array([0x7F7F8000, 0x7F7F7FFF, 0xFF7F8000, 0x00008000, 0x80008000], np.uint32)])
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.float_to_bf16(x), want)


def test_bf16_widen_is_exact():
    h = np.arange(1 << 16, dtype=np.uint16)
    f = O.bf16_to_float(h)
    lib_vals = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    ok = ~np.isnan(lib_vals)
    assert np.array_equal(f.view(np.uint32)[ok], lib_vals.view(np.uint32)[ok])
    assert all(O.lib().ora_bf16_to_float(int(v)) == f[v] for v in h[ok][::257])


# ------------------------------------------------------ candidate scale ----

def test_candidate_codes_are_e4m3_of_fp32_quotient():
    rng = np.random.default_rng(11)
    t = np.concatenate([rng.uniform(0, 1792, 500_000), rng.uniform(0, 0.05, 100_000),
                        np.arange(0, 1793, 0.125)]).astype(np.float32)
    for c in (6.0, 4.0):
        q = (t / np.float32(c)).astype(np.float32)  # numpy: one IEEE fp32 division
        assert np.array_equal(O.candidate_codes(t, c), _torch_e4m3(q))
