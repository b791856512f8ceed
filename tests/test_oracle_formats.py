"""Pins for the oracle's number formats (CPU only).

* bf16 round-to-nearest-even against torch's CPU float32 -> bfloat16 cast (a library routine
  that rounds to nearest even), exhaustively over whole binades plus a dense random sample.
* OCP E4M3 (OFP8 spec, rev. 1.0) with round-to-nearest-even and saturation at 448: against the
  spec's printed code values (tests/golden/ofp8_e4m3_codes.txt), torch's CPU float8_e4m3fn
  cast (round to nearest even; it agrees with saturation for |v| <= 464), an independent
  nearest-value search over the decoded table, every code, every midpoint, and the relative
  error bound of a 3-bit mantissa.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_from_bits(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def binade(lo_exp_field, n_binades=1):
    """All fp32 patterns with biased exponent in [lo, lo + n), both signs excluded (>= 0)."""
    start = np.uint32(lo_exp_field) << np.uint32(23)
    return np.arange(int(start), int(start) + (n_binades << 23), dtype=np.uint32)


# ------------------------------------------------------------------------------------------
# bf16
# ------------------------------------------------------------------------------------------

def torch_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("lo,n", [(0, 2), (127, 1), (200, 1), (253, 2)])
def test_bf16_exhaustive_binades(lo, n):
    """Subnormals, [1, 2), a large binade and the overflow-to-infinity boundary, both signs."""
    bits = binade(lo, n)
    for sign in (np.uint32(0), np.uint32(0x80000000)):
        v = f32_from_bits(bits | sign)
        assert np.array_equal(oracle.bf16_rne(v), torch_bf16(v))


def test_bf16_random_patterns_and_specials():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 32, size=20_000_000, dtype=np.uint64).astype(np.uint32)
    v = f32_from_bits(bits)
    got, want = oracle.bf16_rne(v), torch_bf16(v)
    nan = np.isnan(v)
    assert np.array_equal(got[~nan], want[~nan])
    # every NaN gives the one quiet NaN 0x7FC0 (torch's CPU cast writes its own NaN pattern)
    assert nan.any() and (got[nan] == 0x7FC0).all()


def test_bf16_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: goes to 1 (even); 1 + 3*2^-8 goes up.
    v = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)
    assert oracle.bf16_rne(v).tolist() == [0x3F80, 0x3F82, 0xBF80]


# ------------------------------------------------------------------------------------------
# OCP E4M3
# ------------------------------------------------------------------------------------------

def load_golden_codes():
    rows = []
    with open(os.path.join(GOLDEN, "ofp8_e4m3_codes.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                code, val = line.split()
                rows.append((int(code, 16), float(val)))
    return rows


def test_e4m3_decode_matches_spec_values():
    for code, val in load_golden_codes():
        got = oracle.e4m3_value(code & 0x7F) * (-1 if code & 0x80 else 1)
        if np.isnan(val):
            assert code & 0x7F == 0x7F
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def positive_table():
    """Decoded values of the finite non-negative codes 0x00..0x7E, increasing."""
    vals = np.array([oracle.e4m3_value(c) for c in range(0x7F)], dtype=np.float64)
    assert (np.diff(vals) > 0).all()
    return vals


def nearest_even_search(v):
    """Independent encoder: nearest decoded value by searchsorted, ties to the even code,
    magnitudes >= 448 saturate; sign copied."""
    vals = positive_table()
    a = np.abs(v.astype(np.float64))
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, 0x7E)   # first value >= a
    lo = np.clip(hi - 1, 0, 0x7E)
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(vals[hi] == a, hi, pick)
    pick = np.where(a >= 448.0, 0x7E, pick)
    sign = np.where(np.signbit(v), 0x80, 0)
    return (pick | sign).astype(np.uint8)


def torch_e4m3(v):
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_e4m3_every_code_round_trips():
    vals = positive_table()
    for c in range(0x7F):
        for sign in (0, 0x80):
            v = np.array([vals[c] * (-1 if sign else 1)], dtype=np.float32)
            if c == 0 and sign:
                v = np.array([-0.0], dtype=np.float32)
            assert int(oracle.e4m3_rne_sat(v)[0]) == c | sign


def test_e4m3_midpoints_go_to_even():
    vals = positive_table()
    mids = (vals[:-1] + vals[1:]) / 2               # exact in fp32 (4 significant bits)
    v = mids.astype(np.float32)
    assert (v.astype(np.float64) == mids).all()
    got = oracle.e4m3_rne_sat(v)
    lower = np.arange(0x7E)
    want = np.where(lower % 2 == 0, lower, lower + 1)
    assert got.tolist() == want.tolist()
    # one fp32 ulp either side of each midpoint leaves the tie
    below = np.nextafter(v, np.float32(0))
    above = np.nextafter(v, np.float32(np.inf))
    assert oracle.e4m3_rne_sat(below[1:]).tolist() == lower[1:].tolist()
    assert oracle.e4m3_rne_sat(above).tolist() == (lower + 1).tolist()


@pytest.mark.parametrize("lo,n", [(116, 6), (127, 1), (135, 1)])
def test_e4m3_exhaustive_binades_vs_torch_and_search(lo, n):
    """[2^-11, 2^-5): zero threshold, subnormals, first normal binade; [1, 2); [256, 512):
    the saturation boundary (torch agrees with saturation up to 464; beyond, 448 is pinned by
    the search and the definition)."""
    bits = binade(lo, n)
    v = f32_from_bits(bits)
    got = oracle.e4m3_rne_sat(v)
    small = v <= np.float32(464.0)
    assert np.array_equal(got[small], torch_e4m3(v[small]))
    assert (got[~small] == 0x7E).all()
    step = 7
    assert np.array_equal(got[::step], nearest_even_search(v[::step]))
    neg = oracle.e4m3_rne_sat(-v[::step])
    assert np.array_equal(neg, got[::step] | 0x80)


def test_e4m3_below_half_min_subnormal_is_zero():
    # |v| <= 2^-10 (half the smallest subnormal) rounds to zero; 2^-10 itself is a tie -> 0.
    v = np.array([2.0 ** -10, 2.0 ** -11, 1e-30, -(2.0 ** -10)], dtype=np.float32)
    assert oracle.e4m3_rne_sat(v).tolist() == [0x00, 0x00, 0x00, 0x80]
    v = np.nextafter(np.float32(2.0 ** -10), np.float32(1))
    assert oracle.e4m3_rne_sat(np.array([v]))[0] == 0x01


def test_e4m3_random_patterns():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = f32_from_bits(bits)
    got = oracle.e4m3_rne_sat(v)
    nan = np.isnan(v)
    assert (got[nan] & 0x7F == 0x7F).all()
    fin = ~nan
    assert np.array_equal(got[fin], nearest_even_search(v[fin]))
    small = fin & (np.abs(v) <= 464.0)
    assert np.array_equal(got[small], torch_e4m3(v[small]))


def test_e4m3_saturates_and_keeps_sign():
    v = np.array([448.0, 449.0, 463.99, 464.0, 500.0, 1e38, np.inf, -np.inf, -500.0],
                 dtype=np.float32)
    assert oracle.e4m3_rne_sat(v).tolist() == [0x7E] * 7 + [0xFE, 0xFE]


def test_e4m3_relative_error_bound():
    """A 3-bit mantissa: |v - q| <= 2^-4 |v| in the normal range [2^-6, 448], and
    |v - q| <= 2^-10 below it (half a subnormal step)."""
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(1_000_000) * 30).astype(np.float32)
    v = np.clip(v, -448, 448)
    q = oracle.e4m3_rne_sat(v)
    vals = positive_table()
    dq = vals[q & 0x7F] * np.where(q & 0x80, -1.0, 1.0)
    err = np.abs(v.astype(np.float64) - dq)
    normal = np.abs(v) >= 2.0 ** -6
    assert (err[normal] <= 2.0 ** -4 * np.abs(v[normal])).all()
    assert (err[~normal] <= 2.0 ** -10).all()
