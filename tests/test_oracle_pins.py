"""Pins of the CPU oracle to things other than itself.

The oracle (``oracle/hr_oracle.c``) defines the combine: binary64 add, exact
for binary16 operands, then one round-to-nearest-even to binary16, folded left
in rank order.  These tests check it against

* library routines that implement the same IEEE operations independently:
  numpy's binary16<->binary64 conversions, numpy's float16 ``add`` (computed
  in binary32 and rounded once more, which is still correctly rounded for
  binary16 because 24 >= 2*11 + 2), and CPython's ``struct`` 'e' packing;
* exhaustive enumeration (every bit pattern; every ordered pair on a subset
  of exponent fields; every rounding midpoint);
* closed forms (subnormal sums are exact integers of 2^-24; integer folds
  below 2048 are exact);
* hand-derived worked values in ``tests/golden``.

A dropped term, a wrong sign, a wrong exponent bias, ties rounded away from
zero, flushed subnormals, a missing overflow, or a right fold instead of a
left fold each fail at least one test here (``test_oracle_mutants.py``
plants such mistakes and checks that they are caught).
"""
import os
import struct

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

ALL = np.arange(65536, dtype=np.uint16)
IS_NAN = ((ALL & 0x7C00) == 0x7C00) & ((ALL & 0x03FF) != 0)
NON_NAN = ALL[~IS_NAN]


def f64_bits(x):
    return np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)


def np_f16_bits(x64):
    """numpy's binary64 -> binary16 conversion, as bit patterns."""
    with np.errstate(over="ignore", invalid="ignore"):
        return np.asarray(x64, dtype=np.float64).astype(np.float16).view(np.uint16)


def is_nan16(h):
    h = np.asarray(h, dtype=np.uint16)
    return ((h & 0x7C00) == 0x7C00) & ((h & 0x03FF) != 0)


# ---------------------------------------------------------------- decode ---

def test_decode_every_pattern_matches_numpy():
    got = oracle.decode(ALL)
    ref = ALL.view(np.float16).astype(np.float64)
    nan_got = np.isnan(got)
    assert np.array_equal(nan_got, IS_NAN)
    # bitwise on binary64 so that -0 and +0 are told apart
    assert np.array_equal(f64_bits(got[~nan_got]), f64_bits(ref[~nan_got]))


def test_decode_closed_forms():
    assert oracle.decode(np.array([0x0001], np.uint16))[0] == 2.0 ** -24
    assert oracle.decode(np.array([0x03FF], np.uint16))[0] == 1023 * 2.0 ** -24
    assert oracle.decode(np.array([0x0400], np.uint16))[0] == 2.0 ** -14
    assert oracle.decode(np.array([0x3C00], np.uint16))[0] == 1.0
    assert oracle.decode(np.array([0x7BFF], np.uint16))[0] == 65504.0
    assert oracle.decode(np.array([0xC000], np.uint16))[0] == -2.0
    assert np.signbit(oracle.decode(np.array([0x8000], np.uint16))[0])
    assert oracle.decode(np.array([0xFC00], np.uint16))[0] == -np.inf


# ---------------------------------------------------------------- round ----

def test_round_trip_every_non_nan_pattern():
    back = oracle.round_f16(oracle.decode(NON_NAN))
    assert NON_NAN.size == 63490
    assert np.array_equal(back, NON_NAN)


def test_round_nan_gives_a_nan():
    back = oracle.round_f16(oracle.decode(ALL[IS_NAN]))
    assert is_nan16(back).all()


def _midpoints():
    """Every midpoint between adjacent finite non-negative binary16 values."""
    pos = np.arange(0, 0x7BFF + 1, dtype=np.uint16)          # 0 .. 65504
    v = pos.view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2.0                            # exact in binary64
    return pos[:-1], pos[1:], mids


def test_every_midpoint_rounds_to_the_even_neighbour():
    lo, hi, mids = _midpoints()
    assert mids.size == 31743
    for sign in (0.0, -0.0):
        vals = -mids if np.signbit(sign) else mids
        got = oracle.round_f16(vals)
        mag = got & 0x7FFF
        # one of the two neighbours, and the one with an even fraction
        assert np.all((mag == lo) | (mag == hi))
        assert np.all((mag & 1) == 0)
        assert np.all((got >> 15) == (1 if np.signbit(sign) else 0))
        assert np.array_equal(got, np_f16_bits(vals))
    up = np.count_nonzero(oracle.round_f16(mids) == hi)
    assert (up, mids.size - up) == (15871, 15872)


def test_overflow_threshold():
    # 65520 is the midpoint of 65504 and the (unrepresentable) 65536: ties to even -> inf
    vals = np.array([65504.0, 65519.999, 65520.0, 65536.0, 1e300,
                     -65520.0, -65519.0, np.inf, -np.inf])
    got = oracle.round_f16(vals)
    assert [int(x) for x in got] == [0x7BFF, 0x7BFF, 0x7C00, 0x7C00, 0x7C00,
                                     0xFC00, 0xFBFF, 0x7C00, 0xFC00]


def test_round_random_doubles_matches_numpy():
    rng = np.random.default_rng(20260)
    parts = [
        rng.standard_normal(200_000) * 1e3,
        rng.uniform(-65600, 65600, 200_000),
        rng.uniform(-2.0 ** -13, 2.0 ** -13, 200_000),         # subnormal range
        np.ldexp(rng.uniform(0.5, 1.0, 200_000), rng.integers(-30, 18, 200_000)),
    ]
    vals = np.concatenate(parts)
    vals[::7] *= -1
    assert np.array_equal(oracle.round_f16(vals), np_f16_bits(vals))


def test_round_matches_cpython_struct_pack():
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        np.ldexp(rng.uniform(0.5, 1.0, 20_000), rng.integers(-26, 17, 20_000)),
        _midpoints()[2][::3],
    ])
    vals[::2] *= -1
    got = oracle.round_f16(vals)
    for v, g in zip(vals.tolist(), got.tolist()):
        try:
            ref = struct.unpack("<H", struct.pack("<e", v))[0]
        except OverflowError:
            ref = 0xFC00 if v < 0 else 0x7C00                 # CPython raises on overflow
        assert g == ref, (v, hex(g), hex(ref))


def test_round_tiny_values_underflow_to_signed_zero():
    vals = np.array([2.0 ** -26, 2.0 ** -25, 2.0 ** -25 * 1.0000001, -2.0 ** -25, -1e-300])
    got = oracle.round_f16(vals)
    # 2^-25 is the midpoint of 0 and 2^-24: ties to even (zero)
    assert [int(x) for x in got] == [0x0000, 0x0000, 0x0001, 0x8000, 0x8000]


# ---------------------------------------------------------------- add -----

EXP_SUBSET = (0, 1, 2, 14, 15, 16, 29, 30, 31)


def _subset_values():
    vals = []
    for s in (0, 1):
        for e in EXP_SUBSET:
            base = (s << 15) | (e << 10)
            vals.append(np.arange(base, base + 1024, dtype=np.uint32))
    return np.concatenate(vals).astype(np.uint16)


def test_exhaustive_pairs_on_exponent_subset():
    """All ordered pairs with exponent fields in EXP_SUBSET, both signs:
    18,432 values -> 339,738,624 pairs, against numpy float16 add and against
    numpy binary64 add rounded by numpy; NaN by class."""
    vals = _subset_values()
    assert vals.size == 18432
    vf = vals.view(np.float16)
    vd = vf.astype(np.float64)
    chunk = 384
    checked = 0
    for i in range(0, vals.size, chunk):
        a = np.repeat(vals[i:i + chunk], vals.size)
        b = np.tile(vals, min(chunk, vals.size - i))
        got = oracle.add(a, b)
        with np.errstate(over="ignore", invalid="ignore"):
            ref1 = (a.view(np.float16) + b.view(np.float16)).view(np.uint16)
            ref2 = np_f16_bits(np.repeat(vd[i:i + chunk], vals.size) +
                               np.tile(vd, min(chunk, vals.size - i)))
        for ref in (ref1, ref2):
            ok = oracle.same_bits(got, ref)
            if not ok.all():
                j = int(np.flatnonzero(~ok)[0])
                pytest.fail(f"{a[j]:#06x} + {b[j]:#06x}: oracle {got[j]:#06x}, ref {ref[j]:#06x}")
        checked += a.size
    assert checked == 339_738_624


def test_commutative_on_exponent_subset():
    vals = _subset_values()[::5]
    a = np.repeat(vals, vals.size)
    b = np.tile(vals, vals.size)
    assert oracle.same_bits(oracle.add(a, b), oracle.add(b, a)).all()


def test_identities_over_every_pattern():
    x = NON_NAN
    neg0 = np.full_like(x, 0x8000)
    pos0 = np.zeros_like(x)
    # x + (-0) == x for every non-NaN x
    assert np.array_equal(oracle.add(x, neg0), x)
    # x + (+0) == x except that (-0) + (+0) == +0
    r = oracle.add(x, pos0)
    expect = np.where(x == 0x8000, np.uint16(0), x)
    assert np.array_equal(r, expect)
    # x + (-x) == +0 for finite x
    fin = x[(x & 0x7C00) != 0x7C00]
    assert np.array_equal(oracle.add(fin, fin ^ np.uint16(0x8000)), np.zeros_like(fin))
    # inf + finite == inf; inf + (-inf) is NaN; NaN + anything is NaN
    for inf in (0x7C00, 0xFC00):
        assert np.array_equal(oracle.add(np.full_like(fin, inf), fin), np.full_like(fin, inf))
    assert is_nan16(oracle.add(np.array([0x7C00], np.uint16), np.array([0xFC00], np.uint16))).all()
    nans = ALL[IS_NAN]
    assert is_nan16(oracle.add(nans, np.full_like(nans, 0x3C00))).all()
    assert is_nan16(oracle.add(np.full_like(nans, 0x3C00), nans)).all()


def test_subnormal_sums_are_exact_integers():
    """Every sum of two values with exponent field 0 is an exact multiple of
    2^-24 below 2^-13.  Its pattern is sign | |m_a +- m_b|: for a count of
    2^-24 units up to 2047 the binary16 encoding of k*2^-24 is k itself."""
    sub = np.concatenate([np.arange(0, 1024), np.arange(0x8000, 0x8400)]).astype(np.uint16)
    a = np.repeat(sub, sub.size)
    b = np.tile(sub, sub.size)
    ma = (a & 0x3FF).astype(np.int64) * np.where(a >> 15, -1, 1)
    mb = (b & 0x3FF).astype(np.int64) * np.where(b >> 15, -1, 1)
    s = ma + mb
    both_neg_zero = (a == 0x8000) & (b == 0x8000)
    expect = np.where(s < 0, 0x8000 | (-s), s)
    expect = np.where(both_neg_zero, 0x8000, expect).astype(np.uint16)
    assert np.array_equal(oracle.add(a, b), expect)


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_worked_values_from_golden():
    rows = _read_golden("worked_values.txt")
    assert len(rows) >= 20
    for row in rows:
        a, b, r = (int(t, 16) for t in row[:3])
        got = oracle.add(np.array([a], np.uint16), np.array([b], np.uint16))
        assert oracle.same_bits(got, np.array([r], np.uint16))[0], (row, hex(got[0]))
        # the two-rank combine is commutative (same bits on both ranks)
        got_ba = oracle.add(np.array([b], np.uint16), np.array([a], np.uint16))
        assert oracle.same_bits(got_ba, np.array([r], np.uint16))[0]


# ---------------------------------------------------------------- fold ----

def test_fold_order_from_golden():
    for row in _read_golden("fold_order.txt"):
        xs = [np.array([int(t, 16)], np.uint16) for t in row[0].split(",")]
        r = int(row[1], 16)
        got = oracle.fold(xs)
        assert oracle.same_bits(got, np.array([r], np.uint16))[0], (row, hex(got[0]))


def test_fold_equals_numpy_float16_left_fold():
    rng = np.random.default_rng(99)
    for G in (1, 2, 3, 5, 8, 16):
        n = 50_000
        xs = []
        for g in range(G):
            x = (rng.standard_normal(n).astype(np.float32) * np.float32(10.0 ** rng.integers(-4, 4)))
            x = x.astype(np.float16).view(np.uint16)
            idx = rng.choice(n, 500, replace=False)
            x[idx] = rng.choice(np.array([0x0000, 0x8000, 0x7BFF, 0xFBFF, 0x0001, 0x83FF,
                                          0x7C00, 0xFC00], np.uint16), 500)
            xs.append(x)
        acc = xs[0].view(np.float16).copy()
        with np.errstate(over="ignore", invalid="ignore"):
            for g in range(1, G):
                acc = acc + xs[g].view(np.float16)
        got = oracle.fold(xs)
        assert oracle.same_bits(got, acc.view(np.uint16)).all(), G


def test_integer_folds_below_2048_are_exact():
    rng = np.random.default_rng(5)
    for G in (2, 4, 8, 16):
        n = 20_000
        ints = rng.integers(-2048 // G, 2048 // G + 1, size=(G, n))
        xs = [ints[g].astype(np.float16).view(np.uint16) for g in range(G)]
        got = oracle.fold(xs).view(np.float16).astype(np.float64)
        assert np.array_equal(got, ints.sum(axis=0).astype(np.float64))


def test_fold_threads_identical_and_reports_threads():
    rng = np.random.default_rng(3)
    xs = [rng.standard_normal(100_003).astype(np.float16).view(np.uint16) for _ in range(8)]
    one = oracle.fold(xs)
    many, used = oracle.fold(xs, threads=4)
    assert used >= 1
    assert np.array_equal(one, many)


def test_fold_g2_is_the_pairwise_add():
    rng = np.random.default_rng(11)
    a = rng.integers(0, 65536, 300_000, dtype=np.uint32).astype(np.uint16)
    b = rng.integers(0, 65536, 300_000, dtype=np.uint32).astype(np.uint16)
    assert oracle.same_bits(oracle.fold([a, b]), oracle.add(a, b)).all()
