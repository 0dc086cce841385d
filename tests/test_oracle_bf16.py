"""Pins of the oracle's bfloat16 combine to things other than itself.

numpy has no bfloat16, so the library routines here are torch's CPU
bfloat16 conversions and adds (a bfloat16 add is computed in binary32 and
rounded once more to bfloat16, which is still correctly rounded because
24 >= 2 * 8 + 2), plus exhaustive enumeration, closed forms and hand-derived
worked values in ``tests/golden/worked_values_bf16.txt``.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ALL = np.arange(65536, dtype=np.uint16)
IS_NAN = ((ALL & 0x7F80) == 0x7F80) & ((ALL & 0x007F) != 0)


def t_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def bits_of(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def torch_round_f32(x32):
    """torch's binary32 -> bfloat16 conversion (round to nearest even)."""
    return bits_of(torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16))


def test_decode_every_pattern_matches_torch():
    got = oracle.decode_bf16(ALL)
    ref = t_bf16(ALL).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), IS_NAN)
    assert np.array_equal(got[~IS_NAN].view(np.uint64), ref[~IS_NAN].view(np.uint64))


def test_round_trip_every_non_nan_pattern():
    x = ALL[~IS_NAN]
    assert np.array_equal(oracle.round_bf16(oracle.decode_bf16(x)), x)
    assert (((oracle.round_bf16(oracle.decode_bf16(ALL[IS_NAN]))) & 0x7FFF) > 0x7F80).all()


def test_every_midpoint_rounds_to_the_even_neighbour():
    pos = np.arange(0, 0x7F80, dtype=np.uint16)              # 0 .. max finite
    v = oracle.decode_bf16(pos)
    mids = (v[:-1] + v[1:]) / 2.0                            # exact in binary64 and binary32
    lo, hi = pos[:-1], pos[1:]
    for neg in (False, True):
        vals = -mids if neg else mids
        got = oracle.round_bf16(vals)
        mag = got & 0x7FFF
        assert np.all((mag == lo) | (mag == hi))
        assert np.all((mag & 1) == 0)
        assert np.array_equal(got, torch_round_f32(vals.astype(np.float32)))


def test_round_binary32_values_matches_torch():
    rng = np.random.default_rng(17)
    bits = rng.integers(0, 2 ** 32, 500_000, dtype=np.uint64).astype(np.uint32)
    x32 = bits.view(np.float32)
    x32 = x32[~np.isnan(x32)]
    assert np.array_equal(oracle.round_bf16(x32.astype(np.float64)), torch_round_f32(x32))


def test_overflow_threshold():
    mx = float(oracle.decode_bf16(np.array([0x7F7F], np.uint16))[0])
    half_ulp = 2.0 ** 119
    vals = np.array([mx, mx + half_ulp * 0.999, mx + half_ulp, -(mx + half_ulp), 2.0 ** 128])
    assert [int(v) for v in oracle.round_bf16(vals)] == [0x7F7F, 0x7F7F, 0x7F80, 0xFF80, 0x7F80]


EXP_SUBSET = (0, 1, 2, 126, 127, 128, 253, 254, 255)


def subset_values():
    vals = []
    for s in (0, 1):
        for e in EXP_SUBSET:
            base = (s << 15) | (e << 7)
            vals.append(np.arange(base, base + 128, dtype=np.uint32))
    return np.concatenate(vals).astype(np.uint16)


def test_exhaustive_pairs_on_exponent_subset_match_torch():
    vals = subset_values()
    assert vals.size == 2304
    a = np.repeat(vals, vals.size)
    b = np.tile(vals, vals.size)
    got = oracle.add_bf16(a, b)
    ref = bits_of(t_bf16(a) + t_bf16(b))
    ok = oracle.same_bits_bf16(got, ref)
    if not ok.all():
        j = int(np.flatnonzero(~ok)[0])
        pytest.fail(f"{a[j]:#06x} + {b[j]:#06x}: oracle {got[j]:#06x}, torch {ref[j]:#06x}")
    assert oracle.same_bits_bf16(oracle.add_bf16(b, a), got).all()     # commutative


def test_random_pairs_match_torch():
    rng = np.random.default_rng(23)
    a = rng.integers(0, 65536, 2_000_000, dtype=np.uint32).astype(np.uint16)
    b = rng.integers(0, 65536, 2_000_000, dtype=np.uint32).astype(np.uint16)
    got = oracle.add_bf16(a, b)
    assert oracle.same_bits_bf16(got, bits_of(t_bf16(a) + t_bf16(b))).all()


def test_subnormal_sums_are_exact_integers():
    sub = np.concatenate([np.arange(0, 128), np.arange(0x8000, 0x8080)]).astype(np.uint16)
    a = np.repeat(sub, sub.size)
    b = np.tile(sub, sub.size)
    ma = (a & 0x7F).astype(np.int64) * np.where(a >> 15, -1, 1)
    mb = (b & 0x7F).astype(np.int64) * np.where(b >> 15, -1, 1)
    s = ma + mb
    expect = np.where(s < 0, 0x8000 | (-s), s)
    expect = np.where((a == 0x8000) & (b == 0x8000), 0x8000, expect).astype(np.uint16)
    assert np.array_equal(oracle.add_bf16(a, b), expect)


def test_worked_values_from_golden():
    n = 0
    with open(os.path.join(GOLDEN, "worked_values_bf16.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b, r = (np.array([int(t, 16)], np.uint16) for t in line.split()[:3])
            assert oracle.same_bits_bf16(oracle.add_bf16(a, b), r)[0], line
            assert oracle.same_bits_bf16(oracle.add_bf16(b, a), r)[0], line
            n += 1
    assert n >= 18


def test_fold_matches_torch_left_fold_and_order_matters():
    rng = np.random.default_rng(29)
    for G in (2, 3, 8, 16):
        xs = [torch_round_f32((rng.standard_normal(40_000) *
                               10.0 ** rng.integers(-30, 30)).astype(np.float32)) for _ in range(G)]
        acc = t_bf16(xs[0])
        for x in xs[1:]:
            acc = acc + t_bf16(x)
        assert oracle.same_bits_bf16(oracle.fold_bf16(xs), bits_of(acc)).all(), G
    # 256 + 1 + 1: left fold 256 (tie to even twice); right fold 256 + 2 = 258
    got = oracle.fold_bf16([np.array([0x4380], np.uint16), np.array([0x3F80], np.uint16),
                            np.array([0x3F80], np.uint16)])
    assert int(got[0]) == 0x4380
