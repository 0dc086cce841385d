"""Pins of the oracle's comparators, ``oracle.same_bits`` (binary16) and
``oracle.same_bits_bf16`` (bfloat16).

Every parity verdict goes through them: the 1Cat-vLLM pull request "[Kernel]
Two-rank FP16 all-reduce through pinned host memory for GPUs without P2P"
("Purpose") asks for the same bits on every rank, and IEEE 754 leaves the
payload of a NaN produced by an add open.  So the comparator must say
"equal" exactly when both patterns are NaNs (any sign, any payload) or when
the patterns are identical; in particular +0 differs from -0, +inf from -inf,
and an infinity from every NaN.

The NaN class here comes from library routines, not from a retyped mask:
numpy's ``isnan`` on binary16 values and torch's ``isnan`` on bfloat16
values.  The comparator is run on every one of the 65,536 patterns against a
set of partners holding both zeros, both infinities, NaNs of every sign,
quiet bit and payload extreme, the subnormal and normal extremes, and 4096
random patterns.  Planted mistakes in copies of the comparators' source (an
infinity counted as a NaN, the sign ignored, the other format's masks, NaNs
compared bit for bit, a NaN matched to anything) must each fail the pin.
Nothing here touches a GPU.
"""
import inspect

import numpy as np
import pytest
import torch

import oracle

ALL = np.arange(65536, dtype=np.uint16)


def nan_f16(p: np.ndarray) -> np.ndarray:
    return np.isnan(p.view(np.float16))


def nan_bf16(p: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(p).view(np.int16)).view(torch.bfloat16)
    return torch.isnan(t).numpy()


PARTNERS_F16 = [0x0000, 0x8000, 0x7C00, 0xFC00,            # zeros, infinities
                0x7C01, 0x7DFF, 0x7E00, 0x7FFF,             # NaNs: signalling / quiet, payload extremes
                0xFC01, 0xFDFF, 0xFE00, 0xFFFF,
                0x0001, 0x8001, 0x03FF, 0x83FF,             # subnormal extremes
                0x0400, 0x8400, 0x7BFF, 0xFBFF,             # normal extremes
                0x3C00, 0xBC00]
PARTNERS_BF16 = [0x0000, 0x8000, 0x7F80, 0xFF80,
                 0x7F81, 0x7FBF, 0x7FC0, 0x7FFF,
                 0xFF81, 0xFFBF, 0xFFC0, 0xFFFF,
                 0x0001, 0x8001, 0x007F, 0x807F,
                 0x0080, 0x8080, 0x7F7F, 0xFF7F,
                 0x3F80, 0xBF80]


def partners(fixed):
    rng = np.random.default_rng(20261203)
    return np.concatenate([np.array(fixed, np.uint16),
                           rng.integers(0, 1 << 16, 4096, dtype=np.uint32).astype(np.uint16)])


def comparator_failures(same, nan_of, fixed) -> list:
    """Pairs (a, b) on which `same` disagrees with the definition: equal iff
    both NaN or identical patterns.  Returns up to 5 of them."""
    bad = []
    a_nan = nan_of(ALL)
    for b in partners(fixed):
        bv = np.full(ALL.shape, b, np.uint16)
        want = (a_nan & nan_of(bv)) | (ALL == bv)
        got = np.asarray(same(ALL, bv))
        if got.dtype != np.bool_ or got.shape != ALL.shape:
            return [("shape/dtype", got.dtype, got.shape)]
        diff = np.flatnonzero(got != want)
        for i in diff[:5 - len(bad)]:
            bad.append((int(ALL[i]), int(b), bool(got[i]), bool(want[i])))
        if len(bad) >= 5:
            break
    return bad


def test_nan_classes_from_the_libraries():
    # the library routines agree with the formats' counts: a NaN has an
    # all-ones exponent field and one of 1023 (binary16) or 127 (bfloat16)
    # nonzero fractions, under either sign
    assert int(nan_f16(ALL).sum()) == 2 * 1023
    assert int(nan_bf16(ALL).sum()) == 2 * 127


def test_same_bits_binary16():
    assert comparator_failures(oracle.same_bits, nan_f16, PARTNERS_F16) == []


def test_same_bits_bfloat16():
    assert comparator_failures(oracle.same_bits_bf16, nan_bf16, PARTNERS_BF16) == []


def test_special_pairs_binary16():
    s = lambda a, b: bool(oracle.same_bits(np.array([a], np.uint16), np.array([b], np.uint16))[0])
    assert not s(0x0000, 0x8000)      # +0 and -0 differ
    assert not s(0x7C00, 0xFC00)      # +inf and -inf differ
    assert not s(0x7C00, 0x7E00)      # inf is not a NaN
    assert not s(0x7BFF, 0x7C00)      # overflow is visible
    assert s(0x7E00, 0xFC01)          # any NaN matches any NaN
    assert s(0x3C00, 0x3C00)


def test_special_pairs_bfloat16():
    s = lambda a, b: bool(oracle.same_bits_bf16(np.array([a], np.uint16), np.array([b], np.uint16))[0])
    assert not s(0x0000, 0x8000)
    assert not s(0x7F80, 0xFF80)
    assert not s(0x7F80, 0x7FC0)
    assert s(0x7FC0, 0xFF81)
    # a binary16-only reading of the masks would take these bfloat16 values
    # (exponent field 0x7C..0x7F of the binary16 view) for NaNs
    assert not s(0x7C01, 0x7E00)


def _mutated(fn, old, new):
    src = inspect.getsource(fn)
    assert src.count(old) >= 1, f"mutation site {old!r} not found in {fn.__name__}"
    ns = {"np": np, "_u16": oracle._u16}
    exec(src.replace(old, new), ns)
    return ns[fn.__name__]


MUTANTS_F16 = {
    "inf_counts_as_nan": ("((a & 0x03FF) != 0)", "((a & 0x03FF) >= 0)"),
    "sign_ignored": ("a == b)", "(a & 0x7FFF) == (b & 0x7FFF))"),
    "nan_compared_bitwise": ("a_nan & b_nan, a == b", "a == b, a == b"),
    "nan_matches_anything": ("a_nan & b_nan, a == b", "True, a == b"),
    "bf16_masks": ("((a & 0x7C00) == 0x7C00) & ((a & 0x03FF) != 0)",
                   "((a & 0x7F80) == 0x7F80) & ((a & 0x007F) != 0)"),
}
MUTANTS_BF16 = {
    "inf_counts_as_nan": ("((a & 0x007F) != 0)", "((a & 0x007F) >= 0)"),
    "sign_ignored": ("a == b)", "(a & 0x7FFF) == (b & 0x7FFF))"),
    "nan_compared_bitwise": ("a_nan & b_nan, a == b", "a == b, a == b"),
    "nan_matches_anything": ("a_nan & b_nan, a == b", "True, a == b"),
    "f16_masks": ("((a & 0x7F80) == 0x7F80) & ((a & 0x007F) != 0)",
                  "((a & 0x7C00) == 0x7C00) & ((a & 0x03FF) != 0)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS_F16))
def test_binary16_comparator_mutant_is_caught(name):
    old, new = MUTANTS_F16[name]
    fn = _mutated(oracle.same_bits, old, new)
    assert comparator_failures(fn, nan_f16, PARTNERS_F16), f"mutant {name} passed the pin"


@pytest.mark.parametrize("name", sorted(MUTANTS_BF16))
def test_bfloat16_comparator_mutant_is_caught(name):
    old, new = MUTANTS_BF16[name]
    fn = _mutated(oracle.same_bits_bf16, old, new)
    assert comparator_failures(fn, nan_bf16, PARTNERS_BF16), f"mutant {name} passed the pin"
