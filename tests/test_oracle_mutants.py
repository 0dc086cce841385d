"""Planted mistakes in the oracle must be caught by its pins.

Each case below copies ``oracle/hr_oracle.c``, plants one plausible mistake
(a wrong exponent bias, a lost sign, flushed subnormals, ties rounded the
wrong way, a saturating overflow, a dropped or reordered fold term), builds
the copy with the same host compiler flags into a temporary directory, and
runs a quick battery of the same kinds of pins that ``test_oracle_pins.py``
applies to the real oracle.  The battery must reject every mutant and accept
the unmodified source.  Nothing here touches a GPU.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "hr_oracle.c")
GOLDEN = os.path.join(HERE, "golden")

FOLD_LOOP = """        uint16_t acc = x[0][i];
        for (int g = 1; g < G; ++g)
            acc = hro_round(hro_decode(acc) + hro_decode(x[g][i]));
        out[i] = acc;
    }
}"""

MUTANTS = {
    "exponent_bias": ("ldexp((double)(1024 + frac), efield - 25)",
                      "ldexp((double)(1024 + frac), efield - 24)"),
    "decode_drops_sign": ("return sign ? -mag : mag;", "return mag;"),
    "flush_subnormal_inputs": ("mag = ldexp((double)frac, -24);", "mag = 0.0;"),
    "ties_away_from_zero": ("return (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;",
                            "return lo + 1.0;"),
    "ties_toward_zero": ("return (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;", "return lo;"),
    "truncate_instead_of_round": ("if (rest > 0.5)\n        return lo + 1.0;",
                                  "if (rest > 0.5)\n        return lo;"),
    "saturating_overflow": ("return sign | 0x7C00;                         /* a >= 65536 */",
                            "return sign | 0x7BFF;"),
    "negative_zero_lost": ("uint16_t sign = signbit(v) ? 0x8000 : 0x0000;",
                           "uint16_t sign = (v < 0) ? 0x8000 : 0x0000;"),
    "subnormal_threshold": ("if (a < ldexp(1.0, -14)) {", "if (a < ldexp(1.0, -15)) {"),
    "fold_drops_last_term": ("for (int g = 1; g < G; ++g)\n            acc = hro_round(hro_decode(acc) + hro_decode(x[g][i]));\n        out[i] = acc;\n    }\n}",
                             "for (int g = 1; g < G - 1; ++g)\n            acc = hro_round(hro_decode(acc) + hro_decode(x[g][i]));\n        out[i] = acc;\n    }\n}"),
    "right_fold": (FOLD_LOOP,
                   """        uint16_t acc = x[G - 1][i];
        for (int g = G - 2; g >= 0; --g)
            acc = hro_round(hro_decode(x[g][i]) + hro_decode(acc));
        out[i] = acc;
    }
}"""),
    "single_rounding_of_total": (FOLD_LOOP,
                                 """        double s = hro_decode(x[0][i]);
        for (int g = 1; g < G; ++g)
            s += hro_decode(x[g][i]);
        out[i] = hro_round(s);
    }
}"""),
}


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def battery(o: oracle.Oracle) -> list:
    """Quick pins; returns the names of the ones that fail."""
    failed = []
    allp = np.arange(65536, dtype=np.uint16)
    is_nan = ((allp & 0x7C00) == 0x7C00) & ((allp & 0x3FF) != 0)
    # decode against numpy's conversion, bitwise in binary64
    got = o.decode(allp)
    ref = allp.view(np.float16).astype(np.float64)
    if not (np.array_equal(np.isnan(got), is_nan) and
            np.array_equal(got[~is_nan].view(np.uint64), ref[~is_nan].view(np.uint64))):
        failed.append("decode_vs_numpy")
    # round trip of every non-NaN pattern
    if not np.array_equal(o.round_f16(ref[~is_nan]), allp[~is_nan]):
        failed.append("round_trip")
    # midpoints (both signs) against numpy's rounding
    pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2.0
    mids = np.concatenate([mids, -mids, [65520.0, -65520.0, 1e6]])
    with np.errstate(over="ignore"):
        if not np.array_equal(o.round_f16(mids), mids.astype(np.float16).view(np.uint16)):
            failed.append("midpoints_vs_numpy")
    # worked values
    for row in _golden("worked_values.txt"):
        a, b, r = (np.array([int(t, 16)], np.uint16) for t in row[:3])
        if not oracle.same_bits(o.add(a, b), r)[0]:
            failed.append("worked_values")
            break
    # fold order examples
    for row in _golden("fold_order.txt"):
        xs = [np.array([int(t, 16)], np.uint16) for t in row[0].split(",")]
        if not oracle.same_bits(o.fold(xs), np.array([int(row[1], 16)], np.uint16))[0]:
            failed.append("fold_order")
            break
    # fold against numpy's float16 left fold on random data
    rng = np.random.default_rng(1)
    xs = [rng.standard_normal(4096).astype(np.float16).view(np.uint16) for _ in range(8)]
    acc = xs[0].view(np.float16).copy()
    for x in xs[1:]:
        acc = acc + x.view(np.float16)
    if not oracle.same_bits(o.fold(xs), acc.view(np.uint16)).all():
        failed.append("fold_vs_numpy")
    return failed


MUTANTS_BF16 = {
    "bf16_exponent_bias": ("ldexp((double)(128 + frac), efield - 134)",
                           "ldexp((double)(128 + frac), efield - 133)"),
    "bf16_flush_subnormals": ("mag = ldexp((double)frac, -133);", "mag = 0.0;"),
    "bf16_fraction_width": ("double q = round_half_even(ldexp(f, 8));",
                            "double q = round_half_even(ldexp(f, 7));"),
    "bf16_no_overflow": ("    if (efield >= 255)\n        return sign | 0x7F80;\n    double q = round_half_even(ldexp(f, 8));",
                         "    double q = round_half_even(ldexp(f, 8));"),
    "bf16_right_fold": ("""        uint16_t acc = x[0][i];
        for (int g = 1; g < G; ++g)
            acc = hro_round_bf16(hro_decode_bf16(acc) + hro_decode_bf16(x[g][i]));""",
                        """        uint16_t acc = x[G - 1][i];
        for (int g = G - 2; g >= 0; --g)
            acc = hro_round_bf16(hro_decode_bf16(x[g][i]) + hro_decode_bf16(acc));"""),
}


def battery_bf16(o: oracle.Oracle) -> list:
    import torch
    failed = []
    allp = np.arange(65536, dtype=np.uint16)
    is_nan = ((allp & 0x7F80) == 0x7F80) & ((allp & 0x7F) != 0)
    ref = torch.from_numpy(allp.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = o.decode_bf16(allp)
    if not (np.array_equal(np.isnan(got), is_nan) and
            np.array_equal(got[~is_nan].view(np.uint64), ref[~is_nan].view(np.uint64))):
        failed.append("decode_vs_torch")
    if not np.array_equal(o.round_bf16(ref[~is_nan]), allp[~is_nan]):
        failed.append("round_trip")
    big = np.array([3.3895313892515355e38 + 2.0 ** 119, 2.0 ** 128])   # max + half ulp ties up
    if not (o.round_bf16(big) == 0x7F80).all():
        failed.append("overflow")
    with open(os.path.join(GOLDEN, "worked_values_bf16.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, b, r = (np.array([int(t, 16)], np.uint16) for t in line.split()[:3])
                if not oracle.same_bits_bf16(o.add_bf16(a, b), r)[0]:
                    failed.append("worked_values")
                    break
    xs = [np.array([0x4380], np.uint16), np.array([0x3F80], np.uint16), np.array([0x3F80], np.uint16)]
    if int(o.fold_bf16(xs)[0]) != 0x4380:
        failed.append("fold_order")
    return failed


def _build(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    lib = tmp_path / f"lib{name}.so"
    src.write_text(text)
    cmd = [c for c in oracle.BUILD_CMD]
    cmd[cmd.index(oracle._SRC)] = str(src)
    cmd[cmd.index(oracle._LIB)] = str(lib)
    subprocess.run(cmd, check=True)
    return oracle.Oracle(str(lib))


def test_unmodified_oracle_passes_battery(tmp_path):
    with open(SRC) as f:
        text = f.read()
    assert battery(_build(tmp_path, "orig", text)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    mutated = text.replace(old, new)
    if name == "fold_drops_last_term" or name in ("right_fold", "single_rounding_of_total"):
        # only the single-threaded fold is mutated; hro_fold_threads keeps its own loop
        mutated = text.replace(old, new, 1)
    failed = battery(_build(tmp_path, name, mutated))
    assert failed, f"mutant {name} passed every pin"


def test_unmodified_oracle_passes_bf16_battery(tmp_path):
    with open(SRC) as f:
        text = f.read()
    assert battery_bf16(_build(tmp_path, "orig_bf16", text)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS_BF16))
def test_bf16_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS_BF16[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    failed = battery_bf16(_build(tmp_path, name, text.replace(old, new)))
    assert failed, f"mutant {name} passed every pin"
