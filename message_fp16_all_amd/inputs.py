"""Seeded synthetic inputs for the FP16 all-reduce combine.

This module only draws numbers: it holds none of the combine's arithmetic,
and both the GPU path's tests and the CPU oracle consume what it returns.
Every array is a numpy ``uint16`` array of binary16 bit patterns.

Stream per (workload, rank, call): numpy ``Generator(PCG64(SeedSequence(
1216, spawn_key=(workload, rank, call))))``.  A Gaussian contribution is
``standard_normal(n, float32) * float32(sigma)`` converted to binary16 by
numpy (round to nearest even).

The workloads stand in for the decode and prefill activations the pages
reduce (tokens x hidden, hidden 4096 / 5120 / 6144 / 8192); the pages ship
no data, so seeded Gaussians of those shapes are used:

* workload 1 -- two ranks, 4096 values each (one decode token, hidden 4096),
  sigma 1, with 1% of the values per rank (41 distinct positions) replaced
  by a special drawn uniformly from {subnormal with random sign and fraction
  1..1023, +-65504, +-0};
* workload 2 -- two-rank exchange, 4096 x tokens values per rank for tokens
  in {1, 4, 8, 16, 32}, sigma 0.5;
* workload 3 -- eight ranks, 393216 values each (64 rows x hidden 6144, the
  decode-sized workspace of the SGLang pull request's "Modifications"
  section), sigma 0.1;
* workload 4 -- eight ranks, 2048 tokens x hidden 8192 = 16777216 values
  each (32 MiB per rank, one prefill chunk), sigma 1;
* workload 5 -- two-rank exchange repeated over 1000 calls, 10240 values per
  rank per call (batch 2 x hidden 5120), fresh sigma-1 values per call;
* workload 6 -- exchange among W = 3..8 ranks (the SGLang page's world sizes
  4 and 8), 4096 x tokens values per rank, sigma 0.5, independent per rank.

``edge_pairs`` adds every ordered pair of 17 special values (signed zeros,
subnormal extremes, the smallest normal, one, 2048, the largest finite, the
infinities and a quiet NaN) so that every special meets every other.

bfloat16 contributions (``gaussian_bf16``, ``edge_pairs_bf16``) take the top
16 bits of the same binary32 draws: a bfloat16 sample of the same
distribution, obtained by truncation so that this module does no rounding.
"""
from __future__ import annotations

import numpy as np

SEED = 1216

HIDDEN_DECODE = 4096
TOKENS_EXCHANGE = (1, 4, 8, 16, 32)

WORKLOADS = {
    1: dict(G=2, n=4096, sigma=1.0),
    2: dict(G=2, sigma=0.5),
    3: dict(G=8, n=393_216, sigma=0.1),
    4: dict(G=8, n=16_777_216, sigma=1.0),
    5: dict(G=2, n=10_240, sigma=1.0, calls=1000),
    6: dict(sigma=0.5),
}

EDGE_VALUES = np.array([
    0x0000, 0x8000,          # +0, -0
    0x0001, 0x8001,          # smallest subnormals
    0x03FF, 0x83FF,          # largest subnormals
    0x0400, 0x8400,          # smallest normals
    0x3C00, 0xBC00,          # +-1
    0x6800, 0xE800,          # +-2048
    0x7BFF, 0xFBFF,          # +-65504
    0x7C00, 0xFC00,          # +-inf
    0x7E00,                  # quiet NaN
], dtype=np.uint16)


def rng(workload: int, rank: int, call: int = 0) -> np.random.Generator:
    """The generator for one (workload, rank, call) stream."""
    ss = np.random.SeedSequence(SEED, spawn_key=(int(workload), int(rank), int(call)))
    return np.random.Generator(np.random.PCG64(ss))


def gaussian(n: int, sigma: float, workload: int, rank: int, call: int = 0) -> np.ndarray:
    """n binary16 patterns of N(0, sigma^2) drawn in binary32."""
    g = rng(workload, rank, call)
    x = g.standard_normal(n, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x.astype(np.float16).view(np.uint16)


def _plant_specials(x: np.ndarray, g: np.random.Generator, frac: float = 0.01) -> np.ndarray:
    n = x.size
    k = int(round(frac * n))
    idx = g.choice(n, size=k, replace=False)
    kind = g.integers(0, 3, size=k)                 # 0 subnormal, 1 +-65504, 2 +-0
    sign = g.integers(0, 2, size=k).astype(np.uint16) << 15
    sub = g.integers(1, 1024, size=k).astype(np.uint16)
    val = np.where(kind == 0, sub, np.where(kind == 1, np.uint16(0x7BFF), np.uint16(0)))
    x[idx] = (val.astype(np.uint16) | sign).astype(np.uint16)
    return idx


def workload1(n: int | None = None):
    """Two contributions with planted specials; returns (xs, special_idx)."""
    w = WORKLOADS[1]
    n = w["n"] if n is None else n
    xs, idxs = [], []
    for r in range(w["G"]):
        g = rng(1, r, 0)
        x = g.standard_normal(n, dtype=np.float32).astype(np.float16).view(np.uint16).copy()
        idxs.append(_plant_specials(x, g))
        xs.append(x)
    return xs, idxs


def workload2(tokens: int, call: int = 0):
    """Two contributions of 4096 * tokens values for the exchange."""
    w = WORKLOADS[2]
    n = HIDDEN_DECODE * tokens
    return [gaussian(n, w["sigma"], 2, r, call) for r in range(w["G"])]


def workload3(n: int | None = None):
    w = WORKLOADS[3]
    n = w["n"] if n is None else n
    return [gaussian(n, w["sigma"], 3, r) for r in range(w["G"])]


def workload4(n: int | None = None):
    w = WORKLOADS[4]
    n = w["n"] if n is None else n
    return [gaussian(n, w["sigma"], 4, r) for r in range(w["G"])]


def workload5(calls: int | None = None, n: int | None = None) -> np.ndarray:
    """Per-rank, per-call contributions: array of shape (2, calls, n)."""
    w = WORKLOADS[5]
    calls = w["calls"] if calls is None else calls
    n = w["n"] if n is None else n
    out = np.empty((2, calls, n), dtype=np.uint16)
    for r in range(2):
        for c in range(calls):
            out[r, c] = gaussian(n, w["sigma"], 5, r, c)
    return out


def workload6(world: int, tokens: int, call: int = 0):
    """`world` contributions of 4096 * tokens values for a W-rank exchange."""
    n = HIDDEN_DECODE * tokens
    return [gaussian(n, WORKLOADS[6]["sigma"], 6, r, call) for r in range(world)]


EDGE_VALUES_BF16 = np.array([
    0x0000, 0x8000,          # +0, -0
    0x0001, 0x8001,          # smallest subnormals
    0x007F, 0x807F,          # largest subnormals
    0x0080, 0x8080,          # smallest normals
    0x3F80, 0xBF80,          # +-1
    0x4380, 0xC380,          # +-256
    0x7F7F, 0xFF7F,          # +-largest finite
    0x7F80, 0xFF80,          # +-inf
    0x7FC0,                  # quiet NaN
], dtype=np.uint16)


def gaussian_bf16(n: int, sigma: float, workload: int, rank: int, call: int = 0) -> np.ndarray:
    """n bfloat16 patterns: the top halves of N(0, sigma^2) binary32 draws."""
    g = rng(workload, rank, call)
    x = g.standard_normal(n, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def edge_pairs_bf16():
    """All 289 ordered pairs of EDGE_VALUES_BF16 as two contributions."""
    a = np.repeat(EDGE_VALUES_BF16, EDGE_VALUES_BF16.size)
    b = np.tile(EDGE_VALUES_BF16, EDGE_VALUES_BF16.size)
    return [a.copy(), b.copy()]


def edge_pairs():
    """All 289 ordered pairs of EDGE_VALUES as two contributions."""
    a = np.repeat(EDGE_VALUES, EDGE_VALUES.size)
    b = np.tile(EDGE_VALUES, EDGE_VALUES.size)
    return [a.copy(), b.copy()]


def contributions(G: int, n: int, sigma: float, workload: int, call: int = 0):
    """G independent Gaussian contributions on the stream of ``workload``."""
    return [gaussian(n, sigma, workload, r, call) for r in range(G)]
