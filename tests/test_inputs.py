"""The seeded input generators: determinism, shapes and planted specials."""
import numpy as np

from message_fp16_all_amd import inputs


def test_streams_are_deterministic_and_distinct():
    a = inputs.gaussian(1000, 1.0, 3, 0)
    b = inputs.gaussian(1000, 1.0, 3, 0)
    c = inputs.gaussian(1000, 1.0, 3, 1)
    d = inputs.gaussian(1000, 1.0, 3, 0, call=1)
    assert a.dtype == np.uint16
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    assert not np.array_equal(a, d)


def test_gaussian_statistics():
    for sigma in (1.0, 0.5, 0.1):
        x = inputs.gaussian(200_000, sigma, 2, 0).view(np.float16).astype(np.float64)
        assert abs(x.mean()) < 0.01 * sigma * 5
        assert abs(x.std() / sigma - 1.0) < 0.01


def test_workload1_specials():
    xs, idxs = inputs.workload1()
    assert len(xs) == 2 and all(x.size == 4096 for x in xs)
    for x, idx in zip(xs, idxs):
        assert idx.size == 41 and np.unique(idx).size == 41
        v = x[idx]
        mag = v & 0x7FFF
        sub = (mag >= 1) & (mag <= 0x3FF)
        big = mag == 0x7BFF
        zero = mag == 0
        assert np.all(sub | big | zero)
        # each class present at this seed
        assert sub.any() and big.any() and zero.any()
        # no inf or NaN anywhere in the inputs
        assert not np.any((x & 0x7C00) == 0x7C00)
    again, _ = inputs.workload1()
    assert all(np.array_equal(a, b) for a, b in zip(xs, again))


def test_workload_shapes_and_bytes():
    for t in inputs.TOKENS_EXCHANGE:
        xs = inputs.workload2(t)
        assert len(xs) == 2 and xs[0].size == 4096 * t
    assert inputs.workload2(32)[0].nbytes == 256 * 1024
    xs = inputs.workload3()
    assert len(xs) == 8 and xs[0].size == 393_216
    assert inputs.WORKLOADS[4]["n"] * 2 == 32 * 1024 * 1024
    small = inputs.workload4(n=4096)
    assert len(small) == 8 and small[0].size == 4096
    c5 = inputs.workload5(calls=3)
    assert c5.shape == (2, 3, 10_240)
    assert not np.array_equal(c5[0, 0], c5[0, 1])
    assert np.array_equal(c5[1, 2], inputs.gaussian(10_240, 1.0, 5, 1, 2))


def test_edge_pairs_cover_every_ordered_pair():
    a, b = inputs.edge_pairs()
    assert a.size == b.size == 289
    pairs = set(zip(a.tolist(), b.tolist()))
    assert len(pairs) == 289
