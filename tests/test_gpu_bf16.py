"""GPU parity of hr_reduce_bf16 and hr_allreduce_bf16 against the oracle's
bfloat16 combine (left fold in rank order, one bfloat16 rounding per add),
bit for bit with NaN compared by class, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from message_fp16_all_amd import hr, inputs
from _gpu import assert_same_bits, needs_gpu, specials_mix_bf16, to_dev_bf16, to_host

pytestmark = [pytest.mark.gpu, needs_gpu]


def fold_gpu(xs_bits, offset=0):
    ts = []
    for x in xs_bits:
        buf = to_dev_bf16(np.concatenate([np.zeros(offset, np.uint16), x]))
        ts.append(buf[offset:])
    ob = torch.zeros(xs_bits[0].size + offset, dtype=torch.bfloat16, device="cuda:0")
    out = ob[offset:]
    hr.reduce(ts, out)
    torch.cuda.synchronize()
    return to_host(out)


def test_edge_table_bf16():
    xs = inputs.edge_pairs_bf16()
    assert_same_bits(fold_gpu(xs), oracle.fold_bf16(xs), "bf16 edge table", bf16=True)


@pytest.mark.parametrize("G", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("n", [1, 7, 9, 2049, 100_003])
def test_ragged_sizes_over_the_whole_range(G, n):
    xs = [specials_mix_bf16(n, seed=31 * G + r + n) for r in range(G)]
    assert_same_bits(fold_gpu(xs), oracle.fold_bf16(xs), f"bf16 G={G} n={n}", bf16=True)


def test_unaligned_scalar_path():
    xs = [specials_mix_bf16(5001, seed=3 + r) for r in range(4)]
    assert_same_bits(fold_gpu(xs, offset=3), oracle.fold_bf16(xs), "bf16 unaligned", bf16=True)


def test_eight_ranks_gaussian_large():
    n = 4_194_304 + 5
    xs = [inputs.gaussian_bf16(n, 1.0, 7, r) for r in range(8)]
    assert_same_bits(fold_gpu(xs), oracle.fold_bf16(xs), "bf16 G=8 4M", bf16=True)


def test_torch_bf16_add_agrees():
    xs = [inputs.gaussian_bf16(65_536, 1.0, 8, r) for r in range(2)]
    t = to_dev_bf16(xs[0]) + to_dev_bf16(xs[1])
    assert_same_bits(fold_gpu(xs), to_host(t), "bf16 vs torch", bf16=True)


@pytest.mark.parametrize("algorithm", [hr.HR_ALGO_AUTO, hr.HR_ALGO_LL, hr.HR_ALGO_TWO_SHOT],
                         ids=["auto", "ll", "two-shot"])
@pytest.mark.parametrize("W", [2, 4])
def test_exchange_bf16(W, algorithm):
    streams = hr.LoopbackStreams(0, n=W)
    ch = hr.Channel(world_size=W, timeout_us=2_000_000, algorithm=algorithm)
    try:
        for call, n in enumerate([131_072, 4096, 65_541, 9, 32_768, 12_345]):
            xb = [specials_mix_bf16(n, seed=1000 * call + 10 * W + r) for r in range(W)]
            xs = [to_dev_bf16(b) for b in xb]
            outs = [torch.empty_like(x) for x in xs]
            torch.cuda.synchronize()
            for r in range(W):
                ch.allreduce(r, xs[r], outs[r], streams[r])
            for s in streams:
                s.synchronize()
            assert ch.status() == hr.HR_OK
            ref = oracle.fold_bf16(xb)
            got = [to_host(o) for o in outs]
            for r in range(W):
                assert_same_bits(got[r], ref, f"bf16 exchange W={W} n={n} rank {r}", bf16=True)
                assert np.array_equal(got[r], got[0])
    finally:
        torch.cuda.synchronize()
        ch.destroy()
        streams.destroy()


def test_one_channel_carries_both_types_across_calls():
    streams = hr.LoopbackStreams(0)
    ch = hr.Channel(timeout_us=2_000_000)
    try:
        for call in range(4):
            n = 32_768
            if call % 2:
                xb = [inputs.gaussian_bf16(n, 0.5, 9, r, call) for r in range(2)]
                xs = [to_dev_bf16(b) for b in xb]
                ref = oracle.fold_bf16(xb)
            else:
                xb = [inputs.gaussian(n, 0.5, 9, r, call) for r in range(2)]
                xs = [torch.from_numpy(b.view(np.int16)).view(torch.float16).cuda() for b in xb]
                ref = oracle.fold(xb)
            outs = [torch.empty_like(x) for x in xs]
            torch.cuda.synchronize()
            for r in range(2):
                ch.allreduce(r, xs[r], outs[r], streams[r])
            for s in streams:
                s.synchronize()
            assert ch.status() == hr.HR_OK
            for r in range(2):
                assert_same_bits(to_host(outs[r]), ref, f"call {call} rank {r}", bf16=bool(call % 2))
    finally:
        torch.cuda.synchronize()
        ch.destroy()
        streams.destroy()


def test_workspace_layout_bf16():
    G, n = 8, 1_000_003
    xs = [inputs.gaussian_bf16(n, 1.0, 10, r) for r in range(G)]
    buf, views = hr.workspace(G, n, dtype=torch.bfloat16)
    for v, x in zip(views, xs):
        v.copy_(to_dev_bf16(x))
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")
    hr.reduce(views, out)
    torch.cuda.synchronize()
    assert_same_bits(to_host(out), oracle.fold_bf16(xs), "bf16 workspace", bf16=True)
