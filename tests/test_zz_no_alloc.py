"""GPU parity of hr_allreduce_group_noalloc_f16, the group all-reduce that
allocates nothing, against hr_allreduce_group_f16, the channel call it
stands in for.

Two calls in a row on the same stream, the second smaller than the first
(so the second runs over the array's contents as the first left them), for
every group size from 2 to 8 ranks (each lays the array out differently): every rank's output equals, bit for bit (NaN by
class), the channel group call's output on the same inputs and the oracle's
left fold; the status word reads HR_OK after each call.

Also: calls of random sizes queued on one stream without a host wait (calls
on one stream do not race), and a captured graph of such calls replayed with
fresh inputs and eager calls between the replays.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from message_fp16_all_amd import hr
from _gpu import assert_same_bits, needs_gpu, specials_mix, to_dev, to_host

pytestmark = [pytest.mark.gpu, needs_gpu]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("W", [2, 3, 4, 5, 6, 7, 8])
def test_two_calls_in_a_row_match_the_channel_group_call(W):
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    ch = hr.Channel(world_size=W, timeout_us=2_000_000)
    try:
        for call, n in enumerate([hr.HR_NOALLOC_MAX_NUMEL, 4099]):
            xb = [specials_mix(n, 3100 + 17 * call + r) for r in range(W)]
            xs = [to_dev(b) for b in xb]
            got = [torch.full_like(x, 3.0) for x in xs]
            ref = [torch.full_like(x, 5.0) for x in xs]
            status.fill_(-1)
            torch.cuda.synchronize()
            say(f"no-alloc group call: W={W} call {call} n={n} (algorithm {ch.algorithm_for(n)})")
            hr.allreduce_group_noalloc(xs, got, status=status)
            torch.cuda.synchronize()
            assert int(status.item()) == hr.HR_OK, f"status {int(status.item())}"
            ch.allreduce_group(xs, ref)
            torch.cuda.synchronize()
            assert ch.status() == hr.HR_OK
            fold = oracle.fold(xb)
            for r in range(W):
                g, e = to_host(got[r]), to_host(ref[r])
                assert_same_bits(g, e, f"W={W} call {call} n={n} rank {r} against the channel call")
                assert_same_bits(g, fold, f"W={W} call {call} n={n} rank {r} against the oracle")
    finally:
        torch.cuda.synchronize()
        ch.destroy()


def test_without_a_status_word_and_in_place():
    W, n = 4, 10_240
    xb = [specials_mix(n, 3300 + r) for r in range(W)]
    xs = [to_dev(b) for b in xb]
    torch.cuda.synchronize()
    hr.allreduce_group_noalloc(xs, xs)            # outs[r] is ins[r]
    torch.cuda.synchronize()
    fold = oracle.fold(xb)
    for r in range(W):
        assert_same_bits(to_host(xs[r]), fold, f"in place rank {r}")


def test_oversize_is_refused():
    x = [torch.zeros(hr.HR_NOALLOC_MAX_NUMEL + 1, dtype=torch.float16, device="cuda:0") for _ in range(2)]
    with pytest.raises(hr.HrError) as ei:
        hr.allreduce_group_noalloc(x, [torch.empty_like(t) for t in x])
    assert ei.value.status == hr.HR_ERR_TOO_LARGE


@pytest.mark.parametrize("W", [2, 4, 8])
def test_calls_queued_on_one_stream_without_a_host_wait(W):
    """Calls on one stream do not race: 120 calls of random sizes (crossing
    the automatic choice's switch points, so the algorithm changes from call
    to call) queued before the host waits once, each with its own buffers."""
    rng = np.random.default_rng(3500 + W)
    sizes = [int(max(1, round(2 ** rng.uniform(0, 17)))) for _ in range(120)]
    xb = [[specials_mix(n, int(rng.integers(0, 1 << 30))) for _ in range(W)] for n in sizes]
    xs = [[to_dev(b) for b in row] for row in xb]
    outs = [[torch.full_like(x, 3.0) for x in row] for row in xs]
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    torch.cuda.synchronize()
    say(f"no-alloc: {len(sizes)} queued calls, W={W}")
    for c in range(len(sizes)):
        hr.allreduce_group_noalloc(xs[c], outs[c], status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == hr.HR_OK
    for c, n in enumerate(sizes):
        fold = oracle.fold(xb[c])
        for r in range(W):
            assert_same_bits(to_host(outs[c][r]), fold, f"W={W} call {c} n={n} rank {r}")


def test_graph_of_calls_replayed_with_fresh_inputs():
    """The callers this entry point is for capture it: a graph of 20 calls
    (sizes crossing the switch points, four ranks) replayed three times, with
    fresh inputs, eager calls and host waits between the replays; every replay
    is compared with the oracle."""
    W = 4
    sizes = [4096, 131_072, 9, 16_384, 2048, 65_541, 1, 30_000, 4097, 12_288] * 2
    xs = [[torch.empty(n, dtype=torch.float16, device="cuda:0") for _ in range(W)] for n in sizes]
    outs = [[torch.empty_like(x) for x in row] for row in xs]
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    s = torch.cuda.Stream()
    for c in range(len(sizes)):                      # warm up on the capture stream
        hr.allreduce_group_noalloc(xs[c], outs[c], status=status, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in range(len(sizes)):
            hr.allreduce_group_noalloc(xs[c], outs[c], status=status, stream=s)
    for rep in range(3):
        xb = [[specials_mix(n, 3700 + 100 * rep + 10 * c + r) for r in range(W)] for c, n in enumerate(sizes)]
        for c in range(len(sizes)):
            for r in range(W):
                xs[c][r].copy_(to_dev(xb[c][r]))
                outs[c][r].fill_(3.0)
        status.fill_(-1)
        torch.cuda.synchronize()
        say(f"no-alloc graph replay {rep}")
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == hr.HR_OK
        for c, n in enumerate(sizes):
            fold = oracle.fold(xb[c])
            for r in range(W):
                assert_same_bits(to_host(outs[c][r]), fold, f"replay {rep} call {c} n={n} rank {r}")
        # eager work between replays, on the same state
        e = [to_dev(specials_mix(777, 3900 + rep + r)) for r in range(W)]
        eo = [torch.empty_like(t) for t in e]
        hr.allreduce_group_noalloc(e, eo, stream=s)
        torch.cuda.synchronize()
        ref = oracle.fold([to_host(t) for t in e])
        for r in range(W):
            assert_same_bits(to_host(eo[r]), ref, f"eager after replay {rep} rank {r}")
    del g
    torch.cuda.synchronize()
