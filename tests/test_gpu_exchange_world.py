"""GPU parity of hr_allreduce_f16 for groups of W = 3..8 ranks (every size).

All W ranks run on one GPU as concurrently resident launches on W streams
that each own a hardware queue (loopback).  Every rank's output must equal,
bit for bit (NaN by class), the oracle's left fold of the W contributions in
rank order, and all ranks' outputs must be identical.
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle
from message_fp16_all_amd import hr, inputs
from _gpu import assert_same_bits, needs_gpu, specials_mix, to_dev, to_host

pytestmark = [pytest.mark.gpu, needs_gpu]

TIMEOUT_US = 2_000_000


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_call(ch, xs, outs, streams, order=None, delay=0.0):
    torch.cuda.synchronize()
    for r in (order or range(len(xs))):
        ch.allreduce(r, xs[r], outs[r], streams[r])
        if delay:
            time.sleep(delay)
    for s in streams:
        s.synchronize()
    assert ch.status() == hr.HR_OK, hr.hr_status_str(ch.status())


def check_all(outs, xbits, what):
    ref = oracle.fold(xbits)
    got = [to_host(o) for o in outs]
    for r, g in enumerate(got):
        assert_same_bits(g, ref, f"{what} rank {r}")
    for r in range(1, len(got)):
        assert np.array_equal(got[0], got[r]), f"{what}: rank {r} differs from rank 0"


ALGOS = {"one": hr.HR_ALGO_ONE_SHOT, "two": hr.HR_ALGO_TWO_SHOT, "ll": hr.HR_ALGO_LL}


@pytest.fixture(params=[(3, "one"), (4, "one"), (5, "one"), (6, "one"), (7, "one"), (8, "one"),
                        (2, "two"), (3, "two"), (4, "two"), (5, "two"), (6, "two"), (7, "two"),
                        (8, "two"),
                        (3, "ll"), (4, "ll"), (5, "ll"), (6, "ll"), (7, "ll"), (8, "ll")],
                ids=lambda p: f"W{p[0]}-{p[1]}")
def group(request):
    W, algo = request.param
    streams = hr.LoopbackStreams(0, n=W)
    ch = hr.Channel(world_size=W, timeout_us=TIMEOUT_US, algorithm=ALGOS[algo])
    yield W, ch, streams
    torch.cuda.synchronize()
    ch.destroy()
    streams.destroy()


@pytest.mark.parametrize("tokens", [1, 8, 32])
def test_workload6(group, tokens):
    W, ch, streams = group
    say(f"exchange W={W}: tokens={tokens}")
    xb = inputs.workload6(W, tokens)
    xs = [to_dev(b) for b in xb]
    outs = [torch.empty_like(x) for x in xs]
    run_call(ch, xs, outs, streams)
    check_all(outs, xb, f"W={W} tokens={tokens}")


def test_specials_and_ragged_sizes_across_calls(group):
    W, ch, streams = group
    for call, n in enumerate([1, 7, 9, 4097, 65_541, 131_072, 8]):
        xb = [specials_mix(n, seed=100 * call + r) for r in range(W)]
        xs = [to_dev(b) for b in xb]
        outs = [torch.empty_like(x) for x in xs]
        run_call(ch, xs, outs, streams)
        check_all(outs, xb, f"W={W} call {call} n={n}")


def test_arrival_in_reverse_order_with_delays(group):
    W, ch, streams = group
    xb = inputs.workload6(W, 8, call=1)
    xs = [to_dev(b) for b in xb]
    outs = [torch.empty_like(x) for x in xs]
    run_call(ch, xs, outs, streams, order=list(reversed(range(W))), delay=0.005)
    check_all(outs, xb, f"W={W} reversed")


def test_one_rank_on_the_other_access_path(group):
    W, ch, streams = group
    n = 50_003
    xb = [specials_mix(n, seed=7 + r) for r in range(W)]
    xs, outs = [], []
    for r, b in enumerate(xb):
        off = 1 if r == W - 1 else 0
        buf = to_dev(np.concatenate([np.zeros(off, np.uint16), b]))
        ob = torch.zeros(n + off, dtype=torch.float16, device="cuda:0")
        xs.append(buf[off:])
        outs.append(ob[off:])
    run_call(ch, xs, outs, streams)
    check_all(outs, xb, f"W={W} mixed paths")


@pytest.mark.parametrize("algo", ["one", "two", "ll"])
def test_graph_replays_with_fresh_inputs(algo):
    W, calls, n = 4, 5, 16_384
    streams = hr.LoopbackStreams(0, n=W)
    ch = hr.Channel(world_size=W, timeout_us=TIMEOUT_US, algorithm=ALGOS[algo])
    try:
        xin = [torch.empty((calls, n), dtype=torch.float16, device="cuda:0") for _ in range(W)]
        outs = [torch.empty_like(x) for x in xin]
        run_call(ch, [x[0] for x in xin], [o[0] for o in outs], streams)
        graphs = []
        for r in range(W):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=streams[r]):
                for k in range(calls):
                    ch.allreduce(r, xin[r][k], outs[r][k], streams[r])
            graphs.append(g)
        for replay in range(3):
            xb = [np.stack([inputs.gaussian(n, 0.5, 60 + replay, r, k) for k in range(calls)])
                  for r in range(W)]
            for r in range(W):
                xin[r].copy_(to_dev(xb[r].reshape(-1)).view(calls, n))
            torch.cuda.synchronize()
            for r in range(W):
                with torch.cuda.stream(streams[r]):
                    graphs[r].replay()
            for s in streams:
                s.synchronize()
            assert ch.status() == hr.HR_OK
            check_all([o.reshape(-1) for o in outs], [b.reshape(-1) for b in xb],
                      f"W={W} graph replay {replay}")
    finally:
        torch.cuda.synchronize()
        ch.destroy()
        streams.destroy()


@pytest.mark.parametrize("algo", ["one", "two", "ll"])
def test_missing_rank_times_out_every_waiting_rank(algo):
    W = 4
    streams = hr.LoopbackStreams(0, n=W)
    ch = hr.Channel(world_size=W, timeout_us=20_000, algorithm=ALGOS[algo])
    try:
        xb = inputs.workload6(W, 1)
        xs = [to_dev(b) for b in xb]
        outs = [torch.full_like(x, 3.0) for x in xs]
        torch.cuda.synchronize()
        assert ch.timeout_info() is None
        for r in range(W - 1):                     # rank W-1 never arrives
            ch.allreduce(r, xs[r], outs[r], streams[r])
        for s in streams:
            s.synchronize()
        assert ch.status() == hr.HR_ERR_TIMEOUT
        for r in range(W - 1):
            assert torch.all(outs[r] == 3.0)
        # the timeout record names the missing rank and the call (the first)
        rank, missing, call = ch.timeout_info()
        assert rank in range(W - 1) and missing == [W - 1] and call == 1, (rank, missing, call)
        with pytest.raises(hr.HrError) as ei:
            ch.allreduce(W - 1, xs[W - 1], outs[W - 1], streams[W - 1])
        assert ei.value.status == hr.HR_ERR_TIMEOUT
        assert f"for ranks [{W - 1}]" in str(ei.value)   # the error names the missing rank
    finally:
        torch.cuda.synchronize()
        ch.destroy()
        streams.destroy()


def test_automatic_choice_mixes_algorithms_across_calls():
    """Under HR_ALGO_AUTO a W = 4 channel takes LL up to 4096 values, the
    one-shot below 16384 and the two-shot from there; alternating sizes
    alternate the algorithm while the slot parity keeps advancing."""
    W = 4
    streams = hr.LoopbackStreams(0, n=W)
    ch = hr.Channel(world_size=W, timeout_us=TIMEOUT_US)
    try:
        for call, n in enumerate([4096, 131_072, 16_383, 16_384, 9, 65_539, 10_241, 32_768]):
            xb = [specials_mix(n, seed=500 + 10 * call + r) for r in range(W)]
            xs = [to_dev(b) for b in xb]
            outs = [torch.empty_like(x) for x in xs]
            run_call(ch, xs, outs, streams)
            check_all(outs, xb, f"auto call {call} n={n}")
    finally:
        torch.cuda.synchronize()
        ch.destroy()
        streams.destroy()


def test_two_shot_needs_a_workgroup_per_shard():
    with pytest.raises(hr.HrError) as ei:
        hr.Channel(world_size=8, num_blocks=4, algorithm=hr.HR_ALGO_TWO_SHOT)
    assert ei.value.status == hr.HR_ERR_INVALID_ARG
