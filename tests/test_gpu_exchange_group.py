"""GPU parity of hr_allreduce_group_f16 / _bf16: every rank of a loopback
channel in one launch.

Each rank's output must equal, bit for bit (NaN by class), the oracle's left
fold of the W contributions in rank order, for every algorithm, for ragged
sizes and both access paths, mixed with per-rank calls on the same channel,
and replayed from a graph with fresh inputs.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from message_fp16_all_amd import hr, inputs
from _gpu import (assert_same_bits, needs_gpu, specials_mix, specials_mix_bf16, to_dev, to_dev_bf16,
                  to_host)

pytestmark = [pytest.mark.gpu, needs_gpu]

TIMEOUT_US = 2_000_000
ALGOS = {"auto": hr.HR_ALGO_AUTO, "one": hr.HR_ALGO_ONE_SHOT, "two": hr.HR_ALGO_TWO_SHOT,
         "ll": hr.HR_ALGO_LL}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def group_call(ch, xs, outs, stream=None):
    torch.cuda.synchronize()
    ch.allreduce_group(xs, outs, stream)
    torch.cuda.synchronize()
    assert ch.status() == hr.HR_OK, hr.hr_status_str(ch.status())


def check_all(outs, xbits, what, bf16=False):
    ref = oracle.fold_bf16(xbits) if bf16 else oracle.fold(xbits)
    for r, o in enumerate(outs):
        assert_same_bits(to_host(o) if not bf16 else o.view(torch.int16).cpu().numpy().view(np.uint16),
                         ref, f"{what} rank {r}", bf16=bf16)


@pytest.fixture(params=[(2, "auto"), (2, "one"), (2, "two"), (2, "ll"),
                        (3, "auto"), (3, "one"), (3, "two"), (3, "ll"),
                        (4, "auto"), (4, "two"), (4, "ll"),
                        (5, "auto"), (5, "one"), (5, "two"), (5, "ll"),
                        (6, "auto"), (6, "one"), (6, "two"), (6, "ll"),
                        (7, "auto"), (7, "one"), (7, "two"), (7, "ll"),
                        (8, "auto"), (8, "one"), (8, "two"), (8, "ll")],
                ids=lambda p: f"W{p[0]}-{p[1]}")
def channel(request):
    W, algo = request.param
    ch = hr.Channel(world_size=W, timeout_us=TIMEOUT_US, algorithm=ALGOS[algo])
    yield W, ch
    torch.cuda.synchronize()
    ch.destroy()


@pytest.mark.parametrize("n", [1, 9, 4096, 10_240, 32_768, 70_001, 131_072])
def test_group_call_matches_the_oracle(channel, n):
    W, ch = channel
    say(f"group W={W} algo={ch.algorithm_for(n)} n={n}")
    xb = [specials_mix(n, 7000 + 31 * r + n % 97) for r in range(W)]
    xs = [to_dev(b) for b in xb]
    outs = [torch.empty_like(x) for x in xs]
    group_call(ch, xs, outs)
    check_all(outs, xb, f"W={W} n={n}")


def test_workload6_tokens_and_in_place(channel):
    W, ch = channel
    for tokens in (1, 8, 32):
        xb = inputs.workload6(W, tokens) if W > 2 else list(inputs.workload2(tokens))
        xs = [to_dev(b) for b in xb]
        say(f"group W={W} tokens={tokens} in place")
        group_call(ch, xs, xs)                           # outs[r] is ins[r]
        check_all(xs, xb, f"W={W} tokens={tokens} in place")


def test_unaligned_buffers_take_the_value_path(channel):
    W, ch = channel
    n = 4097
    xb = [specials_mix(n, 7100 + r) for r in range(W)]
    base = [torch.empty(n + 8, dtype=torch.float16, device="cuda") for _ in range(W)]
    xs = [b[1:1 + n] for b in base]                      # 2-byte aligned only
    for x, b in zip(xs, xb):
        x.copy_(to_dev(b))
    outs = [torch.empty(n + 8, dtype=torch.float16, device="cuda")[3:3 + n] for _ in range(W)]
    say(f"group W={W} unaligned n={n}")
    group_call(ch, xs, outs)
    check_all(outs, xb, f"W={W} unaligned")


def test_group_and_per_rank_calls_share_a_channel():
    """The group launch advances each rank's call counters as W separate
    calls do, so the two kinds of call may alternate on one channel."""
    W = 2
    streams = hr.LoopbackStreams(0, n=W)
    ch = hr.Channel(world_size=W, timeout_us=TIMEOUT_US)
    try:
        for k, n in enumerate([4096, 131_072, 9, 32_768, 70_001, 4096, 131_072]):
            xb = [specials_mix(n, 7200 + 10 * k + r) for r in range(W)]
            xs = [to_dev(b) for b in xb]
            outs = [torch.empty_like(x) for x in xs]
            say(f"mixed call {k}: {'group' if k % 2 == 0 else 'per-rank'} n={n}")
            if k % 2 == 0:
                group_call(ch, xs, outs)
            else:
                torch.cuda.synchronize()
                for r in range(W):
                    ch.allreduce(r, xs[r], outs[r], streams[r])
                for s in streams:
                    s.synchronize()
                assert ch.status() == hr.HR_OK
            check_all(outs, xb, f"mixed call {k}")
    finally:
        torch.cuda.synchronize()
        ch.destroy()
        streams.destroy()


@pytest.mark.parametrize("W,algo", [(2, "auto"), (4, "two"), (8, "auto"), (8, "ll")])
def test_graph_of_group_calls_replayed_with_fresh_inputs(W, algo):
    n, calls = 10_240, 25
    ch = hr.Channel(world_size=W, timeout_us=TIMEOUT_US, algorithm=ALGOS[algo])
    try:
        xin = [torch.empty(calls, n, dtype=torch.float16, device="cuda") for _ in range(W)]
        outs = [torch.empty(calls, n, dtype=torch.float16, device="cuda") for _ in range(W)]
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for k in range(calls):
                ch.allreduce_group([x[k] for x in xin], [o[k] for o in outs], s)
        for rep in range(3):
            xb = [[specials_mix(n, 7300 + 1000 * rep + 10 * k + r) for k in range(calls)] for r in range(W)]
            for r in range(W):
                xin[r].copy_(to_dev(np.stack(xb[r])).view(calls, n))
            torch.cuda.synchronize()
            say(f"graph W={W} {algo} replay {rep}")
            g.replay()
            torch.cuda.synchronize()
            assert ch.status() == hr.HR_OK, hr.hr_status_str(ch.status())
            for k in range(calls):
                check_all([o[k] for o in outs], [xb[r][k] for r in range(W)], f"replay {rep} call {k}")
        del g
    finally:
        torch.cuda.synchronize()
        ch.destroy()


@pytest.mark.parametrize("W", [2, 4])
def test_bf16_group_call(W):
    ch = hr.Channel(world_size=W, timeout_us=TIMEOUT_US)
    try:
        for n in (9, 4096, 131_072):
            xb = [specials_mix_bf16(n, 7400 + 17 * r + n % 13) for r in range(W)]
            xs = [to_dev_bf16(b) for b in xb]
            outs = [torch.empty_like(x) for x in xs]
            say(f"bf16 group W={W} n={n}")
            group_call(ch, xs, outs)
            check_all(outs, xb, f"bf16 W={W} n={n}", bf16=True)
    finally:
        torch.cuda.synchronize()
        ch.destroy()


def test_group_arguments_are_checked_before_launch():
    W, n = 4, 4096
    ch = hr.Channel(world_size=W, timeout_us=TIMEOUT_US)
    try:
        xs = [torch.zeros(n, dtype=torch.float16, device="cuda") for _ in range(W)]
        outs = [torch.empty_like(x) for x in xs]
        ip = [x.data_ptr() for x in xs]
        op = [o.data_ptr() for o in outs]
        s = torch.cuda.current_stream().cuda_stream
        assert hr.hr_allreduce_group_f16(ch.handle, ip[:1] + [None] + ip[2:], op, n, s) == hr.HR_ERR_INVALID_ARG
        assert hr.hr_allreduce_group_f16(ch.handle, ip, op[:3] + [None], n, s) == hr.HR_ERR_INVALID_ARG
        assert hr.hr_allreduce_group_f16(ch.handle, ip, [op[0], op[0], op[2], op[3]], n, s) == \
            hr.HR_ERR_INVALID_ARG                        # two ranks write one buffer
        assert hr.hr_allreduce_group_f16(ch.handle, ip, [ip[1]] + op[1:], n, s) == \
            hr.HR_ERR_INVALID_ARG                        # rank 0 writes rank 1's input
        assert hr.hr_allreduce_group_f16(ch.handle, ip, [ip[0] + 2] + op[1:], n, s) == \
            hr.HR_ERR_INVALID_ARG                        # partial overlap with its own input
        assert hr.hr_allreduce_group_f16(ch.handle, [ip[0] + 1] + ip[1:], op, n, s) == hr.HR_ERR_ALIGNMENT
        assert hr.hr_allreduce_group_f16(ch.handle, ip, op, hr.HR_DEFAULT_MAX_NUMEL + 1, s) == \
            hr.HR_ERR_TOO_LARGE
        assert hr.hr_allreduce_group_f16(ch.handle, ip, op, 0, s) == hr.HR_OK
        torch.cuda.synchronize()
        assert ch.status() == hr.HR_OK
        # the channel still works after the refused calls
        xb = [specials_mix(n, 7500 + r) for r in range(W)]
        for x, b in zip(xs, xb):
            x.copy_(to_dev(b))
        group_call(ch, xs, outs)
        check_all(outs, xb, "after refused calls")
    finally:
        torch.cuda.synchronize()
        ch.destroy()
