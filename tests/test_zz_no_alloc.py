"""GPU parity of hr_allreduce_group_noalloc_f16, the group all-reduce that
allocates nothing, against hr_allreduce_group_f16, the channel call it
stands in for.

Two calls in a row on the same stream, the second smaller than the first
(so the second runs over the array's contents as the first left them), for
groups of 2, 4 and 8 ranks: every rank's output equals, bit for bit (NaN by
class), the channel group call's output on the same inputs and the oracle's
left fold; the status word reads HR_OK after each call.
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


@pytest.mark.parametrize("W", [2, 4, 8])
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
