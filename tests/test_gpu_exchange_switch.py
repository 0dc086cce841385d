"""GPU parity at the automatic algorithm's switch points, for every group
size W = 2..8, binary16 and bfloat16, per-rank loopback launches and the
group launch.

Under HR_ALGO_AUTO a channel of W ranks takes the low-latency one-shot up to
a size that falls with W, then the one-shot, and for W >= 3 the two-shot
from a second size that also falls with W (the table in hr.h).  The fold
order is fixed at every group size -- the SGLang pull request "[SM120] Add
optional FlashInfer PCIe-IPC all-reduce for switch-free hosts" ("Accuracy")
shows that another order changes bits -- so every algorithm must give the
oracle's left fold bit for bit.  Each switch point is run at the point
itself and one value either side, and the algorithm the channel reports is
checked against the table.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from message_fp16_all_amd import hr
from _gpu import assert_same_bits, needs_gpu, specials_mix, specials_mix_bf16, to_dev, to_dev_bf16, to_host

pytestmark = [pytest.mark.gpu, needs_gpu]

TIMEOUT_US = 2_000_000

# the automatic choice as hr.h states it: LL up to LL_MAX[W] values, the
# two-shot from TWO_MIN[W] values (W >= 3), the one-shot between
LL_MAX = {2: 20480, 3: 8192, 4: 4096, 5: 4096, 6: 2560, 7: 2048, 8: 1536}
TWO_MIN = {3: 98304, 4: 16384, 5: 10240, 6: 6144, 7: 5120, 8: 3072}


def expected_algorithm(W, n):
    if n <= LL_MAX[W]:
        return hr.HR_ALGO_LL
    if W >= 3 and n >= TWO_MIN[W]:
        return hr.HR_ALGO_TWO_SHOT
    return hr.HR_ALGO_ONE_SHOT


def sizes(W):
    out = [LL_MAX[W] - 1, LL_MAX[W], LL_MAX[W] + 1]
    if W in TWO_MIN:
        out += [TWO_MIN[W] - 1, TWO_MIN[W], TWO_MIN[W] + 1]
    return out


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# every group size with each of its switch points and one value either side
CASES = [(W, n) for W in range(2, 9) for n in sizes(W)]


@pytest.fixture(scope="module")
def group(request):
    W = request.param
    streams = hr.LoopbackStreams(0, n=W)
    ch = hr.Channel(world_size=W, timeout_us=TIMEOUT_US)
    yield W, ch, streams
    torch.cuda.synchronize()
    ch.destroy()
    streams.destroy()


@pytest.mark.parametrize("launch", ["per-rank", "group"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("group,n", CASES, indirect=["group"], ids=[f"W{W}-n{n}" for W, n in CASES])
def test_switch_point(group, n, dtype, launch):
    W, ch, streams = group
    k = sizes(W).index(n)
    want = expected_algorithm(W, n)
    assert ch.algorithm_for(n) == want, f"W={W} n={n}: algorithm {ch.algorithm_for(n)}, table says {want}"
    bf = dtype == "bf16"
    seed = 9000 + 100 * W + 10 * k + (5 if bf else 0)
    xb = [(specials_mix_bf16 if bf else specials_mix)(n, seed + r) for r in range(W)]
    xs = [(to_dev_bf16 if bf else to_dev)(b) for b in xb]
    outs = [torch.empty_like(x) for x in xs]
    say(f"switch point: W={W} n={n} algorithm={want} {dtype} {launch}")
    torch.cuda.synchronize()
    if launch == "group":
        ch.allreduce_group(xs, outs)
    else:
        for r in range(W):
            ch.allreduce(r, xs[r], outs[r], streams[r])
    torch.cuda.synchronize()
    assert ch.status() == hr.HR_OK, hr.hr_status_str(ch.status())
    ref = oracle.fold_bf16(xb) if bf else oracle.fold(xb)
    got = [o.view(torch.int16).cpu().numpy().view(np.uint16) for o in outs]
    for r, g in enumerate(got):
        assert_same_bits(g, ref, f"W={W} n={n} {dtype} {launch} rank {r}", bf16=bf)
        assert np.array_equal(g, got[0]), f"rank {r} differs from rank 0"
