"""Randomised parity of the exchange: a seeded sequence of calls mixing
sizes (decode to prefill), algorithms, group sizes, element types, buffer
alignments and in-place calls, every output compared bit for bit with the
oracle's left fold (NaN by class)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from message_fp16_all_amd import hr
from _gpu import assert_same_bits, needs_gpu, specials_mix, specials_mix_bf16, to_dev, to_dev_bf16, to_host

pytestmark = [pytest.mark.gpu, needs_gpu]

CALLS = 400
MAX_NUMEL = 1 << 20


def _buffers(bits, offset, bf16):
    """A device copy of `bits` starting `offset` values into its allocation."""
    pad = np.zeros(offset, np.uint16)
    dev = (to_dev_bf16 if bf16 else to_dev)(np.concatenate([pad, bits]))
    return dev[offset:]


@pytest.mark.parametrize("world,algorithm", [(2, hr.HR_ALGO_AUTO), (2, hr.HR_ALGO_TWO_SHOT),
                                             (2, hr.HR_ALGO_LL), (3, hr.HR_ALGO_AUTO),
                                             (4, hr.HR_ALGO_ONE_SHOT)],
                         ids=["W2-auto", "W2-two", "W2-ll", "W3-auto", "W4-one"])
def test_random_call_sequence(world, algorithm):
    rng = np.random.default_rng(2024 + 10 * world + algorithm)
    streams = hr.LoopbackStreams(0, n=world)
    ch = hr.Channel(world_size=world, max_numel=MAX_NUMEL, timeout_us=2_000_000, algorithm=algorithm)
    try:
        for call in range(CALLS):
            # sizes log-uniform over [1, MAX_NUMEL]
            n = int(min(MAX_NUMEL, max(1, round(2 ** rng.uniform(0, 20)))))
            bf16 = bool(rng.integers(0, 2))
            in_place = bool(rng.integers(0, 4) == 0)
            offsets = [int(rng.choice([0, 0, 0, 1, 3])) for _ in range(world)]
            seed = int(rng.integers(0, 1 << 30))
            make = specials_mix_bf16 if bf16 else specials_mix
            xb = [make(n, seed=seed + r) for r in range(world)]
            xs = [_buffers(xb[r], offsets[r], bf16) for r in range(world)]
            outs = xs if in_place else [_buffers(np.zeros(n, np.uint16), offsets[r], bf16) for r in range(world)]
            print(f"call {call}: W={world} n={n} bf16={bf16} in_place={in_place} offsets={offsets} "
                  f"algorithm={ch.algorithm_for(n)}", flush=True)
            sys.stdout.flush()
            torch.cuda.synchronize()
            for r in rng.permutation(world):
                ch.allreduce(int(r), xs[r], outs[r], streams[int(r)])
            for s in streams:
                s.synchronize()
            assert ch.status() == hr.HR_OK, hr.hr_status_str(ch.status())
            ref = oracle.fold_bf16(xb) if bf16 else oracle.fold(xb)
            for r in range(world):
                assert_same_bits(to_host(outs[r]), ref, f"call {call} rank {r}", bf16=bf16)
    finally:
        torch.cuda.synchronize()
        ch.destroy()
        streams.destroy()


def test_random_fold_sequence():
    """hr_reduce_* on a seeded sequence of G (1..16), sizes, alignments,
    element types, in-place outputs and the workspace layout."""
    rng = np.random.default_rng(77)
    for call in range(300):
        G = int(rng.integers(1, 17))
        n = int(max(1, round(2 ** rng.uniform(0, 21))))
        bf16 = bool(rng.integers(0, 2))
        layout = rng.choice(["separate", "workspace", "in_place"])
        seed = int(rng.integers(0, 1 << 30))
        make = specials_mix_bf16 if bf16 else specials_mix
        xb = [make(n, seed=seed + g) for g in range(G)]
        dt = torch.bfloat16 if bf16 else torch.float16
        print(f"fold {call}: G={G} n={n} bf16={bf16} layout={layout}", flush=True)
        if layout == "workspace":
            _buf, ts = hr.workspace(G, n, dtype=dt)
            for t, b in zip(ts, xb):
                t.copy_((to_dev_bf16 if bf16 else to_dev)(b))
            out = torch.empty(n, dtype=dt, device="cuda:0")
        else:
            offs = [int(rng.choice([0, 0, 1, 5])) for _ in range(G)]
            ts = [_buffers(b, o, bf16) for b, o in zip(xb, offs)]
            out = ts[int(rng.integers(0, G))] if layout == "in_place" else _buffers(np.zeros(n, np.uint16), 0, bf16)
        hr.reduce(ts, out)
        torch.cuda.synchronize()
        ref = oracle.fold_bf16(xb) if bf16 else oracle.fold(xb)
        assert_same_bits(to_host(out), ref, f"fold {call}", bf16=bf16)


def test_low_latency_graph_replayed_with_fresh_inputs():
    """10 replays of a 1000-call low-latency graph per rank (N = 10240, the
    decode workload), fresh inputs before every replay: every one of the
    20000 outputs is compared with the oracle.  Guards the low-latency
    protocol's reliance on whole 8-byte words over many calls."""
    calls, n, replays = 1000, 10_240, 10
    streams = hr.LoopbackStreams(0)
    ch = hr.Channel(timeout_us=2_000_000, algorithm=hr.HR_ALGO_LL)
    try:
        assert ch.algorithm_for(n) == hr.HR_ALGO_LL
        xin = [torch.empty((calls, n), dtype=torch.float16, device="cuda:0") for _ in range(2)]
        outs = [torch.empty_like(x) for x in xin]
        ch.allreduce(0, xin[0][0], outs[0][0], streams[0])
        ch.allreduce(1, xin[1][0], outs[1][0], streams[1])
        torch.cuda.synchronize()
        graphs = []
        for r in range(2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=streams[r]):
                for k in range(calls):
                    ch.allreduce(r, xin[r][k], outs[r][k], streams[r])
            graphs.append(g)
        rng = np.random.default_rng(5)
        for rep in range(replays):
            xb = [rng.standard_normal((calls, n), dtype=np.float32).astype(np.float16).view(np.uint16)
                  for _ in range(2)]
            for r in range(2):
                xin[r].copy_(to_dev(xb[r].reshape(-1)).view(calls, n))
            torch.cuda.synchronize()
            for r in range(2):
                with torch.cuda.stream(streams[r]):
                    graphs[r].replay()
            for s in streams:
                s.synchronize()
            assert ch.status() == hr.HR_OK
            ref = oracle.add(xb[0].reshape(-1), xb[1].reshape(-1))
            for r in range(2):
                assert_same_bits(to_host(outs[r]).reshape(-1), ref, f"replay {rep} rank {r}")
    finally:
        torch.cuda.synchronize()
        ch.destroy()
        streams.destroy()


@pytest.mark.parametrize("world,launch", [(2, "per-rank"), (4, "per-rank"), (4, "group"), (8, "group")],
                         ids=["W2-per-rank", "W4-per-rank", "W4-group", "W8-group"])
def test_random_sizes_queued_without_host_sync(world, launch):
    """A seeded sequence of calls whose sizes cross every switch point of the
    automatic choice (so consecutive calls change algorithm, and with it the
    slots, flags and low-latency words they use), all queued before the host
    waits once: ranks run up to a call apart on the device, which is when the
    double buffering by call parity (the 1Cat-vLLM page, "Purpose") has to
    hold.  Each call has its own buffers; every output is then compared with
    the oracle's left fold."""
    calls, max_numel = 240, 1 << 18
    rng = np.random.default_rng(4100 + world + (100 if launch == "group" else 0))
    streams = hr.LoopbackStreams(0, n=world) if launch == "per-rank" else None
    group_stream = torch.cuda.Stream() if launch == "group" else None
    ch = hr.Channel(world_size=world, max_numel=max_numel, timeout_us=2_000_000)
    try:
        sizes = [int(min(max_numel, max(1, round(2 ** rng.uniform(0, 18))))) for _ in range(calls)]
        algos = {ch.algorithm_for(n) for n in sizes}
        assert algos == {hr.HR_ALGO_LL, hr.HR_ALGO_ONE_SHOT} | ({hr.HR_ALGO_TWO_SHOT} if world > 2 else set())
        xb = [[specials_mix(n, seed=int(rng.integers(0, 1 << 30))) for _ in range(world)] for n in sizes]
        xs = [[to_dev(b) for b in row] for row in xb]
        outs = [[torch.empty_like(x) for x in row] for row in xs]
        torch.cuda.synchronize()
        print(f"queueing {calls} calls, W={world} {launch}, algorithms {sorted(algos)}", flush=True)
        for c in range(calls):
            if launch == "group":
                ch.allreduce_group(xs[c], outs[c], group_stream)
            else:
                for r in rng.permutation(world):
                    ch.allreduce(int(r), xs[c][int(r)], outs[c][int(r)], streams[int(r)])
        torch.cuda.synchronize()
        assert ch.status() == hr.HR_OK, hr.hr_status_str(ch.status())
        for c in range(calls):
            ref = oracle.fold(xb[c])
            for r in range(world):
                assert_same_bits(to_host(outs[c][r]), ref, f"call {c} n={sizes[c]} rank {r}")
    finally:
        torch.cuda.synchronize()
        ch.destroy()
        if streams is not None:
            streams.destroy()
