"""Per-phase timeline of the exchange kernels (a diagnostic tool).

Builds ``libhr_timeline.so``: the library compiled with ``HR_TIMELINE``, in
which lane 0 of every active exchange workgroup records wall-clock stamps of
its protocol phases (the GPU's constant-rate clock) and its poll count.  It
then runs graph-captured two-rank loopback calls through that build -- each
rank's calls captured in its own graph, both graphs released together by a
device-side gate -- and prints, per workload, the median and 90th percentile
of every phase over the calls of one replay.

Also, for groups of four and eight ranks in one launch, the two-shot: the
phases of its last-ending workgroup and of the owner of the same shard part.
For the two-rank LL cases it also prints how far apart the ranks' calls start
and, per rank, how often a lane 0 needed a second poll.

Phases of a one-shot workgroup: entry (its start after the call's first
workgroup), counter (loading the first input batch and advancing the call
counter), pace (its turn on the host link), publish (slot stores, their
acknowledgement, the flag), wait (the peers' flags), combine (peer reads,
fold, stores).  Of a low-latency (LL) workgroup: entry, counter, publish
(issuing the words), lane 0's hold before its first poll and its polling
until its peer words carry the call's field, the rest of the workgroup (the
barrier), and the fold and stores.
"gap" is the time from a call's last workgroup ending to the next call's
first workgroup starting (the kernel's end and the next graph node's
dispatch).  The clock's rate is taken from the same replay: stamp ticks over
the HIP-event time of the whole replay.

Usage:  python -m message_fp16_all_amd.timeline [--calls K] [--rebuild]
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

from . import build as _build
from . import hr, inputs

LIB = os.path.join(_build.PKG, "libhr_timeline.so")
WORDS = 8   # stamps t0..t5, count, call number per record


def ensure_built(rebuild: bool) -> str:
    srcs = _build.SOURCES + [os.path.join(_build.INCLUDE, "hr.h"), os.path.join(_build.CSRC, "hr_internal.h")]
    stale = not os.path.exists(LIB) or any(os.path.getmtime(f) > os.path.getmtime(LIB) for f in srcs)
    if rebuild or stale:
        _build.build(defines=("HR_TIMELINE",), lib=LIB)
    return LIB


def load_timeline_library():
    """Point the binding at the instrumented library (before anything loads
    libhr.so in this process) and bind its extra entry point."""
    if hr._lib is not None and hr.LIB_PATH != LIB:
        raise RuntimeError("libhr.so is already loaded in this process")
    hr.LIB_PATH = LIB
    lib = hr.load()
    lib.hr_timeline_attach.argtypes = [ctypes.c_void_p, ctypes.c_uint64]
    lib.hr_timeline_attach.restype = ctypes.c_int
    return lib


def run(lib, n, algorithm, calls, fresh_inputs):
    import torch
    streams = hr.LoopbackStreams(0)
    ch = hr.Channel(timeout_us=2_000_000, algorithm=algorithm)
    nb = ch.info().num_blocks
    try:
        sets = calls if fresh_inputs else 1        # fresh inputs per call, or one input reused
        xb = [np.stack([inputs.gaussian(n, 1.0 if fresh_inputs else 0.5, 5, r, k) for k in range(sets)])
              for r in range(2)]
        x = [torch.from_numpy(b.reshape(-1).view(np.int16)).view(torch.float16).cuda().view(sets, n)
             for b in xb]
        o = [torch.empty_like(t) for t in x]
        buf = torch.zeros(calls * 2 * nb * WORDS, dtype=torch.int64, device="cuda:0")
        hr._check(lib.hr_timeline_attach(buf.data_ptr(), calls), "hr_timeline_attach")
        for k in range(3):                                   # eager warm-up
            for r in range(2):
                ch.allreduce(r, x[r][k % sets], o[r][k % sets], streams[r])
        torch.cuda.synchronize()
        graphs = []
        for r in range(2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=streams[r]):
                for k in range(calls):
                    ch.allreduce(r, x[r][k % sets], o[r][k % sets], streams[r])
            graphs.append(g)
        gate_stream = torch.cuda.Stream()
        elapsed = 0.0
        for rep in range(3):
            torch.cuda.synchronize()
            buf.zero_()
            torch.cuda.synchronize()
            with torch.cuda.stream(gate_stream):
                torch.cuda._sleep(60_000_000)                # holds both ranks until both graphs are queued
                gate = torch.cuda.Event()
                gate.record(gate_stream)
            for s in streams:
                s.wait_event(gate)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(streams[0])
            for g, s in zip(graphs, streams):
                with torch.cuda.stream(s):
                    g.replay()
            done = torch.cuda.Event()
            done.record(streams[1])
            streams[0].wait_event(done)
            e1.record(streams[0])
            torch.cuda.synchronize()
            elapsed = e0.elapsed_time(e1) * 1e-3
        if ch.status() != hr.HR_OK:
            raise RuntimeError(hr.hr_status_str(ch.status()))
        del graphs
        rec = buf.cpu().numpy().view(np.uint64).reshape(calls, 2, nb, WORDS)
        algo = ch.algorithm_for(n)
        lib.hr_timeline_attach(None, 0)
    finally:
        torch.cuda.synchronize()
        ch.destroy()
        streams.destroy()
    return rec, elapsed, algo


def run_group(lib, world, n, algorithm, calls):
    """Every rank of a `world`-rank channel in one launch per call
    (hr_allreduce_group_f16), `calls` calls captured in one graph, released
    by a device-side gate; returns the records, the replay's time and the
    algorithm the calls took."""
    import torch
    ch = hr.Channel(world_size=world, timeout_us=2_000_000, algorithm=algorithm)
    nb = ch.info().num_blocks
    s = torch.cuda.Stream()
    try:
        xs = [torch.from_numpy(inputs.gaussian(n, 1.0, 6, r, 0).view(np.int16)).view(torch.float16).cuda()
              for r in range(world)]
        outs = [torch.empty_like(t) for t in xs]
        buf = torch.zeros(calls * world * nb * WORDS, dtype=torch.int64, device="cuda:0")
        hr._check(lib.hr_timeline_attach(buf.data_ptr(), calls), "hr_timeline_attach")
        for _ in range(3):
            ch.allreduce_group(xs, outs, s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(calls):
                ch.allreduce_group(xs, outs, s)
        gate_stream = torch.cuda.Stream()
        elapsed = 0.0
        for rep in range(3):
            torch.cuda.synchronize()
            buf.zero_()
            torch.cuda.synchronize()
            with torch.cuda.stream(gate_stream):
                torch.cuda._sleep(60_000_000)
                gate = torch.cuda.Event()
                gate.record(gate_stream)
            s.wait_event(gate)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            with torch.cuda.stream(s):
                g.replay()
            e1.record(s)
            torch.cuda.synchronize()
            elapsed = e0.elapsed_time(e1) * 1e-3
        if ch.status() != hr.HR_OK:
            raise RuntimeError(hr.hr_status_str(ch.status()))
        del g
        rec = buf.cpu().numpy().view(np.uint64).reshape(calls, world, nb, WORDS)
        algo = ch.algorithm_for(n)
        lib.hr_timeline_attach(None, 0)
    finally:
        torch.cuda.synchronize()
        ch.destroy()
    return rec, elapsed, algo


def analyse_two_shot(rec, elapsed):
    """Phases of the two-shot's last-ending workgroup (usually a gathering
    rank's) and of the owner of the same shard part in the same call."""
    calls, world, nb, _ = rec.shape
    active = rec[..., 7] != 0
    t = rec[..., :6].astype(np.int64)
    e = rec[..., 7]
    order = np.argsort(np.where(active, e, np.iinfo(np.uint64).max).min(axis=(1, 2)))
    t, active, role = t[order], active[order], rec[..., 6][order]
    big = np.iinfo(np.int64).max
    start = np.where(active, t[..., 0], big).min(axis=(1, 2))
    end = np.where(active, t[..., 5], 0).max(axis=(1, 2))
    ticks_per_us = (end[-1] - start[0]) / (elapsed * 1e6)
    flat_end = np.where(active, t[..., 5], 0).reshape(calls, -1)
    crit = flat_end.argmax(axis=1)
    cr, cb = crit // nb, crit % nb                      # rank and workgroup of the critical one
    tc = t[np.arange(calls), cr, cb]
    # the owner of that workgroup's shard part: the rank whose role there is 1
    own_rank = np.array([int(np.argmax(role[k, :, cb[k]] == 1)) for k in range(calls)])
    to = t[np.arange(calls), own_rank, cb]
    ph = {"entry": tc[:, 0] - start,
          "counter": tc[:, 1] - tc[:, 0],
          "pace (turn on the link)": tc[:, 2] - tc[:, 1],
          "publish (stores, ack, flag)": tc[:, 3] - tc[:, 2],
          "its wait (owner: peers' flags; other: the owner's flag 2)": tc[:, 4] - tc[:, 3],
          "its last step (owner: reads, fold, shard and flag 2; other: shard copy)": tc[:, 5] - tc[:, 4],
          "the shard owner: publish done to peers' flags seen": to[:, 4] - to[:, 3],
          "the shard owner: reads, fold, shard and flag 2": to[:, 5] - to[:, 4],
          "the owner's flag 2 raised to this workgroup seeing it": tc[:, 4] - to[:, 5],
          "gap to the next call's first workgroup": np.concatenate([start[1:] - end[:-1], [0]]),
          "call period (start to next start)": np.concatenate([np.diff(start), [0]])}
    skip = calls // 10
    rows = []
    for name, v in ph.items():
        v = v[skip:-1] / ticks_per_us
        rows.append((name, float(np.median(v)), float(np.percentile(v, 90))))
    crit_role = role[np.arange(calls), cr, cb][skip:]
    nact = int(active[skip:].sum(axis=(1, 2)).max())
    return rows, elapsed * 1e6 / calls, ticks_per_us, nact, float(np.mean(crit_role == 2))


def analyse(rec, elapsed, algo):
    calls = rec.shape[0]
    active = rec[..., 7] != 0
    t = rec[..., :6].astype(np.int64)
    e = rec[..., 7]
    order = np.argsort(np.where(active, e, np.iinfo(np.uint64).max).min(axis=(1, 2)))
    t, active = t[order], active[order]
    big = np.iinfo(np.int64).max
    start = np.where(active, t[..., 0], big).min(axis=(1, 2))
    end = np.where(active, t[..., 5], 0).max(axis=(1, 2))
    ticks_per_us = (end[-1] - start[0]) / (elapsed * 1e6)
    per_call_us = elapsed * 1e6 / calls
    # the workgroup that ends last in each call
    flat_end = np.where(active, t[..., 5], 0).reshape(calls, -1)
    crit = flat_end.argmax(axis=1)
    tc = t.reshape(calls, -1, 6)[np.arange(calls), crit]
    ph = {"entry": tc[:, 0] - start,
          "counter": tc[:, 1] - tc[:, 0]}
    if algo == hr.HR_ALGO_LL:
        ph.update({"publish (issue words)": tc[:, 2] - tc[:, 1],
                   "lane 0's hold and polls until its peer words match": tc[:, 3] - tc[:, 2],
                   "rest of the workgroup (barrier)": tc[:, 4] - tc[:, 3],
                   "fold + store": tc[:, 5] - tc[:, 4]})
    else:
        ph.update({"pace (turn on the link)": tc[:, 2] - tc[:, 1],
                   "publish (stores, ack, flag)": tc[:, 3] - tc[:, 2],
                   "wait (peer flags)": tc[:, 4] - tc[:, 3],
                   "combine (peer reads, fold, stores)": tc[:, 5] - tc[:, 4]})
    ph["gap to the next call's first workgroup"] = start[1:] - end[:-1]
    ph["call period (start to next start)"] = np.diff(start)
    skip = calls // 10                                         # the replay's head
    rows = []
    for name, v in ph.items():
        v = v[skip:] / ticks_per_us
        rows.append((name, float(np.median(v)), float(np.percentile(v, 90))))
    polls = rec[..., 6][order].reshape(calls, -1)[np.arange(calls), crit][skip:]
    nact = int(active[skip:].sum(axis=(1, 2)).max())
    return rows, per_call_us, ticks_per_us, nact, float(np.median(polls))


def analyse_ll_ranks(rec, ticks_per_us):
    """Two-rank LL calls, rank by rank: how far rank 1's first workgroup
    starts after rank 0's, and, per rank, the share of calls in which some
    active workgroup's lane 0 needed a second poll, with the median skew of
    those calls.  Returns (skew median, p10, p90 in us, {rank: (share, median
    skew of those calls)}); the replay's first tenth is skipped."""
    calls = rec.shape[0]
    active = rec[..., 7] != 0
    t = rec[..., :6].astype(np.int64)
    e = rec[..., 7]
    order = np.argsort(np.where(active, e, np.iinfo(np.uint64).max).min(axis=(1, 2)))
    t, active, polls = t[order], active[order], rec[..., 6][order].astype(np.int64)
    big = np.iinfo(np.int64).max
    start = np.where(active, t[..., 0], big).min(axis=2)               # [calls, rank]
    skip = calls // 10
    skew = (start[skip:, 1] - start[skip:, 0]) / ticks_per_us
    out = {}
    for r in range(rec.shape[1]):
        extra = (np.where(active[skip:, r], polls[skip:, r], 0) >= 2).any(axis=1)
        share = float(extra.mean())
        out[r] = (share, float(np.median(skew[extra])) if extra.any() else float("nan"))
    return (float(np.median(skew)), float(np.percentile(skew, 10)), float(np.percentile(skew, 90))), out


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--calls", type=int, default=1000)
    p.add_argument("--rebuild", action="store_true")
    args = p.parse_args(argv)
    ensure_built(args.rebuild)
    lib = load_timeline_library()
    cases = [("two ranks, N = 10240 (2 x 5120), fresh inputs per call, LL", 10_240, hr.HR_ALGO_AUTO, True),
             ("two ranks, N = 4096 (one token), fresh inputs per call, LL", 4096, hr.HR_ALGO_AUTO, True),
             ("two ranks, N = 10240, one-shot", 10_240, hr.HR_ALGO_ONE_SHOT, True),
             ("two ranks, N = 131072 (32 x 4096), one-shot", 131_072, hr.HR_ALGO_AUTO, False)]
    for world, n in ((4, 4096), (8, 4096)):
        rec, elapsed, algo = run_group(lib, world, n, hr.HR_ALGO_TWO_SHOT, args.calls)
        rows, per_call, tpu, nact, gather = analyse_two_shot(rec, elapsed)
        print(f"\n### {world} ranks in one group launch, N = {n}, two-shot: graph of {args.calls} calls\n")
        print(f"{per_call:.3f} us per call from HIP events; {nact} active workgroups per call "
              f"(all ranks); clock {tpu:.2f} ticks/us; the last-ending workgroup was a gathering "
              f"rank's in {100 * gather:.0f} % of the calls\n")
        print("| phase | median us | p90 us |")
        print("|---|---|---|")
        for name, med, p90 in rows:
            print(f"| {name} | {med:.3f} | {p90:.3f} |")
        sys.stdout.flush()
    for title, n, algorithm, fresh in cases:
        rec, elapsed, algo = run(lib, n, algorithm, args.calls, fresh)
        rows, per_call, tpu, nact, polls = analyse(rec, elapsed, algo)
        print(f"\n### {title}: graph of {args.calls} calls per rank\n")
        print(f"{per_call:.3f} us per call from HIP events; {nact} active workgroups per call "
              f"(both ranks); clock {tpu:.2f} ticks/us; critical workgroup's lane 0 polled "
              f"{polls:.0f} times (LL)\n")
        print("| phase of the last-ending workgroup | median us | p90 us |")
        print("|---|---|---|")
        for name, med, p90 in rows:
            print(f"| {name} | {med:.3f} | {p90:.3f} |")
        if algo == hr.HR_ALGO_LL:
            (sm, s10, s90), ranks = analyse_ll_ranks(rec, tpu)
            print(f"\nRank 1's first workgroup starts {sm:+.3f} us after rank 0's (median; p10 "
                  f"{s10:+.3f}, p90 {s90:+.3f}).")
            for r, (share, sk) in ranks.items():
                print(f"Rank {r}: some lane 0 polled twice or more in {100 * share:.0f} % of the calls "
                      f"(median skew of those calls {sk:+.3f} us).")
        sys.stdout.flush()


if __name__ == "__main__":
    main()
