#!/usr/bin/env python3
"""Benchmark of the FP16 all-reduce combine on one MI355X.

Headline (the JSON line's ``value``): the two-rank exchange through pinned
host slots at 32 tokens x hidden 4096 = 131072 binary16 values (256 KiB) per
rank, both ranks on one GPU (loopback).  Each rank's 1000 back-to-back calls
are captured into its own hipGraph; one step is one replay of both graphs
(1000 all-reduce calls), ``--steps`` replays are timed after ``--warmup``
untimed ones.  ``value`` is algorithmic GB/s = (G + 1) * N * 2 bytes per
call over the per-call time (G = 2); the roofline peak of this path is the
host-link bandwidth measured in the same run by a pinned hipMemcpy probe.

The last stdout line is one compact JSON object (a few KB): the headline,
its roofline, the eight-rank prefill-size fold's HBM roofline, the CPU
oracle baseline and a short table of every workload's us/call and fraction
of its roofline.  The full per-workload results -- the two-rank fold with
planted specials in HBM, the exchange at 1..32 tokens eager and
graph-captured under every algorithm, groups of 4 and 8 ranks, the
eight-rank decode-sized and prefill-sized folds in HBM (cold and warm
cache), the graph of 1000 exchange calls with fresh inputs per call,
bfloat16, the host-link probe -- go to the file named by ``--dump``.

Every timed output is checked bit for bit (NaN by class) against torch's own
binary16 adds on the device (a library cross-check; parity with the CPU
oracle is the test suite's job).  Only the CPU-baseline leg runs the oracle:
it times it and checks the headline's GPU output against it.

Usage: python bench.py [--steps K] [--warmup W] [--quick] [--no-cpu] [--dump FILE]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/call and GB/s (% of HBM / host-link roofline), FP16 all-reduce combine"
HBM_PEAK_GBS = 8000.0
HIDDEN = 4096
# device-side hold before timed back-to-back folds: longer than the host
# takes to queue 50 launches through the binding (about 1 ms)
FOLD_GATE_MS = 5.0
# all-reduce calls per rank captured in the headline graph; one step is one
# replay of both ranks' graphs
CALLS_PER_STEP = 1000
# largest size of the compact stdout line
LINE_MAX_BYTES = 4096


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20,
                   help=f"timed steps: replays of both ranks' {CALLS_PER_STEP}-call graphs")
    p.add_argument("--warmup", type=int, default=3, help="untimed replays before the timed ones")
    p.add_argument("--dump", default=os.path.join(ROOT, "gpurun_out", "bench_full.json"),
                   help="file that receives the full per-workload results")
    p.add_argument("--tokens", type=int, default=32)
    p.add_argument("--quick", action="store_true", help="headline only")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle timing")
    p.add_argument("--only", default="", help="comma list of sections: exchange,world,fold,c5,bf16")
    p.add_argument("--profile-kernel", choices=("fold", "fold-separate", "exchange", "copy", "link-probe"),
                   default=None,
                   help="run one kernel --reps times and nothing else (for rocprofv3 counters)")
    p.add_argument("--reps", type=int, default=10)
    p.add_argument("--numel", type=int, default=0,
                   help="values per rank of the exchange profiling target (0: workload 2 at "
                        "32 tokens, 131072); smaller sizes take the first values of it")
    p.add_argument("--num-blocks", type=int, default=0,
                   help="workgroups per rank of the channel the exchange profiling target makes "
                        "(0: the library's default)")
    p.add_argument("--link-mbps", type=int, default=0,
                   help="pacing rate of the channel the exchange profiling target makes (0: the "
                        "library's default; 4294967295: unpaced)")
    p.add_argument("--gate-ms", type=float, default=None,
                   help="hold both rank streams this long before a timed replay (default "
                        "5 ms + 10 us per call; raise it under a profiler, which slows graph "
                        "submission)")
    return p.parse_args()


# ------------------------------------------------------------------ helpers

class Ctx:
    def __init__(self):
        import numpy as np
        import torch
        from message_fp16_all_amd import hr, inputs
        self.np, self.torch, self.hr, self.inputs = np, torch, hr, inputs
        self.dev = torch.device("cuda", 0)
        self.streams = hr.LoopbackStreams(0)
        self._streams_w = {2: self.streams}
        self.gate_stream = torch.cuda.Stream()
        self.sleep_rate = None  # sleep-kernel cycles per ms

    def to_dev(self, bits):
        np, torch = self.np, self.torch
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(self.dev)

    def to_host(self, t):
        np, torch = self.np, self.torch
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def event(self):
        return self.torch.cuda.Event(enable_timing=True)

    def streams_for(self, world):
        if world not in self._streams_w:
            self._streams_w[world] = self.hr.LoopbackStreams(0, n=world)
        return self._streams_w[world]

    def destroy_streams(self):
        for st in self._streams_w.values():
            st.destroy()
        self._streams_w = {}

    def calibrate_sleep(self):
        torch = self.torch
        s = self.gate_stream
        cycles = 2_000_000
        for _ in range(2):
            e0, e1 = self.event(), self.event()
            with torch.cuda.stream(s):
                e0.record(s)
                torch.cuda._sleep(cycles)
                e1.record(s)
            s.synchronize()
            ms = e0.elapsed_time(e1)
        self.sleep_rate = cycles / max(ms, 1e-3)

    def gate(self, ms):
        """Event that completes `ms` milliseconds from now on the gate stream."""
        torch = self.torch
        if self.sleep_rate is None:
            self.calibrate_sleep()
        ev = torch.cuda.Event()
        with torch.cuda.stream(self.gate_stream):
            torch.cuda._sleep(int(self.sleep_rate * ms))
            ev.record(self.gate_stream)
        return ev


def same(np_mod, got, ref):
    """Bitwise equality of binary16 patterns, any NaN matching any NaN."""
    np = np_mod
    got = np.asarray(got, dtype=np.uint16)
    ref = np.asarray(ref, dtype=np.uint16)
    g_nan = ((got & 0x7C00) == 0x7C00) & ((got & 0x03FF) != 0)
    r_nan = ((ref & 0x7C00) == 0x7C00) & ((ref & 0x03FF) != 0)
    return bool(np.where(g_nan | r_nan, g_nan & r_nan, got == ref).all())


def torch_fold(c: Ctx, bits_list):
    """Left fold in rank order with torch's binary16 add on the device (each
    add rounds once to binary16), returned as bit patterns."""
    ts = [c.to_dev(b) for b in bits_list]
    acc = ts[0].clone()
    for t in ts[1:]:
        acc = acc + t
    return c.to_host(acc)


# ----------------------------------------------------------- host-link probe

def host_link_probe(c: Ctx):
    torch = c.torch
    out = {}
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    for label, nbytes in (("20KiB", 20 * 1024), ("256KiB", 256 * 1024), ("64MiB", 64 << 20)):
        h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        h2 = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        d = torch.empty(nbytes, dtype=torch.uint8, device=c.dev)
        d2 = torch.empty(nbytes, dtype=torch.uint8, device=c.dev)
        res = {}
        for kind in ("h2d", "d2h", "bidir"):
            times = []
            for it in range(25):
                e0, e1 = c.event(), c.event()
                torch.cuda.synchronize()
                e0.record(s0)
                s1.wait_event(e0)
                if kind in ("h2d", "bidir"):
                    with torch.cuda.stream(s0):
                        d.copy_(h, non_blocking=True)
                if kind in ("d2h", "bidir"):
                    with torch.cuda.stream(s1):
                        h2.copy_(d2, non_blocking=True)
                e_s1 = torch.cuda.Event()
                e_s1.record(s1)
                s0.wait_event(e_s1)
                e1.record(s0)
                torch.cuda.synchronize()
                if it >= 5:
                    times.append(e0.elapsed_time(e1) * 1e-3)
            t = statistics.median(times)
            moved = nbytes * (2 if kind == "bidir" else 1)
            res[kind] = {"us": round(t * 1e6, 2), "GBps": round(moved / t / 1e9, 2)}
        out[label] = res
    peak = max(out["64MiB"]["h2d"]["GBps"], out["64MiB"]["d2h"]["GBps"])
    return out, peak


# ------------------------------------------------------------ the exchange

def capture_calls(c: Ctx, ch, rank, xin, out, stream, calls):
    torch = c.torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for k in range(calls):
            xi = xin[k] if xin.dim() == 2 else xin
            xo = out[k] if out.dim() == 2 else out
            ch.allreduce(rank, xi, xo, stream)
    return g


def replay_all(c: Ctx, graphs, streams, gate_ms, replays=1):
    """Replay every rank's graph `replays` times behind a common device-side
    gate; returns (elapsed seconds on the GPU from gate open to all graphs
    done, host submission seconds)."""
    torch = c.torch
    torch.cuda.synchronize()
    gate = c.gate(gate_ms)
    for st in streams:
        st.wait_event(gate)
    e0, e1 = c.event(), c.event()
    e0.record(streams[0])
    t_host = time.perf_counter()
    for _ in range(replays):
        for g, st in zip(graphs, streams):
            with torch.cuda.stream(st):
                g.replay()
    t_host = time.perf_counter() - t_host
    for st in streams[1:]:
        ev = torch.cuda.Event()
        ev.record(st)
        streams[0].wait_event(ev)
    e1.record(streams[0])
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3, t_host


def replay_pair(c: Ctx, graphs, gate_ms):
    return replay_all(c, graphs, c.streams, gate_ms)


def eager_calls(c: Ctx, ch, x, o, streams, calls):
    torch = c.torch
    torch.cuda.synchronize()
    e0, e1 = c.event(), c.event()
    e0.record(streams[0])
    for st in streams[1:]:
        st.wait_event(e0)
    for _ in range(calls):
        for r, st in enumerate(streams):
            ch.allreduce(r, x[r], o[r], st)
    for st in streams[1:]:
        ev = torch.cuda.Event()
        ev.record(st)
        streams[0].wait_event(ev)
    e1.record(streams[0])
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / calls


ALGO_NAMES = {1: "one-shot", 2: "two-shot", 3: "low-latency"}


def exchange_workload(c: Ctx, tokens, steps, warmup, link_peak, eager_calls_n=200, gate_ms=None,
                      world=2, algorithm=0, replays=1, warm_replays=2):
    """`steps` calls per rank captured in one graph per rank; `warmup` eager
    calls, then `warm_replays` untimed replays, then `replays` timed ones."""
    torch, hr, inputs = c.torch, c.hr, c.inputs
    xb = inputs.workload2(tokens) if world == 2 else inputs.workload6(world, tokens)
    n = xb[0].size
    streams = c.streams_for(world)
    x = [c.to_dev(b) for b in xb]
    o = [torch.empty_like(t) for t in x]
    ref = torch_fold(c, xb)
    ch = hr.Channel(max_numel=hr.HR_DEFAULT_MAX_NUMEL, timeout_us=5_000_000, world_size=world,
                    algorithm=algorithm)
    taken = ch.algorithm_for(n)
    link_mbps = ch.info().link_mbps
    try:
        for _ in range(warmup):
            for r in range(world):
                ch.allreduce(r, x[r], o[r], streams[r])
        torch.cuda.synchronize()
        t_eager = eager_calls(c, ch, x, o, streams, eager_calls_n)
        graphs = [capture_calls(c, ch, r, x[r], o[r], streams[r], steps) for r in range(world)]
        if gate_ms is None:
            gate_ms = 5.0 + steps * replays * 0.01 * world / 2
        for _ in range(max(warm_replays, 1)):    # upload + settle, untimed
            replay_all(c, graphs, streams, gate_ms)
        for t in o:
            t.zero_()
        torch.cuda.synchronize()
        elapsed, host_s = replay_all(c, graphs, streams, gate_ms, replays)
        if ch.status() != hr.HR_OK:
            raise RuntimeError(f"exchange failed: {hr.hr_status_str(ch.status())}")
        got0 = c.to_host(o[0])
        exact = all(same(c.np, c.to_host(t), ref) for t in o)
        del graphs
        torch.cuda.synchronize()
    finally:
        ch.destroy()
    t_graph = elapsed / (steps * replays)
    alg = (world + 1) * n * 2
    two = taken == hr.HR_ALGO_TWO_SHOT
    if two:
        d2h = world * n * 2 + n * 2                 # contributions + folded shards
        h2d = 2 * (world - 1) * n * 2               # peers' shard parts + folded shards
    else:
        d2h = world * n * 2                 # each rank publishes its slice once
        h2d = world * (world - 1) * n * 2   # each rank reads every peer's slice
        if taken == hr.HR_ALGO_LL:          # every 6 bytes of values travel with 2 of call field
            units = -(-n // 8)              # and a unit of 8 values takes three 8-byte words
            d2h = world * units * 24
            h2d = world * (world - 1) * units * 24
    return {
        "world": world, "algorithm": ALGO_NAMES[taken], "link_mbps": link_mbps,
        "tokens": tokens, "N": n, "bytes_per_call": alg,
        "graph_us": round(t_graph * 1e6, 3), "graph_GBps": round(alg / t_graph / 1e9, 2),
        "graph_frac_link": round(alg / t_graph / 1e9 / link_peak, 4),
        "link_GBps_per_dir": round(max(d2h, h2d) / t_graph / 1e9, 2),
        "link_busiest_dir_frac": round(max(d2h, h2d) / t_graph / 1e9 / link_peak, 4),
        "eager_us": round(t_eager * 1e6, 3), "eager_GBps": round(alg / t_eager / 1e9, 2),
        "eager_frac_link": round(alg / t_eager / 1e9 / link_peak, 4),
        "graph_calls": steps, "replays": replays, "gate_ms": gate_ms,
        "host_submit_ms": round(host_s * 1e3, 3),
        "gate_covered_submit": host_s * 1e3 < gate_ms,
        "bit_exact": exact,
        "_elapsed_s": elapsed,
        "_out": got0,
    }


def group_workload(c: Ctx, tokens, steps, link_peak, world, algorithm=0, gate_ms=None):
    """Every rank of a loopback channel in one launch per call
    (hr_allreduce_group_f16): a graph of `steps` calls on one stream, timed
    behind a device-side gate; checked against torch's left fold."""
    torch, hr, inputs = c.torch, c.hr, c.inputs
    xb = inputs.workload2(tokens) if world == 2 else inputs.workload6(world, tokens)
    n = xb[0].size
    x = [c.to_dev(b) for b in xb]
    o = [torch.empty_like(t) for t in x]
    ref = torch_fold(c, xb)
    ch = hr.Channel(max_numel=hr.HR_DEFAULT_MAX_NUMEL, timeout_us=5_000_000, world_size=world,
                    algorithm=algorithm)
    taken = ch.algorithm_for(n)
    s = torch.cuda.Stream()
    try:
        for _ in range(20):
            ch.allreduce_group(x, o, s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(steps):
                ch.allreduce_group(x, o, s)
        if gate_ms is None:
            gate_ms = 5.0
        for rep in range(3):                     # two untimed (upload, settle), then the timed one
            if rep == 2:
                for t in o:
                    t.zero_()
            elapsed, _ = replay_all(c, [g], [s], gate_ms)
        if ch.status() != hr.HR_OK:
            raise RuntimeError(f"group exchange failed: {hr.hr_status_str(ch.status())}")
        exact = all(same(c.np, c.to_host(t), ref) for t in o)
        del g
        torch.cuda.synchronize()
    finally:
        ch.destroy()
    t = elapsed / steps
    alg = (world + 1) * n * 2
    return {"world": world, "launch": "group", "algorithm": ALGO_NAMES[taken], "tokens": tokens, "N": n,
            "graph_us": round(t * 1e6, 3), "graph_GBps": round(alg / t / 1e9, 2),
            "graph_frac_link": round(alg / t / 1e9 / link_peak, 4), "graph_calls": steps,
            "bit_exact": exact}


def exchange_prefill(c: Ctx, link_peak, sizes=(1 << 19, 1 << 23), calls=20):
    """Two-rank calls far above the decode cap (1 and 16 MiB per rank), on a
    channel made for them: paced one-shot (the automatic choice), the same
    unpaced, and the two-shot."""
    torch, hr, inputs = c.torch, c.hr, c.inputs
    rows = []
    for n in sizes:
        xb = [inputs.gaussian(n, 0.5, 77, r) for r in range(2)]
        x = [c.to_dev(b) for b in xb]
        o = [torch.empty_like(t) for t in x]
        ref = torch_fold(c, xb)
        for algo, rate in ((hr.HR_ALGO_AUTO, 0), (hr.HR_ALGO_AUTO, hr.HR_LINK_UNPACED),
                           (hr.HR_ALGO_TWO_SHOT, 0)):
            ch = hr.Channel(max_numel=n, timeout_us=5_000_000, algorithm=algo, link_mbps=rate)
            try:
                for _ in range(3):
                    for r in range(2):
                        ch.allreduce(r, x[r], o[r], c.streams[r])
                torch.cuda.synchronize()
                graphs = [capture_calls(c, ch, r, x[r], o[r], c.streams[r], calls) for r in range(2)]
                replay_pair(c, graphs, 20.0)
                for t in o:
                    t.zero_()
                elapsed, _ = replay_pair(c, graphs, 20.0)
                if ch.status() != hr.HR_OK:
                    raise RuntimeError(f"exchange failed: {hr.hr_status_str(ch.status())}")
                exact = all(same(c.np, c.to_host(t), ref) for t in o)
                algo_name = ALGO_NAMES[ch.algorithm_for(n)]
                del graphs
                torch.cuda.synchronize()
            finally:
                ch.destroy()
            t = elapsed / calls
            alg = 3 * n * 2
            rows.append({"N": n, "MiB_per_rank": n * 2 / 2**20, "algorithm": algo_name,
                         "paced": rate != hr.HR_LINK_UNPACED, "graph_us": round(t * 1e6, 2),
                         "graph_GBps": round(alg / t / 1e9, 2), "graph_frac_link": round(alg / t / 1e9 / link_peak, 4),
                         "link_GBps_per_dir": round(2 * n * 2 / t / 1e9, 2), "bit_exact": exact})
    return rows


def workload5(c: Ctx, link_peak, algorithm=0, gate_ms=None):
    torch, hr, inputs = c.torch, c.hr, c.inputs
    calls = 1000
    xb = inputs.workload5(calls=calls)
    n = xb.shape[2]
    xin = [c.to_dev(xb[r].reshape(-1)).view(calls, n) for r in range(2)]
    outs = [torch.empty_like(xin[r]) for r in range(2)]
    ch = hr.Channel(timeout_us=5_000_000, algorithm=algorithm)
    taken = ch.algorithm_for(n)
    try:
        for k in range(4):
            ch.allreduce(0, xin[0][k], outs[0][k], c.streams[0])
            ch.allreduce(1, xin[1][k], outs[1][k], c.streams[1])
        torch.cuda.synchronize()
        graphs = [capture_calls(c, ch, r, xin[r], outs[r], c.streams[r], calls) for r in range(2)]
        gate_ms = 15.0 if gate_ms is None else gate_ms
        replay_pair(c, graphs, gate_ms)
        outs[0].zero_()
        outs[1].zero_()
        torch.cuda.synchronize()
        elapsed, host_s = replay_pair(c, graphs, gate_ms)
        if ch.status() != hr.HR_OK:
            raise RuntimeError(f"exchange failed: {hr.hr_status_str(ch.status())}")
        ref = torch_fold(c, [xb[0].reshape(-1), xb[1].reshape(-1)])
        exact = (same(c.np, c.to_host(outs[0]).reshape(-1), ref) and
                 same(c.np, c.to_host(outs[1]).reshape(-1), ref))
        del graphs
        torch.cuda.synchronize()
    finally:
        ch.destroy()
    t = elapsed / calls
    alg = 3 * n * 2
    return {"N": n, "calls": calls, "algorithm": ALGO_NAMES[taken], "us_per_call": round(t * 1e6, 3),
            "GBps": round(alg / t / 1e9, 2), "frac_link": round(alg / t / 1e9 / link_peak, 4),
            "host_submit_ms": round(host_s * 1e3, 3), "gate_covered_submit": host_s * 1e3 < gate_ms,
            "bit_exact": exact}


# ------------------------------------------------------------ the HBM fold

def fold_time_warm(c: Ctx, ts, out, reps, gated=False):
    """Back-to-back launches on the same inputs.  Gated: the stream is held
    until every launch is queued, so the time is the GPU's (kernels and the
    dispatch gaps between them), not the host's submission rate."""
    torch, hr = c.torch, c.hr
    s = torch.cuda.current_stream()
    hr.reduce(ts, out)
    torch.cuda.synchronize()
    e0, e1 = c.event(), c.event()
    if gated:
        s.wait_event(c.gate(FOLD_GATE_MS))
    e0.record(s)
    for _ in range(reps):
        hr.reduce(ts, out)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def fold_time_graph(c: Ctx, ts, out, calls):
    """Per-launch time of a graph of `calls` folds; the stream is held behind
    a device-side gate until the replay is queued, so the host's submission
    of the graph is not timed."""
    torch, hr = c.torch, c.hr
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(calls):
            hr.reduce(ts, out, s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = c.event(), c.event()
    cur = torch.cuda.current_stream()
    cur.wait_event(c.gate(FOLD_GATE_MS))
    e0.record(cur)
    g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / calls


def fold_time_cold_single(c: Ctx, ts, out, reps, flush):
    """One launch after a read-only pass over 512 MiB has replaced the MALL's
    contents with clean lines; includes the single launch's dispatch."""
    torch, hr = c.torch, c.hr
    s = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        flush.sum()                          # reads 512 MiB, writes nothing back
        e0, e1 = c.event(), c.event()
        e0.record(s)
        hr.reduce(ts, out)
        e1.record(s)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    return statistics.median(times)


def fold_time_rotating(c: Ctx, sets, outs, reps=30):
    """Back-to-back launches cycling over >= 3 input sets (768 MiB for the
    prefill-sized workload), so each launch finds none of its inputs in the
    256 MB MALL; the per-launch time includes the dispatch gap.  The stream
    is held behind a device-side gate until all launches are queued, so the
    host's submission of the first launch is not timed."""
    torch, hr = c.torch, c.hr
    s = torch.cuda.current_stream()
    k = len(sets)
    for i in range(k):
        hr.reduce(sets[i], outs[i])
    torch.cuda.synchronize()
    res = []
    for _ in range(3):
        e0, e1 = c.event(), c.event()
        s.wait_event(c.gate(FOLD_GATE_MS))
        e0.record(s)
        for i in range(reps):
            hr.reduce(sets[i % k], outs[i % k])
        e1.record(s)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) * 1e-3 / reps)
    return statistics.median(res)


def fold_time_rotating_graph(c: Ctx, sets, outs, reps=30):
    """As fold_time_rotating, with the back-to-back launches captured in one
    graph, so host submission cannot gap them; gated like it, so the host's
    submission of the graph launch is not timed either."""
    torch, hr = c.torch, c.hr
    k = len(sets)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        for i in range(reps):
            hr.reduce(sets[i % k], outs[i % k], s)
    g.replay()
    torch.cuda.synchronize()
    res = []
    cur = torch.cuda.current_stream()
    for _ in range(3):
        e0, e1 = c.event(), c.event()
        cur.wait_event(c.gate(FOLD_GATE_MS))
        e0.record(cur)
        g.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) * 1e-3 / reps)
    del g
    return statistics.median(res)


def fold_graph_floor(c: Ctx, calls=100):
    """Per-call time of a graph of `calls` folds of one 16-byte unit (G = 1,
    N = 8, one workgroup): the launch floor of a graph node on this GPU,
    against which the decode-sized folds' graph rates are read."""
    torch = c.torch
    src = torch.zeros(8, dtype=torch.float16, device=c.dev)
    dst = torch.empty_like(src)
    t = fold_time_graph(c, [src], dst, calls)
    return {"G": 1, "N": 8, "graph_calls": calls, "graph_us": round(t * 1e6, 3)}


def fold_workload(c: Ctx, name, xs, prefill=False):
    torch = c.torch
    G, n = len(xs), xs[0].size
    ts = [c.to_dev(x) for x in xs]
    out = torch.empty_like(ts[0])
    alg = (G + 1) * n * 2

    def rate(prefix, t, res):
        res[prefix + "_us"] = round(t * 1e6, 3)
        res[prefix + "_GBps"] = round(alg / t / 1e9, 2)
        res[prefix + "_frac_hbm"] = round(alg / t / 1e9 / HBM_PEAK_GBS, 4)

    res = {"G": G, "N": n, "bytes_per_call": alg}
    # small calls: host-bound eager rate (the graph rate is the device's);
    # prefill-size calls: the device's back-to-back rate
    rate("warm", fold_time_warm(c, ts, out, reps=200 if n < 1_000_000 else 50, gated=prefill), res)
    if n < 1_000_000:
        rate("graph", fold_time_graph(c, ts, out, calls=100), res)
    ref = torch_fold(c, xs)
    exact = same(c.np, c.to_host(out), ref)
    if prefill:
        flush = torch.ones(512 << 20, dtype=torch.uint8, device=c.dev)
        rate("cold_single", fold_time_cold_single(c, ts, out, 15, flush), res)
        del flush
        # three sets of separately allocated contributions (the caller's layout)
        sets = [ts] + [[t.clone() for t in ts] for _ in range(2)]
        outs = [out] + [torch.empty_like(out) for _ in range(2)]
        rate("cold", fold_time_rotating(c, sets, outs), res)
        rate("cold_graph", fold_time_rotating_graph(c, sets, outs), res)
        exact = exact and all(same(c.np, c.to_host(o), ref) for o in outs)
        del sets, outs
        # the same with the contributions in one workspace per set, laid out
        # by hr_workspace_stride (2 MiB-rounded stride plus 4 KiB)
        wss = [c.hr.workspace(G, n) for _ in range(3)]
        sets = [views for _, views in wss]
        for st in sets:
            for g in range(G):
                st[g].copy_(ts[g])
        outs = [torch.empty_like(out) for _ in range(3)]
        rate("cold_workspace", fold_time_rotating(c, sets, outs), res)
        rate("cold_workspace_graph", fold_time_rotating_graph(c, sets, outs), res)
        exact = exact and all(same(c.np, c.to_host(o), ref) for o in outs)
        res["workspace_stride_values"] = c.hr.hr_workspace_stride(n)
        del wss, sets, outs
    torch.cuda.synchronize()
    res["bit_exact"] = exact
    del ts, out
    return res


# ------------------------------------------------------------------ bf16

def bf16_workloads(c: Ctx, link_peak):
    """The bfloat16 variants at the prefill-sized fold and the 256 KiB
    exchange, checked against torch's bfloat16 adds on the device."""
    torch, hr, inputs = c.torch, c.hr, c.inputs

    def dev(bits):
        return torch.from_numpy(c.np.ascontiguousarray(bits).view(c.np.int16)).view(
            torch.bfloat16).to(c.dev)

    res = {}
    n, G = 16_777_216, 8
    xs = [inputs.gaussian_bf16(n, 1.0, 4, r) for r in range(G)]
    wss = [hr.workspace(G, n, dtype=torch.bfloat16) for _ in range(3)]
    sets = [views for _, views in wss]
    for st in sets:
        for v, x in zip(st, xs):
            v.copy_(dev(x))
    outs = [torch.empty_like(sets[0][0]) for _ in range(3)]
    t_cold = fold_time_rotating(c, sets, outs)
    acc = sets[0][0].clone()
    for t in sets[0][1:]:
        acc = acc + t
    exact = all(torch.equal(o.view(torch.int16), acc.view(torch.int16)) for o in outs)
    alg = (G + 1) * n * 2
    res["fold_G8_N16777216_workspace"] = {"cold_us": round(t_cold * 1e6, 3),
                                "cold_GBps": round(alg / t_cold / 1e9, 2),
                                "cold_frac_hbm": round(alg / t_cold / 1e9 / HBM_PEAK_GBS, 4),
                                "bit_exact": exact}
    del wss, sets, outs, acc

    xb = [inputs.gaussian_bf16(131_072, 0.5, 2, r) for r in range(2)]
    x = [dev(b) for b in xb]
    o = [torch.empty_like(t) for t in x]
    ref = (x[0] + x[1]).view(torch.int16)
    ch = hr.Channel(timeout_us=5_000_000)
    try:
        for _ in range(20):
            ch.allreduce(0, x[0], o[0], c.streams[0])
            ch.allreduce(1, x[1], o[1], c.streams[1])
        torch.cuda.synchronize()
        steps = 500
        graphs = [capture_calls(c, ch, r, x[r], o[r], c.streams[r], steps) for r in range(2)]
        replay_pair(c, graphs, 10.0)
        elapsed, _ = replay_pair(c, graphs, 10.0)
        if ch.status() != hr.HR_OK:
            raise RuntimeError(hr.hr_status_str(ch.status()))
        exact = all(torch.equal(t.view(torch.int16), ref) for t in o)
        del graphs
        torch.cuda.synchronize()
    finally:
        ch.destroy()
    t = elapsed / steps
    alg = 3 * 131_072 * 2
    res["exchange_2rank_256KiB_graph"] = {"us": round(t * 1e6, 3), "GBps": round(alg / t / 1e9, 2),
                                          "frac_link": round(alg / t / 1e9 / link_peak, 4),
                                          "bit_exact": exact}
    return res


# -------------------------------------------------------------- CPU oracle

def cpu_baseline(c: Ctx, tokens, gpu_out):
    """The oracle, as it stands, on this host's cores: the headline's two
    contributions folded repeatedly for a bounded time.  Its result is also
    compared with the headline's GPU output."""
    import oracle
    x0b, x1b = c.inputs.workload2(tokens)
    n = x0b.size
    alg = 3 * n * 2
    cores = len(os.sched_getaffinity(0))
    res = {}
    # all cores, about 1.5 s wall
    calls, t0 = 0, time.perf_counter()
    used = 1
    while True:
        _, used = oracle.fold([x0b, x1b], threads=cores) if cores > 1 else (oracle.fold([x0b, x1b]), 1)
        calls += 1
        if time.perf_counter() - t0 > 1.5 and calls >= 3:
            break
    wall = time.perf_counter() - t0
    t = wall / calls
    res["all"] = {"us_per_call": t * 1e6, "GBps": alg / t / 1e9, "cores": used, "calls": calls,
                  "wall_s": wall}
    calls, t0 = 0, time.perf_counter()
    while True:
        oracle.fold([x0b, x1b])
        calls += 1
        if time.perf_counter() - t0 > 3.0 and calls >= 3:
            break
    t = (time.perf_counter() - t0) / calls
    res["one"] = {"us_per_call": t * 1e6, "GBps": alg / t / 1e9, "cores": 1, "calls": calls}
    res["gpu_matches_oracle"] = bool(oracle.same_bits(gpu_out, oracle.fold([x0b, x1b])).all())
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


# ---------------------------------------------------- counters (profiles/)

def code_text(src):
    """Source text without comments and with whitespace runs collapsed, so
    that a digest of it changes only when the code does."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_digest():
    """Digest of the kernel sources' code (comments and layout ignored)."""
    h = hashlib.sha256()
    for f in ("fold.hip", "exchange.hip", "hr_internal.h"):
        with open(os.path.join(ROOT, "message_fp16_all_amd", "csrc", f)) as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM/host bytes per launch of `kernel` from the committed counter
    summary, or None when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "counters.txt")
    if not os.path.exists(path):
        return None
    digest = source_digest()
    with open(path) as f:
        for line in f:
            m = re.match(r"traffic\s+(\S+)\s+(\S+)\s+sources=(\S+)", line.strip())
            if m and m.group(1) == kernel and m.group(3) == digest:
                return float(m.group(2))
    return None


# ------------------------------------------------------- profiling targets

def profile_kernel(which, reps, link_mbps=0, num_blocks=0, numel=0):
    """Launch one kernel `reps` times with nothing else timed, for
    rocprofv3 (counter collection serialises dispatches, so the exchange runs
    one rank against a peer that the host plays: the host writes the peer's
    slot and raises its flags before each launch)."""
    import ctypes
    import numpy as np
    import torch
    from message_fp16_all_amd import hr, inputs
    dev = torch.device("cuda", 0)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(dev)

    if which == "copy":
        # plain device copy of known size: 256 MiB read + 256 MiB written
        src = torch.ones(128 << 20, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy: {reps} x 256 MiB")
        return
    if which == "link-probe":
        # a channel that measures the host link at creation: its probe kernel
        # (1 warm-up + 3 timed launches) reads 16 MiB of device memory and
        # writes them to pinned host memory while it reads 16 MiB of pinned
        # host memory -- known host-read bytes, to read the memory counters by
        ch = hr.Channel(link_mbps=hr.HR_LINK_CALIBRATE)
        log(f"link probe: {ch.info().link_mbps} MB/s")
        ch.destroy()
        return
    if which in ("fold", "fold-separate"):
        # the cold protocol of the timed run: launches cycle over three sets
        # of inputs (864 MiB), so none finds its inputs in the MALL; the sets
        # are workspaces (hr_workspace_stride layout) or, for fold-separate,
        # separately allocated tensors
        xs = inputs.workload4()
        if which == "fold":
            wss = [hr.workspace(len(xs), xs[0].size) for _ in range(3)]
        else:
            wss = [(None, [torch.empty(xs[0].size, dtype=torch.float16, device=dev) for _ in xs])
                   for _ in range(3)]
        for _buf, ts in wss:
            for t, x in zip(ts, xs):
                t.copy_(to_dev(x))
        outs = [torch.empty_like(wss[0][1][0]) for _ in range(3)]
        torch.cuda.synchronize()
        for i in range(reps):
            hr.reduce(wss[i % 3][1], outs[i % 3])
        torch.cuda.synchronize()
        ts = wss[0][1]
        acc = ts[0].clone()
        for t in ts[1:]:
            acc = acc + t
        ok = all(bool(torch.equal(o.view(torch.int16), acc.view(torch.int16))) for o in outs[:min(reps, 3)])
        log(f"fold G=8 N={xs[0].size}: {reps} launches over 3 rotating "
            f"{'workspaces' if which == 'fold' else 'sets of separate tensors'}, bit_exact={ok}")
        return
    x0b, x1b = inputs.workload2(32)
    if numel:
        if not 0 < numel <= x0b.size:
            raise ValueError(f"--numel must be in 1..{x0b.size}")
        x0b, x1b = x0b[:numel].copy(), x1b[:numel].copy()
    n = x0b.size
    x0 = to_dev(x0b)
    out = torch.empty_like(x0)
    streams = hr.LoopbackStreams(0)
    # the one-shot at every size: the host-played peer follows its protocol
    ch = hr.Channel(timeout_us=2_000_000, link_mbps=link_mbps, num_blocks=num_blocks,
                    algorithm=hr.HR_ALGO_ONE_SHOT)
    info = ch.info()
    algo = ch.algorithm_for(n)
    if algo != hr.HR_ALGO_ONE_SHOT:
        raise RuntimeError("the host-played peer follows the one-shot protocol")
    ref = (x0 + to_dev(x1b)).view(torch.int16)
    ok = True
    try:
        for call in range(1, reps + 1):
            parity = call & 1
            peer_slot = info.host_slots + (2 * parity + 1) * info.slot_stride * 2
            ctypes.memmove(peer_slot, x1b.ctypes.data, n * 2)
            for b in range(info.num_blocks):
                info.host_flags[(1 * info.num_blocks + b) * info.flag_stride] = call
            torch.cuda.synchronize()
            ch.allreduce(0, x0, out, streams[0])
            streams[0].synchronize()
            if ch.status() != hr.HR_OK:
                raise RuntimeError(hr.hr_status_str(ch.status()))
            ok = ok and bool(torch.equal(out.view(torch.int16), ref))
    finally:
        torch.cuda.synchronize()
        ch.destroy()
        streams.destroy()
    log(f"exchange ({ALGO_NAMES[algo]}) rank 0 against a host-played peer, N={n}: {reps} calls, "
        f"bit_exact={ok}")


# -------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.profile_kernel:
        profile_kernel(args.profile_kernel, args.reps, args.link_mbps, args.num_blocks, args.numel)
        return
    c = Ctx()
    torch = c.torch
    only = set(filter(None, args.only.split(",")))
    want = (lambda s: not only or s in only)
    props = torch.cuda.get_device_properties(0)
    cfgs = {}

    log("host-link probe")
    probe, link_peak = host_link_probe(c)
    cfgs["host_link_probe"] = probe

    log(f"headline: exchange graphs of {CALLS_PER_STEP} calls, tokens={args.tokens}, "
        f"{args.warmup} untimed + {args.steps} timed replays")
    head = exchange_workload(c, args.tokens, CALLS_PER_STEP, 200, link_peak, gate_ms=args.gate_ms,
                             replays=args.steps, warm_replays=args.warmup)
    elapsed = head.pop("_elapsed_s")
    head_out = head.pop("_out")

    if not args.quick:
        if want("exchange"):
            rows = []
            for t in c.inputs.TOKENS_EXCHANGE:
                taken = set()
                for algo in (c.hr.HR_ALGO_AUTO, c.hr.HR_ALGO_ONE_SHOT, c.hr.HR_ALGO_LL,
                             c.hr.HR_ALGO_TWO_SHOT):
                    log(f"exchange tokens={t} algorithm={algo}")
                    r = exchange_workload(c, t, 500, 50, link_peak, algorithm=algo)
                    r.pop("_elapsed_s")
                    r.pop("_out")
                    if r["algorithm"] not in taken:       # AUTO first, then the others once
                        taken.add(r["algorithm"])
                        r["auto"] = algo == c.hr.HR_ALGO_AUTO
                        rows.append(r)
            cfgs["exchange_2rank_host_slots"] = rows
            log("exchange at prefill sizes (1 and 16 MiB per rank)")
            cfgs["exchange_2rank_prefill"] = exchange_prefill(c, link_peak)
        if want("world"):
            rows = []
            for w in (4, 8):
                for t in (1, 8, 32):
                    for algo in (c.hr.HR_ALGO_ONE_SHOT, c.hr.HR_ALGO_TWO_SHOT, c.hr.HR_ALGO_LL):
                        if algo == c.hr.HR_ALGO_LL and t * 4096 > 32768:
                            continue
                        log(f"exchange world={w} tokens={t} algorithm={algo}")
                        r = exchange_workload(c, t, 300, 20, link_peak, eager_calls_n=50, world=w,
                                              algorithm=algo, gate_ms=args.gate_ms)
                        r.pop("_elapsed_s")
                        r.pop("_out")
                        rows.append(r)
            cfgs["exchange_world_host_slots"] = rows
            rows = []
            for w in (2, 4, 8):
                for t in (1, 8, 32):
                    for algo in (c.hr.HR_ALGO_AUTO, c.hr.HR_ALGO_ONE_SHOT, c.hr.HR_ALGO_TWO_SHOT):
                        log(f"group launch world={w} tokens={t} algorithm={algo}")
                        rows.append(group_workload(c, t, 300, link_peak, w, algorithm=algo,
                                                   gate_ms=args.gate_ms))
            cfgs["exchange_group_launch_host_slots"] = rows
        if want("c5"):
            log("exchange graph of 1000 fresh calls, N=10240")
            cfgs["exchange_graph_1000_calls_N10240"] = workload5(c, link_peak, gate_ms=args.gate_ms)
            log("the same with the one-shot")
            cfgs["exchange_graph_1000_calls_N10240_one_shot"] = workload5(c, link_peak, c.hr.HR_ALGO_ONE_SHOT,
                                                                          gate_ms=args.gate_ms)
        if want("fold"):
            log("graph node floor: one-unit fold")
            cfgs["fold_graph_node_floor"] = fold_graph_floor(c)
            log("fold G=2 N=4096 with specials")
            cfgs["fold_G2_N4096_specials"] = fold_workload(c, "w1", c.inputs.workload1()[0])
            log("fold G=8 N=393216")
            cfgs["fold_G8_N393216"] = fold_workload(c, "w3", c.inputs.workload3())
            log("fold G=8 N=16777216")
            cfgs["fold_G8_N16777216"] = fold_workload(c, "w4", c.inputs.workload4(), prefill=True)

    if not args.quick and want("bf16"):
        log("bf16: fold G=8 N=16777216 and two-rank exchange at 256 KiB")
        cfgs["bf16"] = bf16_workloads(c, link_peak)

    cpu = None
    if not args.no_cpu:
        log("CPU oracle baseline")
        cpu = cpu_baseline(c, args.tokens, head_out)

    c.destroy_streams()
    full = {
        "args": {"steps": args.steps, "warmup": args.warmup, "tokens": args.tokens,
                 "quick": args.quick, "only": args.only},
        "elapsed_s": elapsed, "link_peak": link_peak, "headline": head, "configs": cfgs,
        "cpu": cpu,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "hip": torch.version.hip, "torch": torch.__version__},
        "host": {"cpu": cpu_model(), "cores": len(os.sched_getaffinity(0))},
        "traffic": {"exchange": measured_traffic("exchange_k<2,true,F16>"),
                    "fold": measured_traffic("fold_vec<8,4,F16>")},
    }
    dump = args.dump
    try:
        os.makedirs(os.path.dirname(os.path.abspath(dump)), exist_ok=True)
        with open(dump, "w") as f:
            json.dump(full, f, indent=1, default=str)
        log(f"full results: {dump}")
    except OSError as e:
        log(f"full results not written ({e})")
        dump = None
    print(json.dumps(make_line(full, dump), separators=(",", ":")), flush=True)


def _r(x, nd=3):
    return None if x is None else round(float(x), nd)


def summary_table(full):
    """Short per-workload table: name -> [us per call, fraction of roofline]
    (the host link P for the exchange, 8 TB/s for the folds)."""
    cfgs, t = full["configs"], {}
    for r in cfgs.get("exchange_2rank_host_slots", []):
        if r.get("auto"):
            t[f"C2_{r['tokens']}tok_graph"] = [_r(r["graph_us"], 2), _r(r["graph_frac_link"])]
    for r in cfgs.get("exchange_2rank_host_slots", []):
        if r["tokens"] == 1 and not r.get("auto") and r["algorithm"] == "one-shot":
            t["C2_1tok_one_shot_graph"] = [_r(r["graph_us"], 2), _r(r["graph_frac_link"])]
    for key, name in (("fold_G2_N4096_specials", "C1_fold_G2_N4096_graph"),
                      ("fold_G8_N393216", "C3_fold_G8_N393216_graph")):
        if key in cfgs:
            t[name] = [_r(cfgs[key]["graph_us"], 2), _r(cfgs[key]["graph_frac_hbm"])]
    f4 = cfgs.get("fold_G8_N16777216")
    if f4:
        for k, name in (("cold_workspace", "C4_fold_cold_workspace"),
                        ("cold_workspace_graph", "C4_fold_cold_workspace_graph"),
                        ("cold", "C4_fold_cold_separate"), ("cold_graph", "C4_fold_cold_separate_graph"),
                        ("warm", "C4_fold_warm_separate"), ("cold_single", "C4_fold_single_after_flush")):
            if k + "_us" in f4:
                t[name] = [_r(f4[k + "_us"], 2), _r(f4[k + "_frac_hbm"])]
    for key, name in (("exchange_graph_1000_calls_N10240", "C5_graph1000"),
                      ("exchange_graph_1000_calls_N10240_one_shot", "C5_graph1000_one_shot")):
        if key in cfgs:
            t[name] = [_r(cfgs[key]["us_per_call"], 2), _r(cfgs[key]["frac_link"])]
    if "fold_graph_node_floor" in cfgs:
        t["graph_node_floor"] = [_r(cfgs["fold_graph_node_floor"]["graph_us"], 2), None]
    for r in cfgs.get("exchange_2rank_prefill", []):
        if r["paced"] and r["algorithm"] == "one-shot":
            t[f"exchange_2rank_{r['MiB_per_rank']:g}MiB_graph"] = [_r(r["graph_us"], 1),
                                                                   _r(r["graph_frac_link"])]
    for r in cfgs.get("exchange_group_launch_host_slots", []):
        if r["world"] in (4, 8) and r["tokens"] in (1, 32) and r["algorithm"] == "two-shot":
            t.setdefault(f"group_W{r['world']}_{r['tokens']}tok_two_shot",
                         [_r(r["graph_us"], 2), _r(r["graph_frac_link"])])
    b = cfgs.get("bf16", {})
    if "fold_G8_N16777216_workspace" in b:
        x = b["fold_G8_N16777216_workspace"]
        t["bf16_C4_fold_cold_workspace"] = [_r(x["cold_us"], 2), _r(x["cold_frac_hbm"])]
    if "exchange_2rank_256KiB_graph" in b:
        x = b["exchange_2rank_256KiB_graph"]
        t["bf16_C2_32tok_graph"] = [_r(x["us"], 2), _r(x["frac_link"])]
    return t


def all_bit_exact(obj):
    """False when any result anywhere in `obj` has bit_exact false."""
    if isinstance(obj, dict):
        if obj.get("bit_exact") is False:
            return False
        return all(all_bit_exact(v) for v in obj.values())
    if isinstance(obj, list):
        return all(all_bit_exact(v) for v in obj)
    return True


def make_line(full, dump=None):
    """The compact JSON line bench.py ends with (at most LINE_MAX_BYTES)."""
    head, args, peak = full["headline"], full["args"], full["link_peak"]
    calls = args["steps"] * CALLS_PER_STEP
    t_call = full["elapsed_s"] / calls
    n = head["N"]
    alg = 3 * n * 2
    achieved = alg / t_call / 1e9
    traffic = full["traffic"]["exchange"]
    # the method's least traffic per rank launch: read the own input once,
    # write the own slot, read the peer's slot, write the output
    method_min = 4 * n * 2
    line = {
        "metric": METRIC,
        "value": round(achieved, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args["steps"],
        "warmup": args["warmup"],
        "ms_per_step": round(full["elapsed_s"] / args["steps"] * 1e3, 4),
        "us_per_call": round(t_call * 1e6, 3),
        "calls_per_step": CALLS_PER_STEP,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic: seeded N(0, 0.5^2) binary16 per rank",
        "config": {"workload": "two-rank FP16 all-reduce through pinned host slots, 32 tokens x "
                               "hidden 4096 (256 KiB per rank), loopback on one GPU, graph of "
                               f"{CALLS_PER_STEP} calls per rank",
                   "G": 2, "tokens": args["tokens"], "hidden": HIDDEN, "N": n, "bytes_per_call": alg,
                   "algorithm": head["algorithm"], "parallelism": "none (one GPU; two ranks as two "
                                                                  "co-resident launches)"},
        "roofline": {"bound": "host-link", "achieved": round(achieved, 3), "peak": peak, "unit": "GB/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": "hr::exchange_k<2, true, hr::F16>",
                     "kernel_avg_us": round(t_call * 1e6, 3),
                     "busiest_dir_GBps": head["link_GBps_per_dir"],
                     "busiest_dir_frac": head["link_busiest_dir_frac"],
                     "traffic_over_method_min": None if traffic is None else round(traffic / method_min, 4),
                     "peak_source": "pinned hipMemcpyAsync probe, max(H2D, D2H) at 64 MiB, this run",
                     "traffic_unit": "bytes per rank launch, HBM and host reads and writes (rocprofv3 "
                                     "TCC_EA0 DRAM/IO 32-byte request counters, copy scale 1.0)"},
        "bit_exact": head["bit_exact"] and all_bit_exact(full["configs"]),
    }
    f4 = full["configs"].get("fold_G8_N16777216")
    if f4:
        line["roofline_hbm_fold"] = {
            "bound": "hbm", "kernel": "hr::fold_vec<8, 4, hr::F16>", "G": 8, "N": f4["N"],
            "achieved": f4["cold_workspace_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": f4["cold_workspace_frac_hbm"], "kernel_avg_us": f4["cold_workspace_us"],
            "traffic": full["traffic"]["fold"],
            "protocol": "3 rotating workspaces (hr_workspace_stride layout), back-to-back",
            "graph_frac": f4.get("cold_workspace_graph_frac_hbm"),
            "separate_allocations_frac": f4.get("cold_frac_hbm"),
        }
    cpu = full.get("cpu")
    if cpu is not None:
        line["cpu_baseline"] = {
            "value": round(cpu["all"]["GBps"], 4), "unit": "GB/s", "cores": cpu["all"]["cores"],
            "kind": "oracle",
            "sample": f"the headline's two {n}-value contributions folded {cpu['all']['calls']} "
                      f"times by the C oracle on all cores (~{cpu['all']['wall_s']:.0f} s wall)",
            "us_per_call": round(cpu["all"]["us_per_call"], 2),
            "one_core_us_per_call": round(cpu["one"]["us_per_call"], 2),
            "gpu_headline_matches_oracle": cpu["gpu_matches_oracle"],
        }
    line["table_us_frac"] = summary_table(full)
    line["host"] = f"{full['host']['cores']} cores, {full['host']['cpu']}"[:60]
    line["full_results"] = None if dump is None else os.path.relpath(dump, ROOT)
    return line


if __name__ == "__main__":
    main()
