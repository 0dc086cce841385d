"""GPU parity of hr_allreduce_f16: the two-rank exchange through host slots.

Both ranks run on one GPU as two concurrently resident launches on two
streams that each own a hardware queue (loopback).  Every output value of both ranks is
compared bit for bit (NaN by class) with the oracle's single-rounding sum of
the two contributions, and the two ranks' outputs with each other.
"""
import ctypes
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


@pytest.fixture
def streams():
    # one dedicated hardware queue per rank, so the two launches of a call
    # always run at the same time
    ls = hr.LoopbackStreams(0)
    yield ls
    ls.destroy()


# AUTO takes the low-latency one-shot up to 20480 values and the one-shot
# above; the two-shot is also correct for two ranks (each rank owns half of
# the values), so the whole two-rank battery runs on every algorithm
ALGOS = [hr.HR_ALGO_AUTO, hr.HR_ALGO_ONE_SHOT, hr.HR_ALGO_TWO_SHOT, hr.HR_ALGO_LL]
ALGO_IDS = ["auto", "one-shot", "two-shot", "ll"]


@pytest.fixture(params=ALGOS, ids=ALGO_IDS)
def channel(request):
    ch = hr.Channel(max_numel=hr.HR_DEFAULT_MAX_NUMEL, timeout_us=TIMEOUT_US, algorithm=request.param)
    yield ch
    torch.cuda.synchronize()
    ch.destroy()


def loopback(ch, x0, x1, out0, out1, streams):
    s0, s1 = streams
    torch.cuda.synchronize()
    ch.allreduce(0, x0, out0, s0)
    ch.allreduce(1, x1, out1, s1)
    s0.synchronize()
    s1.synchronize()
    assert ch.status() == hr.HR_OK, hr.hr_status_str(ch.status())


def check_pair(out0, out1, x0_bits, x1_bits, what):
    ref = oracle.add(x0_bits, x1_bits)
    g0, g1 = to_host(out0), to_host(out1)
    assert_same_bits(g0, ref, f"{what} rank 0")
    assert_same_bits(g1, ref, f"{what} rank 1")
    assert np.array_equal(g0, g1), f"{what}: ranks differ"


@pytest.mark.parametrize("tokens", inputs.TOKENS_EXCHANGE)
def test_workload2_loopback(channel, streams, tokens):
    x0b, x1b = inputs.workload2(tokens)
    say(f"exchange: workload 2, tokens={tokens} N={x0b.size}")
    x0, x1 = to_dev(x0b), to_dev(x1b)
    out0, out1 = torch.empty_like(x0), torch.empty_like(x1)
    loopback(channel, x0, x1, out0, out1, streams)
    check_pair(out0, out1, x0b, x1b, f"tokens {tokens}")


def test_edge_table_through_the_exchange(channel, streams):
    a, b = inputs.edge_pairs()
    x0, x1 = to_dev(a), to_dev(b)
    out0, out1 = torch.empty_like(x0), torch.empty_like(x1)
    loopback(channel, x0, x1, out0, out1, streams)
    ref = oracle.add(a, b)
    assert_same_bits(to_host(out0), ref, "edge rank 0")
    assert_same_bits(to_host(out1), ref, "edge rank 1")


def test_consecutive_calls_alternate_parity_with_varying_sizes(channel, streams):
    sizes = [4096, 131_072, 1, 65_541, 8, 9, 131_072, 32_768, 7, 100_000, 4096, 2]
    for call, n in enumerate(sizes):
        x0b = specials_mix(n, seed=10 * call)
        x1b = specials_mix(n, seed=10 * call + 1)
        x0, x1 = to_dev(x0b), to_dev(x1b)
        out0, out1 = torch.empty_like(x0), torch.empty_like(x1)
        loopback(channel, x0, x1, out0, out1, streams)
        check_pair(out0, out1, x0b, x1b, f"call {call} n={n}")


def test_back_to_back_calls_without_host_sync(channel, streams):
    """Many calls queued at once on both streams: the slot parity alternates
    on the device while the host never waits between calls."""
    s0, s1 = streams
    calls, n = 64, 16_384
    x = [[inputs.gaussian(n, 1.0, 20, r, c) for c in range(calls)] for r in range(2)]
    xin = [torch.stack([to_dev(v) for v in x[r]]) for r in range(2)]
    outs = [torch.empty_like(xin[r]) for r in range(2)]
    torch.cuda.synchronize()
    for c in range(calls):
        channel.allreduce(0, xin[0][c], outs[0][c], s0)
        channel.allreduce(1, xin[1][c], outs[1][c], s1)
    s0.synchronize()
    s1.synchronize()
    assert channel.status() == hr.HR_OK
    for c in range(calls):
        check_pair(outs[0][c], outs[1][c], x[0][c], x[1][c], f"call {c}")


@pytest.mark.parametrize("n", [1, 7, 8, 9, 1000, 4097, 131_071, 131_072])
def test_ragged_sizes(channel, streams, n):
    x0b, x1b = specials_mix(n, seed=n), specials_mix(n, seed=n + 1)
    x0, x1 = to_dev(x0b), to_dev(x1b)
    out0, out1 = torch.empty_like(x0), torch.empty_like(x1)
    loopback(channel, x0, x1, out0, out1, streams)
    check_pair(out0, out1, x0b, x1b, f"n={n}")


@pytest.mark.parametrize("offset", [1, 3])
def test_unaligned_buffers(channel, streams, offset):
    n = 20_000
    x0b, x1b = specials_mix(n, 5), specials_mix(n, 6)
    pad = np.zeros(offset, np.uint16)
    b0, b1 = to_dev(np.concatenate([pad, x0b])), to_dev(np.concatenate([pad, x1b]))
    o0 = torch.zeros(n + offset, dtype=torch.float16, device="cuda:0")
    o1 = torch.zeros(n + offset, dtype=torch.float16, device="cuda:0")
    loopback(channel, b0[offset:], b1[offset:], o0[offset:], o1[offset:], streams)
    check_pair(o0[offset:], o1[offset:], x0b, x1b, f"offset {offset}")
    assert np.all(to_host(o0[:offset]) == 0) and np.all(to_host(o1[:offset]) == 0)


@pytest.mark.parametrize("unaligned_rank", [0, 1])
@pytest.mark.parametrize("n", [4096 * 32, 70_001, 9])
def test_ranks_on_different_access_paths(channel, streams, unaligned_rank, n):
    """One rank's buffers are 16-byte aligned, the other's only 2-byte
    aligned: the ranks take different access paths but must split the
    values between workgroups identically."""
    x0b, x1b = specials_mix(n, 11), specials_mix(n, 12)
    bufs, outs = [], []
    for r, xb in enumerate((x0b, x1b)):
        off = 1 if r == unaligned_rank else 0
        buf = to_dev(np.concatenate([np.zeros(off, np.uint16), xb]))
        ob = torch.zeros(n + off, dtype=torch.float16, device="cuda:0")
        bufs.append(buf[off:])
        outs.append(ob[off:])
    for call in range(3):
        loopback(channel, bufs[0], bufs[1], outs[0], outs[1], streams)
        check_pair(outs[0], outs[1], x0b, x1b, f"mixed paths n={n} call {call}")


def test_in_place(channel, streams):
    n = 131_072
    x0b, x1b = inputs.workload2(32, call=7)
    x0, x1 = to_dev(x0b), to_dev(x1b)
    loopback(channel, x0, x1, x0, x1, streams)
    check_pair(x0, x1, x0b, x1b, "in place")


def test_too_large_is_refused_and_channel_stays_usable(channel, streams):
    n = hr.HR_DEFAULT_MAX_NUMEL + 1
    x = torch.zeros(n, dtype=torch.float16, device="cuda:0")
    with pytest.raises(hr.HrError) as ei:
        channel.allreduce(0, x, x, streams[0])
    assert ei.value.status == hr.HR_ERR_TOO_LARGE
    x0b, x1b = inputs.workload2(1)
    x0, x1 = to_dev(x0b), to_dev(x1b)
    out0, out1 = torch.empty_like(x0), torch.empty_like(x1)
    loopback(channel, x0, x1, out0, out1, streams)
    check_pair(out0, out1, x0b, x1b, "after refusal")


@pytest.mark.parametrize("first", [0, 1])
def test_skewed_arrival(channel, streams, first):
    """One rank arrives 30 ms after the other; the early one waits."""
    x0b, x1b = inputs.workload2(8, call=3)
    x = [to_dev(x0b), to_dev(x1b)]
    out = [torch.empty_like(x[0]), torch.empty_like(x[1])]
    torch.cuda.synchronize()
    channel.allreduce(first, x[first], out[first], streams[first])
    time.sleep(0.03)
    other = first ^ 1
    channel.allreduce(other, x[other], out[other], streams[other])
    streams[0].synchronize()
    streams[1].synchronize()
    assert channel.status() == hr.HR_OK
    check_pair(out[0], out[1], x0b, x1b, f"skew first={first}")


@pytest.mark.parametrize("algorithm", [hr.HR_ALGO_ONE_SHOT, hr.HR_ALGO_LL], ids=["one-shot", "ll"])
def test_peer_never_arrives_times_out(streams, algorithm):
    ch = hr.Channel(timeout_us=20_000, algorithm=algorithm)
    try:
        x = to_dev(inputs.workload2(4)[0])
        out = torch.full_like(x, 3.0)
        torch.cuda.synchronize()
        t0 = time.time()
        ch.allreduce(0, x, out, streams[0])
        streams[0].synchronize()
        dt = time.time() - t0
        assert ch.status() == hr.HR_ERR_TIMEOUT
        assert dt < 5.0
        # the timed-out kernel left out unwritten
        assert torch.all(out == 3.0)
        # the timeout record: rank 0 waited, rank 1 never published, call 1
        assert ch.timeout_info() == (0, [1], 1)
        # sticky: the next call is refused without a launch
        with pytest.raises(hr.HrError) as ei:
            ch.allreduce(1, x, out, streams[1])
        assert ei.value.status == hr.HR_ERR_TIMEOUT
    finally:
        torch.cuda.synchronize()
        ch.destroy()


@pytest.mark.parametrize("algorithm", [hr.HR_ALGO_ONE_SHOT, hr.HR_ALGO_LL], ids=["one-shot", "ll"])
def test_abort_releases_a_waiting_kernel(streams, algorithm):
    ch = hr.Channel(timeout_us=5_000_000, algorithm=algorithm)
    try:
        x = to_dev(inputs.workload2(4)[0])
        out = torch.full_like(x, 3.0)
        torch.cuda.synchronize()
        t0 = time.time()
        ch.allreduce(0, x, out, streams[0])
        time.sleep(0.05)
        ch.abort()
        streams[0].synchronize()
        dt = time.time() - t0
        assert ch.status() == hr.HR_ERR_ABORTED
        assert dt < 2.5, dt
        assert torch.all(out == 3.0)
    finally:
        torch.cuda.synchronize()
        ch.destroy()


def test_host_acts_as_the_peer(streams):
    """Integrity of both directions of the host link: the kernel's slot writes
    are read back by the CPU bit for bit, and values the CPU writes into the
    peer's slot (then flags) are what the kernel adds."""
    ch = hr.Channel(timeout_us=TIMEOUT_US, algorithm=hr.HR_ALGO_ONE_SHOT)
    try:
        info = ch.info()
        n = 65_536 + 3
        x0b, x1b = specials_mix(n, 41), specials_mix(n, 42)
        x0 = to_dev(x0b)
        out0 = torch.empty_like(x0)
        torch.cuda.synchronize()
        ch.allreduce(0, x0, out0, streams[0])          # call 1 -> parity 1
        stride_bytes = info.slot_stride * 2
        peer_slot = info.host_slots + (2 * 1 + 1) * stride_bytes
        own_slot = info.host_slots + (2 * 1 + 0) * stride_bytes
        ctypes.memmove(peer_slot, x1b.ctypes.data, n * 2)
        for b in range(info.num_blocks):
            info.host_flags[(1 * info.num_blocks + b) * info.flag_stride] = 1
        streams[0].synchronize()
        assert ch.status() == hr.HR_OK
        assert_same_bits(to_host(out0), oracle.add(x0b, x1b), "host peer")
        seen = np.frombuffer(ctypes.string_at(own_slot, n * 2), dtype=np.uint16)
        assert np.array_equal(seen, x0b)
        # workgroups that carried values raised their flag for call 1; the
        # idle ones never touch the flags (active: about one 16-byte unit per
        # lane, at least 16 / W = 8 for two ranks)
        active = min(info.num_blocks, max(16 // 2, -(-(n // 8) // info.block_threads)))
        raised = [info.host_flags[(0 * info.num_blocks + b) * info.flag_stride]
                  for b in range(info.num_blocks)]
        assert raised == [1] * active + [0] * (info.num_blocks - active)
    finally:
        torch.cuda.synchronize()
        ch.destroy()


def ll_field(call):
    """The 16-bit call field of a low-latency word (hr.h): the call number's
    low 15 bits with the top bit set."""
    return (call & 0x7FFF) | 0x8000


def ll_words(bits, call, plane_words):
    """The low-latency slot image of one contribution (hr.h): three planes of
    plane_words 64-bit words; unit u (values v0..v7, the last unit
    zero-padded) is word u of each plane -- v0 v1 v2, v3 v4 v5 and v6 v7 0 in
    bits 0..47 -- with the call field in bits 48..63."""
    n = bits.size
    units = -(-n // 8)
    v = np.zeros(units * 8, np.uint64)
    v[:n] = bits
    v = v.reshape(units, 8)
    sh = lambda x, k: x << np.uint64(k)
    f = sh(np.uint64(ll_field(call)), 48)
    img = np.zeros((3, plane_words), np.uint64)
    img[0, :units] = v[:, 0] | sh(v[:, 1], 16) | sh(v[:, 2], 32) | f
    img[1, :units] = v[:, 3] | sh(v[:, 4], 16) | sh(v[:, 5], 32) | f
    img[2, :units] = v[:, 6] | sh(v[:, 7], 16) | f
    return img, units


@pytest.mark.parametrize("n", [4096, 9, 32_768])
def test_host_acts_as_the_peer_ll(streams, n):
    """The low-latency protocol seen from the host: the CPU writes the peer's
    words for call 1 (values and call number) into the parity-1 slot; the
    kernel adds them, and its own slot holds exactly the word image of its
    contribution."""
    ch = hr.Channel(timeout_us=TIMEOUT_US, algorithm=hr.HR_ALGO_LL)
    try:
        info = ch.info()
        assert ch.algorithm_for(n) == hr.HR_ALGO_LL
        x0b, x1b = specials_mix(n, 45), specials_mix(n, 46)
        x0 = to_dev(x0b)
        out0 = torch.empty_like(x0)
        slot_bytes = info.ll_stride * 8
        plane = info.ll_stride // 3
        peer, _ = ll_words(x1b, 1, plane)
        ctypes.memmove(info.host_ll + (2 * 1 + 1) * slot_bytes, peer.ctypes.data, peer.nbytes)
        torch.cuda.synchronize()
        ch.allreduce(0, x0, out0, streams[0])          # call 1 -> parity 1
        streams[0].synchronize()
        assert ch.status() == hr.HR_OK
        assert_same_bits(to_host(out0), oracle.add(x0b, x1b), "host peer, LL")
        own, units = ll_words(x0b, 1, plane)
        seen = np.frombuffer(ctypes.string_at(info.host_ll + (2 * 1 + 0) * slot_bytes, slot_bytes),
                             dtype=np.uint64).reshape(3, plane)
        assert np.array_equal(seen[:, :units], own[:, :units])
    finally:
        torch.cuda.synchronize()
        ch.destroy()


def test_two_channels_in_one_process(streams):
    chs = [hr.Channel(max_numel=32_768, timeout_us=TIMEOUT_US),
           hr.Channel(max_numel=32_768, num_blocks=16, timeout_us=TIMEOUT_US)]
    try:
        for call in range(6):
            ch = chs[call % 2]
            x0b, x1b = inputs.gaussian(32_768, 1, 30, 0, call), inputs.gaussian(32_768, 1, 30, 1, call)
            x0, x1 = to_dev(x0b), to_dev(x1b)
            out0, out1 = torch.empty_like(x0), torch.empty_like(x1)
            loopback(ch, x0, x1, out0, out1, streams)
            check_pair(out0, out1, x0b, x1b, f"channel {call % 2} call {call}")
    finally:
        torch.cuda.synchronize()
        for ch in chs:
            ch.destroy()


def _capture(ch, rank, xin, out, stream):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for k in range(xin.shape[0]):
            ch.allreduce(rank, xin[k], out[k], stream)
    return g


def _replay_both(graphs, streams):
    torch.cuda.synchronize()
    with torch.cuda.stream(streams[0]):
        graphs[0].replay()
    with torch.cuda.stream(streams[1]):
        graphs[1].replay()
    streams[0].synchronize()
    streams[1].synchronize()


def test_workload5_graph_of_1000_calls(channel, streams):
    """Each rank captures 1000 calls into its own graph; both graphs are
    captured and instantiated before either is launched, then both replay
    concurrently; all 2000 outputs match the oracle."""
    calls = 1000
    xb = inputs.workload5(calls=calls)
    say("exchange: workload 5, graph of 1000 calls N=10240")
    xin = [to_dev(xb[r].reshape(-1)).view(calls, -1) for r in range(2)]
    outs = [torch.empty_like(xin[r]) for r in range(2)]
    # one eager call per rank before capture
    loopback(channel, xin[0][0], xin[1][0], outs[0][0], outs[1][0], streams)
    graphs = [_capture(channel, r, xin[r], outs[r], streams[r]) for r in range(2)]
    outs[0].zero_()
    outs[1].zero_()
    _replay_both(graphs, streams)
    assert channel.status() == hr.HR_OK
    ref = oracle.add(xb[0].reshape(-1), xb[1].reshape(-1))
    g0, g1 = to_host(outs[0]).reshape(-1), to_host(outs[1]).reshape(-1)
    assert_same_bits(g0, ref, "graph rank 0")
    assert_same_bits(g1, ref, "graph rank 1")
    assert np.array_equal(g0, g1)


def test_graph_replays_with_odd_call_count_and_fresh_inputs(channel, streams):
    calls, n = 3, 10_240
    xin = [torch.empty((calls, n), dtype=torch.float16, device="cuda:0") for _ in range(2)]
    outs = [torch.empty_like(xin[r]) for r in range(2)]
    loopback(channel, xin[0][0], xin[1][0], outs[0][0], outs[1][0], streams)
    graphs = [_capture(channel, r, xin[r], outs[r], streams[r]) for r in range(2)]
    for replay in range(4):
        xb = [np.stack([inputs.gaussian(n, 1.0, 40 + replay, r, k) for k in range(calls)])
              for r in range(2)]
        for r in range(2):
            xin[r].copy_(to_dev(xb[r].reshape(-1)).view(calls, n))
        _replay_both(graphs, streams)
        assert channel.status() == hr.HR_OK
        ref = oracle.add(xb[0].reshape(-1), xb[1].reshape(-1))
        assert_same_bits(to_host(outs[0]).reshape(-1), ref, f"replay {replay} rank 0")
        assert_same_bits(to_host(outs[1]).reshape(-1), ref, f"replay {replay} rank 1")
        # eager calls between replays keep the device-side parity consistent
        x0b, x1b = inputs.workload2(1, call=replay)
        x0, x1 = to_dev(x0b), to_dev(x1b)
        o0, o1 = torch.empty_like(x0), torch.empty_like(x1)
        loopback(channel, x0, x1, o0, o1, streams)
        check_pair(o0, o1, x0b, x1b, f"eager after replay {replay}")


def test_algorithm_choice():
    """Which algorithm a call takes, as the library reports it: a function of
    the channel and numel only, whatever each rank's buffers."""
    ch2 = hr.Channel(timeout_us=TIMEOUT_US)
    ch2t = hr.Channel(timeout_us=TIMEOUT_US, algorithm=hr.HR_ALGO_TWO_SHOT)
    ch2l = hr.Channel(timeout_us=TIMEOUT_US, algorithm=hr.HR_ALGO_LL)
    ch4 = hr.Channel(world_size=4, timeout_us=TIMEOUT_US)
    ch4o = hr.Channel(world_size=4, timeout_us=TIMEOUT_US, algorithm=hr.HR_ALGO_ONE_SHOT)
    chs = (ch2, ch2t, ch2l, ch4, ch4o)
    try:
        assert ch2.algorithm_for(1) == hr.HR_ALGO_LL
        assert ch2.algorithm_for(20_480) == hr.HR_ALGO_LL
        assert ch2.algorithm_for(20_481) == hr.HR_ALGO_ONE_SHOT
        assert ch2.algorithm_for(131_072) == hr.HR_ALGO_ONE_SHOT
        assert ch2t.algorithm_for(1) == hr.HR_ALGO_TWO_SHOT
        assert ch2l.algorithm_for(32_768) == hr.HR_ALGO_LL
        assert ch2l.algorithm_for(32_769) == hr.HR_ALGO_ONE_SHOT
        assert ch4.algorithm_for(10_240) == hr.HR_ALGO_ONE_SHOT
        assert ch4.algorithm_for(16_383) == hr.HR_ALGO_ONE_SHOT
        assert ch4.algorithm_for(16_384) == hr.HR_ALGO_TWO_SHOT
        assert ch4.algorithm_for(4096) == hr.HR_ALGO_LL
        assert ch4.algorithm_for(4097) == hr.HR_ALGO_ONE_SHOT
        for W, ll_max, first in ((3, 8192, 98_304), (5, 4096, 10_240), (6, 2560, 6144), (7, 2048, 5120),
                                 (8, 1536, 3072)):
            chw = hr.Channel(world_size=W, timeout_us=TIMEOUT_US)
            try:
                assert chw.algorithm_for(1) == hr.HR_ALGO_LL, W
                assert chw.algorithm_for(ll_max) == hr.HR_ALGO_LL, W
                assert chw.algorithm_for(ll_max + 1) == hr.HR_ALGO_ONE_SHOT, W
                assert chw.algorithm_for(first - 1) == hr.HR_ALGO_ONE_SHOT, W
                assert chw.algorithm_for(first) == hr.HR_ALGO_TWO_SHOT, W
            finally:
                chw.destroy()
        assert ch4o.algorithm_for(4096) == hr.HR_ALGO_ONE_SHOT
        with pytest.raises(hr.HrError) as ei:
            ch2.algorithm_for(hr.HR_DEFAULT_MAX_NUMEL + 1)
        assert ei.value.status == hr.HR_ERR_TOO_LARGE
    finally:
        for ch in chs:
            ch.destroy()


def _hip_runtime():
    """The HIP runtime this process already uses (the library torch loaded),
    found by path so that no second copy is loaded."""
    with open("/proc/self/maps") as f:
        for line in f:
            path = line.split()[-1]
            if "libamdhip64.so" in path and path.startswith("/"):
                lib = ctypes.CDLL(path)
                lib.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
                return lib
    raise RuntimeError("libamdhip64 is not loaded")


def _counters(ch, value=None):
    """Read (or first set) every rank's per-workgroup call counters."""
    info = ch.info()
    n = info.world_size * info.num_blocks
    arr = (ctypes.c_uint64 * n)()
    hip = _hip_runtime()
    torch.cuda.synchronize()
    if value is not None:
        for i in range(n):
            arr[i] = value
        assert hip.hipMemcpy(info.dev_epochs, ctypes.addressof(arr), ctypes.sizeof(arr), 1) == 0
    assert hip.hipMemcpy(ctypes.addressof(arr), info.dev_epochs, ctypes.sizeof(arr), 2) == 0
    torch.cuda.synchronize()
    return list(arr)


def _next_call_number(prev):
    e = prev + 1
    return e + 2 if e % (1 << 32) == 0 else e


@pytest.mark.parametrize("start", [(1 << 31) + 5, (1 << 32) - 3, (1 << 33) - 2])
def test_call_numbers_far_from_zero(streams, start):
    """Long-running channels: with every call counter set to `start` on a
    fresh channel (all flags and low-latency words still zero, as for
    workgroups and units a long-running process has never used), a sequence
    of calls of every algorithm across the 2^31 and 2^32 boundaries gives
    the oracle's bits, and every counter advances by the call-number rule."""
    ch = hr.Channel(max_numel=hr.HR_DEFAULT_MAX_NUMEL, timeout_us=TIMEOUT_US)
    try:
        _counters(ch, start)
        sizes = [131_072, 10_240, 4096, 65_541, 9, 131_072]
        for call, n in enumerate(sizes):
            x0b, x1b = specials_mix(n, seed=700 + call), specials_mix(n, seed=800 + call)
            x0, x1 = to_dev(x0b), to_dev(x1b)
            out0, out1 = torch.empty_like(x0), torch.empty_like(x1)
            say(f"exchange: counters from {start}, call {call}, n={n}, "
                f"algorithm {ch.algorithm_for(n)}")
            loopback(ch, x0, x1, out0, out1, streams)
            check_pair(out0, out1, x0b, x1b, f"start {start} call {call} n={n}")
        want = start
        for _ in sizes:
            want = _next_call_number(want)
        assert _counters(ch) == [want] * (2 * ch.info().num_blocks)
    finally:
        torch.cuda.synchronize()
        ch.destroy()


@pytest.mark.parametrize("link_mbps", [hr.HR_LINK_UNPACED, 1000, 0, hr.HR_LINK_CALIBRATE],
                         ids=["unpaced", "1GBps", "default", "calibrated"])
@pytest.mark.parametrize("algorithm", [hr.HR_ALGO_ONE_SHOT, hr.HR_ALGO_TWO_SHOT], ids=["one-shot", "two-shot"])
def test_publish_pacing(streams, link_mbps, algorithm):
    """Paced or not, the one-shot and the two-shot give the oracle's bits.
    At 1 GB/s the last workgroup of a 256 KiB call starts about half a
    millisecond after the first; the watchdog does not mistake that for a
    missing peer."""
    ch = hr.Channel(timeout_us=TIMEOUT_US, algorithm=algorithm, link_mbps=link_mbps)
    try:
        got = ch.info().link_mbps
        if link_mbps in (hr.HR_LINK_CALIBRATE, 0):
            # measured anew, or once per device for the default; a PCIe 5.0
            # x16 host link moves about 50-60 GB/s each way
            say(f"measured host link ({'anew' if link_mbps else 'default'}): {got} MB/s")
            assert 20_000 <= got <= 80_000
        else:
            assert got == link_mbps
        for call, n in enumerate([131_072, 65_541, 4096]):
            x0b, x1b = specials_mix(n, seed=900 + call), specials_mix(n, seed=950 + call)
            x0, x1 = to_dev(x0b), to_dev(x1b)
            out0, out1 = torch.empty_like(x0), torch.empty_like(x1)
            loopback(ch, x0, x1, out0, out1, streams)
            check_pair(out0, out1, x0b, x1b, f"pacing {link_mbps} call {call} n={n}")
    finally:
        torch.cuda.synchronize()
        ch.destroy()


@pytest.mark.parametrize("algorithm", [hr.HR_ALGO_AUTO, hr.HR_ALGO_TWO_SHOT], ids=["auto", "two-shot"])
def test_prefill_sized_calls(streams, algorithm):
    """Calls far above the 256 KiB decode cap (a channel made for them):
    several 16-byte units per lane and long paced slices, ragged sizes,
    every value checked against the oracle."""
    n_max = 1 << 21                                    # 4 MiB per rank
    ch = hr.Channel(max_numel=n_max, timeout_us=TIMEOUT_US, algorithm=algorithm)
    try:
        for call, n in enumerate([n_max, (1 << 20) + 3, 333_333, n_max - 7]):
            x0b, x1b = inputs.gaussian(n, 0.5, 80, 0, call), inputs.gaussian(n, 0.5, 80, 1, call)
            x0, x1 = to_dev(x0b), to_dev(x1b)
            out0, out1 = torch.empty_like(x0), torch.empty_like(x1)
            say(f"exchange: prefill-sized call {call}, n={n}, algorithm {ch.algorithm_for(n)}")
            loopback(ch, x0, x1, out0, out1, streams)
            check_pair(out0, out1, x0b, x1b, f"prefill call {call} n={n}")
    finally:
        torch.cuda.synchronize()
        ch.destroy()


@pytest.mark.parametrize("algorithm", [hr.HR_ALGO_AUTO, hr.HR_ALGO_TWO_SHOT], ids=["auto", "two-shot"])
def test_channel_at_the_size_limit(streams, algorithm):
    """One call of HR_MAX_NUMEL_LIMIT values (1 GiB per rank) on a channel of
    that size, where slot offsets reach 2^30 bytes: every rank's output is
    checked against the oracle on a million seeded sample positions and on
    the first and last 4096 values."""
    n = hr.HR_MAX_NUMEL_LIMIT
    rng = np.random.default_rng(2029)
    x0b = rng.integers(0, 1 << 16, n, dtype=np.uint16)   # every pattern class, NaN and inf included
    x1b = rng.integers(0, 1 << 16, n, dtype=np.uint16)
    say(f"exchange: channel at the size limit, n={n}, algorithm {algorithm}")
    ch = hr.Channel(max_numel=n, timeout_us=TIMEOUT_US, algorithm=algorithm)
    try:
        x0, x1 = to_dev(x0b), to_dev(x1b)
        out0, out1 = torch.empty_like(x0), torch.empty_like(x1)
        loopback(ch, x0, x1, out0, out1, streams)
        idx = np.unique(np.concatenate([rng.integers(0, n, 1_000_000), np.arange(4096),
                                        np.arange(n - 4096, n)]))
        ref = oracle.add(x0b[idx], x1b[idx])
        for r, out in enumerate((out0, out1)):
            got = to_host(out)[idx]
            assert_same_bits(got, ref, f"size-limit call rank {r}")
        del x0, x1, out0, out1
    finally:
        torch.cuda.synchronize()
        ch.destroy()


# ---------------------------------------------------------------- stale values
#
# Slots are double buffered by call parity (the 1Cat-vLLM page, "Purpose"):
# a flag or a low-latency word left by an earlier call must never release a
# waiter.  The host plays rank 1 and leaves values of earlier calls where a
# waiter of call e looks; the kernel of rank 0 must not take them, so it ends
# at its own short watchdog with `out` unwritten.  The same setup with the
# current call number then completes, on a fresh channel.

STALE_START = 1000          # counters before the call: the call number is 1001


def _peer_flags(info, value):
    for b in range(info.num_blocks):
        info.host_flags[(1 * info.num_blocks + b) * info.flag_stride] = value


def _peer_ll_words(info, bits, call, tag):
    slot_bytes = info.ll_stride * 8
    img, _ = ll_words(bits, tag, info.ll_stride // 3)
    ctypes.memmove(info.host_ll + (2 * (call & 1) + 1) * slot_bytes, img.ctypes.data, img.nbytes)


@pytest.mark.parametrize("stale", [1, 2], ids=["e-1", "e-2"])
@pytest.mark.parametrize("algorithm", [hr.HR_ALGO_ONE_SHOT, hr.HR_ALGO_LL], ids=["one-shot", "ll"])
def test_stale_peer_values_do_not_release(streams, algorithm, stale):
    n = 4096
    x0b, x1b = specials_mix(n, 51), specials_mix(n, 52)
    x0 = to_dev(x0b)
    e = _next_call_number(STALE_START)
    # the peer's values are in place, but marked with call e - stale
    ch = hr.Channel(timeout_us=20_000, algorithm=algorithm)
    try:
        info = ch.info()
        _counters(ch, STALE_START)
        out = torch.full_like(x0, 3.0)
        if algorithm == hr.HR_ALGO_LL:
            _peer_ll_words(info, x1b, e, e - stale)
        else:
            peer_slot = info.host_slots + (2 * (e & 1) + 1) * info.slot_stride * 2
            ctypes.memmove(peer_slot, x1b.ctypes.data, n * 2)
            _peer_flags(info, e - stale)
        torch.cuda.synchronize()
        say(f"stale peer values: algorithm {algorithm}, call {e}, peer marked {e - stale}")
        ch.allreduce(0, x0, out, streams[0])
        streams[0].synchronize()
        assert ch.status() == hr.HR_ERR_TIMEOUT
        assert torch.all(out == 3.0), "a stale value released the waiter"
        assert ch.timeout_info() == (0, [1], e & ((1 << 48) - 1))
    finally:
        torch.cuda.synchronize()
        ch.destroy()
    # the current call number releases the same wait
    ch = hr.Channel(timeout_us=TIMEOUT_US, algorithm=algorithm)
    try:
        info = ch.info()
        _counters(ch, STALE_START)
        out = torch.full_like(x0, 3.0)
        if algorithm == hr.HR_ALGO_LL:
            _peer_ll_words(info, x1b, e, e)
        else:
            peer_slot = info.host_slots + (2 * (e & 1) + 1) * info.slot_stride * 2
            ctypes.memmove(peer_slot, x1b.ctypes.data, n * 2)
            _peer_flags(info, e)
        torch.cuda.synchronize()
        ch.allreduce(0, x0, out, streams[0])
        streams[0].synchronize()
        assert ch.status() == hr.HR_OK
        assert_same_bits(to_host(out), oracle.add(x0b, x1b), "current call number")
    finally:
        torch.cuda.synchronize()
        ch.destroy()


def _ll_slot(info, parity, rank):
    slot_bytes = info.ll_stride * 8
    raw = ctypes.string_at(info.host_ll + (info.world_size * parity + rank) * slot_bytes, slot_bytes)
    return np.frombuffer(raw, dtype=np.uint64).reshape(3, info.ll_stride // 3).copy()


def _fields(words):
    return (words >> np.uint64(48)).astype(np.int64)


def _plant_ll(info, parity, rank, tag):
    """Every word of slot[parity][rank] set to three values 1.0 (0x3c00) and
    the call field of call `tag`, as a call of that number would leave them."""
    img = np.full((3, info.ll_stride // 3),
                  0x3C00 | 0x3C00 << 16 | 0x3C00 << 32 | ll_field(tag) << 48, np.uint64)
    slot_bytes = info.ll_stride * 8
    ctypes.memmove(info.host_ll + (info.world_size * parity + rank) * slot_bytes, img.ctypes.data,
                   img.nbytes)


@pytest.mark.parametrize("first", [hr.HR_ALGO_LL, hr.HR_ALGO_ONE_SHOT], ids=["ll", "one-shot"])
def test_ll_clearing_removes_words_of_calls_2_32_earlier(streams, first):
    """Low-latency words carry a 15-bit call field.  Words planted in both
    ranks' even-parity slots with the field of call c + 2 stand for words
    left by call c + 2 - 2^15 that no later call overwrote.  Call
    c = 2^31 + 2 is a clearing point of the even parity (its low 14 bits are
    2): both ranks zero their slot there except the units the call itself
    writes.  So afterwards rank 0 alone at call c + 2 finds nothing to take
    and ends at its watchdog with `out` unwritten.  At a call that is not a
    clearing point (c + 2) the planted words stay, which shows the planting
    is what a reader would see."""
    c = (1 << 31) + 2
    ch = hr.Channel(timeout_us=TIMEOUT_US, algorithm=first)
    small = 8                                   # one 8-value unit
    try:
        info = ch.info()
        _counters(ch, c - 1)
        for r in range(2):
            _plant_ll(info, 0, r, c + 2)
        # calls c and c + 1 of both ranks, `small` values each
        for call in range(2):
            x0b, x1b = specials_mix(small, 60 + call), specials_mix(small, 70 + call)
            x0, x1 = to_dev(x0b), to_dev(x1b)
            out0, out1 = torch.empty_like(x0), torch.empty_like(x1)
            say(f"ll clearing: call {c + call}, first algorithm {first}")
            loopback(ch, x0, x1, out0, out1, streams)
            check_pair(out0, out1, x0b, x1b, f"call {c + call}")
        keep = 1 if first == hr.HR_ALGO_LL else 0
        for r in range(2):
            slot = _ll_slot(info, 0, r)
            assert not slot[:, keep:].any(), f"rank {r}: planted words survived the clearing call"
            if keep:
                assert (_fields(slot[:, 0]) == ll_field(c)).all()
    finally:
        torch.cuda.synchronize()
        ch.destroy()

    # rank 0 alone at call c + 2 on a channel in the same state
    ch = hr.Channel(timeout_us=20_000, algorithm=hr.HR_ALGO_LL)
    try:
        info = ch.info()
        _counters(ch, c - 1)
        for r in range(2):
            _plant_ll(info, 0, r, c + 2)
        for call in range(2):
            x0b, x1b = specials_mix(small, 60 + call), specials_mix(small, 70 + call)
            x0, x1 = to_dev(x0b), to_dev(x1b)
            loopback(ch, x0, x1, torch.empty_like(x0), torch.empty_like(x1), streams)
        x = to_dev(specials_mix(4096, 80))
        out = torch.full_like(x, 3.0)
        torch.cuda.synchronize()
        say(f"ll clearing: rank 0 alone at call {c + 2}")
        ch.allreduce(0, x, out, streams[0])
        streams[0].synchronize()
        assert ch.status() == hr.HR_ERR_TIMEOUT
        assert torch.all(out == 3.0), "a word of an earlier call released the reader"
    finally:
        torch.cuda.synchronize()
        ch.destroy()

    # control: no clearing at c + 2 (even, not a clearing point) -- the
    # planted words that this call does not write stay in place
    ch = hr.Channel(timeout_us=TIMEOUT_US, algorithm=hr.HR_ALGO_LL)
    try:
        info = ch.info()
        _counters(ch, c + 1)
        for r in range(2):
            _plant_ll(info, 0, r, c + 4)
        x0b, x1b = specials_mix(small, 90), specials_mix(small, 91)
        x0, x1 = to_dev(x0b), to_dev(x1b)
        out0, out1 = torch.empty_like(x0), torch.empty_like(x1)
        loopback(ch, x0, x1, out0, out1, streams)
        check_pair(out0, out1, x0b, x1b, f"call {c + 2}")
        for r in range(2):
            slot = _ll_slot(info, 0, r)
            assert (_fields(slot[:, 1:]) == ll_field(c + 4)).all()
            assert (_fields(slot[:, 0]) == ll_field(c + 2)).all()
    finally:
        torch.cuda.synchronize()
        ch.destroy()


def test_loopback_streams_are_not_non_blocking(streams):
    """hr.h states that a loopback stream is ordered with the null stream
    (HIP creates a compute-unit-mask stream without hipStreamNonBlocking);
    the runtime's own flags say so."""
    hip = _hip_runtime()
    hip.hipStreamGetFlags.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint)]
    for s in streams:
        flags = ctypes.c_uint(0xFFFF)
        assert hip.hipStreamGetFlags(ctypes.c_void_p(s.cuda_stream), ctypes.byref(flags)) == 0
        say(f"loopback stream flags: {flags.value:#x}")
        assert flags.value & 1 == 0       # hipStreamNonBlocking is 0x1


def test_default_rate_is_measured_once_per_device():
    """Channels created with link_mbps = 0 all pace by one rate, measured
    on the device by the first of them and kept by the library."""
    rates = []
    for _ in range(3):
        ch = hr.Channel(timeout_us=TIMEOUT_US)
        try:
            rates.append(ch.info().link_mbps)
        finally:
            ch.destroy()
    say(f"default pacing rates: {rates}")
    assert len(set(rates)) == 1 and 20_000 <= rates[0] <= 80_000


def test_ll_graph_across_the_call_field_wrap(streams):
    """Low-latency words carry the call number's low 15 bits.  With every
    counter set 300 calls below 2^15, three replays of a 1000-call graph per
    rank run real low-latency traffic through the field's wrap (call 2^15
    has the field of call 0) and through the clearing calls 2^15 + 2 and
    2^15 + 3, with fresh inputs before every replay; every output is compared
    with the oracle and the counters end 3000 calls on."""
    calls, n, replays = 1000, 10_240, 3
    start = (1 << 15) - 300
    ch = hr.Channel(timeout_us=TIMEOUT_US, algorithm=hr.HR_ALGO_LL)
    try:
        assert ch.algorithm_for(n) == hr.HR_ALGO_LL
        xin = [torch.zeros((calls, n), dtype=torch.float16, device="cuda:0") for _ in range(2)]
        outs = [torch.empty_like(x) for x in xin]
        loopback(ch, xin[0][0], xin[1][0], outs[0][0], outs[1][0], streams)   # warm-up
        _counters(ch, start)
        graphs = [_capture(ch, r, xin[r], outs[r], streams[r]) for r in range(2)]
        rng = np.random.default_rng(7)
        for rep in range(replays):
            xb = [rng.standard_normal((calls, n), dtype=np.float32).astype(np.float16).view(np.uint16)
                  for _ in range(2)]
            for r in range(2):
                xin[r].copy_(to_dev(xb[r].reshape(-1)).view(calls, n))
            torch.cuda.synchronize()
            say(f"LL graph across the field wrap: replay {rep}, calls {start + 1 + rep * calls}..")
            _replay_both(graphs, streams)
            assert ch.status() == hr.HR_OK
            ref = oracle.add(xb[0].reshape(-1), xb[1].reshape(-1))
            for r in range(2):
                assert_same_bits(to_host(outs[r]).reshape(-1), ref, f"replay {rep} rank {r}")
        assert set(_counters(ch)) == {start + replays * calls}
        del graphs
    finally:
        torch.cuda.synchronize()
        ch.destroy()
