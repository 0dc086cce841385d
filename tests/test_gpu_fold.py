"""GPU parity of hr_reduce_f16 (G contributions in HBM) against the oracle.

Every case compares every output value bit for bit (NaN by class) with the
CPU oracle's left fold on the same seeded inputs, through the C ABI.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from message_fp16_all_amd import hr, inputs
from _gpu import assert_same_bits, needs_gpu, specials_mix, to_dev, to_host

pytestmark = [pytest.mark.gpu, needs_gpu]


def run_fold(xs_bits, out=None, stream=None):
    ts = [to_dev(x) for x in xs_bits]
    if out is None:
        out = torch.empty_like(ts[0])
    hr.reduce(ts, out, stream)
    torch.cuda.synchronize()
    return to_host(out)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_workload1_two_ranks_with_specials():
    xs, _ = inputs.workload1()
    say("fold: workload 1, G=2 N=4096")
    got = run_fold(xs)
    assert_same_bits(got, oracle.fold(xs), "workload 1")
    # second library check: torch's own fp16 add on the device
    t = (to_dev(xs[0]) + to_dev(xs[1]))
    assert_same_bits(got, to_host(t), "torch fp16 add")


def test_edge_table_every_ordered_pair():
    xs = inputs.edge_pairs()
    say("fold: edge table 289 pairs")
    got = run_fold(xs)
    assert_same_bits(got, oracle.fold(xs), "edge table")


def test_workload3_eight_ranks_decode_workspace():
    xs = inputs.workload3()
    say("fold: workload 3, G=8 N=393216")
    got = run_fold(xs)
    assert_same_bits(got, oracle.fold(xs), "workload 3")


def test_workload4_eight_ranks_prefill_chunk_full():
    xs = inputs.workload4()
    say("fold: workload 4, G=8 N=16777216")
    got = run_fold(xs)
    ref, _ = oracle.fold(xs, threads=8)
    assert_same_bits(got, ref, "workload 4")


@pytest.mark.parametrize("G", [1, 2, 3, 5, 8, 13, 16])
@pytest.mark.parametrize("n", [1, 7, 8, 9, 255, 2049, 16 * 2048 + 3, 100_003])
def test_ragged_sizes_and_group_sizes(G, n):
    xs = [specials_mix(n, seed=1000 * G + r + n) for r in range(G)]
    got = run_fold(xs)
    assert_same_bits(got, oracle.fold(xs), f"G={G} n={n}")


def test_grid_stride_path_beyond_the_grid_cap():
    # G=16 uses one 16-byte unit per lane per tile; 9M values need more tiles
    # than the grid holds, so each workgroup loops.
    n = 9_000_001
    xs = inputs.contributions(16, n, 1.0, workload=90)
    say("fold: G=16 N=9000001 (grid-stride)")
    got = run_fold(xs)
    ref, _ = oracle.fold(xs, threads=8)
    assert_same_bits(got, ref, "grid stride")


@pytest.mark.parametrize("offset", [1, 3, 4, 7])
def test_unaligned_pointers_take_the_scalar_path(offset):
    G, n = 3, 5000
    xs = [specials_mix(n, seed=77 + r) for r in range(G)]
    bufs = [to_dev(np.concatenate([np.zeros(offset, np.uint16), x])) for x in xs]
    views = [b[offset:] for b in bufs]
    out_buf = torch.zeros(n + offset, dtype=torch.float16, device="cuda:0")
    out = out_buf[offset:]
    hr.reduce(views, out)
    torch.cuda.synchronize()
    assert_same_bits(to_host(out), oracle.fold(xs), f"offset {offset}")
    # values before the view are untouched
    assert np.all(to_host(out_buf[:offset]) == 0)


@pytest.mark.parametrize("which", [0, 2])
def test_in_place_output_aliases_an_input(which):
    G, n = 3, 70_001
    xs = [specials_mix(n, seed=500 + r) for r in range(G)]
    ts = [to_dev(x) for x in xs]
    hr.reduce(ts, ts[which])
    torch.cuda.synchronize()
    assert_same_bits(to_host(ts[which]), oracle.fold(xs), "in place")


def test_empty_input_is_a_no_op():
    a = torch.ones(8, dtype=torch.float16, device="cuda:0")
    out = torch.full((8,), 7.0, dtype=torch.float16, device="cuda:0")
    assert hr.hr_reduce_f16([a.data_ptr(), a.data_ptr()], 2, out.data_ptr(), 0,
                            torch.cuda.current_stream().cuda_stream) == hr.HR_OK
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_partial_overlap_rejected_on_device_buffers():
    buf = torch.zeros(1024, dtype=torch.float16, device="cuda:0")
    st = hr.hr_reduce_f16([buf.data_ptr(), buf[512:].data_ptr()], 2, buf[8:].data_ptr(), 256,
                          torch.cuda.current_stream().cuda_stream)
    assert st == hr.HR_ERR_INVALID_ARG


def test_runs_on_the_given_stream_after_earlier_work():
    """Work queued earlier on the caller's non-blocking stream is seen."""
    n = 1 << 20
    s = torch.cuda.Stream()
    xs = inputs.contributions(4, n, 1.0, workload=91)
    ts = [to_dev(x) for x in xs]
    out = torch.empty_like(ts[0])
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        # the last contribution is produced on s just before the reduce
        ts[3].mul_(-1.0)
        hr.reduce(ts, out, s)
    s.synchronize()
    flipped = xs[3] ^ np.uint16(0x8000)
    assert_same_bits(to_host(out), oracle.fold(xs[:3] + [flipped]), "stream order")


def test_graph_capture_and_replay_with_new_inputs():
    n, G = 300_000, 8
    ts = [torch.empty(n, dtype=torch.float16, device="cuda:0") for _ in range(G)]
    out = torch.empty(n, dtype=torch.float16, device="cuda:0")
    s = torch.cuda.Stream()
    first = inputs.contributions(G, n, 0.1, workload=92, call=0)
    for t, x in zip(ts, first):
        t.copy_(to_dev(x))
    torch.cuda.synchronize()
    # eager once before capture
    hr.reduce(ts, out, s)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        hr.reduce(ts, out, s)
    for call in range(1, 4):
        xs = inputs.contributions(G, n, 0.1, workload=92, call=call)
        for t, x in zip(ts, xs):
            t.copy_(to_dev(x))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same_bits(to_host(out), oracle.fold(xs), f"replay {call}")


@pytest.mark.parametrize("G,n", [(8, 16_777_216), (8, 100_003), (8, 9), (4, 70_001), (16, 300_007)])
def test_contributions_in_the_workspace_layout(G, n):
    """Inputs placed hr_workspace_stride apart in one buffer (the layout the
    eight-rank fold streams fastest from) fold to the same bits."""
    xs = inputs.contributions(G, n, 1.0, workload=93) if n > 1000 else [specials_mix(n, 9 + r) for r in range(G)]
    buf, views = hr.workspace(G, n)
    for v, x in zip(views, xs):
        v.copy_(to_dev(x))
    out = torch.empty(n, dtype=torch.float16, device="cuda:0")
    say(f"fold: workspace layout G={G} n={n}")
    hr.reduce(views, out)
    torch.cuda.synchronize()
    ref = oracle.fold(xs, threads=8)[0] if n > 1_000_000 else oracle.fold(xs)
    assert_same_bits(to_host(out), ref, f"workspace G={G} n={n}")
    # in place, onto the first contribution
    hr.reduce(views, views[0])
    torch.cuda.synchronize()
    assert_same_bits(to_host(views[0]), ref, f"workspace in place G={G} n={n}")


def test_binding_takes_torchs_current_stream():
    """With no stream given, the binding enqueues on torch's current stream,
    also inside a stream context."""
    t = torch.zeros(8, dtype=torch.float16, device="cuda:0")
    assert hr._stream_handle(None, t) == torch.cuda.current_stream().cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert hr._stream_handle(None, t) == s.cuda_stream
        assert hr._stream_handle(None) == s.cuda_stream
