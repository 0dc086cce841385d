"""The Python binding refuses, before any call into the library, the tensors
the C entry points cannot take: another element type, mixed element types,
host tensors, non-contiguous views and mismatched sizes.  Each refusal
raises in the binding; nothing is launched, and the channel stays healthy
(a correct call after them still matches the oracle)."""
import numpy as np
import pytest
import torch

import oracle
from message_fp16_all_amd import hr
from _gpu import assert_same_bits, needs_gpu, specials_mix, to_dev, to_host

pytestmark = [pytest.mark.gpu, needs_gpu]


def test_allreduce_refusals_then_a_correct_call():
    ch = hr.Channel(timeout_us=2_000_000)
    streams = hr.LoopbackStreams(0)
    try:
        x = torch.zeros(4096, dtype=torch.float16, device="cuda:0")
        y = torch.empty_like(x)
        s = streams[0]
        with pytest.raises(TypeError):
            ch.allreduce(0, x.float(), y, s)                  # float32 input
        with pytest.raises(TypeError):
            ch.allreduce(0, x, y.bfloat16(), s)               # float16 in, bfloat16 out
        with pytest.raises(TypeError):
            ch.allreduce(0, x.bfloat16(), y, s)               # bfloat16 in, float16 out
        with pytest.raises(TypeError):
            ch.allreduce(0, x, y.cpu(), s)                    # host output
        with pytest.raises(ValueError):
            ch.allreduce(0, x[::2], y[:2048], s)              # non-contiguous input
        with pytest.raises(ValueError):
            ch.allreduce(0, x, y[:100], s)                    # sizes differ
        assert ch.status() == hr.HR_OK

        n = 5000
        xb = [specials_mix(n, 4400 + r) for r in range(2)]
        xs = [to_dev(b) for b in xb]
        outs = [torch.full_like(t, 3.0) for t in xs]
        torch.cuda.synchronize()
        for r in range(2):
            ch.allreduce(r, xs[r], outs[r], streams[r])
        for st in streams:
            st.synchronize()
        assert ch.status() == hr.HR_OK
        ref = oracle.fold(xb)
        for r in range(2):
            assert_same_bits(to_host(outs[r]), ref, f"rank {r} after the refusals")
    finally:
        torch.cuda.synchronize()
        ch.destroy()
        streams.destroy()


def test_reduce_and_group_refusals():
    ch = hr.Channel(timeout_us=2_000_000)
    try:
        a = torch.zeros(1024, dtype=torch.float16, device="cuda:0")
        b = torch.zeros_like(a)
        out = torch.empty_like(a)
        with pytest.raises(TypeError):
            hr.reduce([a, b.float()], out)                    # one contribution float32
        with pytest.raises(TypeError):
            hr.reduce([a, b], out.bfloat16())                 # float16 inputs, bfloat16 out
        with pytest.raises(ValueError):
            hr.reduce([a, b[:512]], out)                      # sizes differ
        with pytest.raises(ValueError):
            ch.allreduce_group([a], [out])                    # one rank of two
        with pytest.raises(TypeError):
            ch.allreduce_group([a, b.bfloat16()], [out, torch.empty_like(b)])
        assert ch.status() == hr.HR_OK

        xb = [specials_mix(1024, 4500 + g) for g in range(3)]
        ts = [to_dev(x) for x in xb]
        hr.reduce(ts, out)
        torch.cuda.synchronize()
        assert_same_bits(to_host(out), oracle.fold(xb), "reduce after the refusals")
    finally:
        torch.cuda.synchronize()
        ch.destroy()
