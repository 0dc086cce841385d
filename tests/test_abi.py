"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments synchronously, before any HIP call or launch.

No test here computes anything on a device; on a host without a GPU the
calls that get past argument validation must fail cleanly with HR_ERR_HIP.
"""
import ctypes
import os
import re
import subprocess

import pytest

from message_fp16_all_amd import hr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hr.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"HR_API\s+[\w\s\*]+?\b(hr_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_symbols() == sorted(hr.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = hr.load()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", hr.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(declared_symbols()) <= exported
    # nothing else leaks out of the library's C ABI
    assert {s for s in exported if s.startswith("hr_")} == set(declared_symbols())


def test_library_does_not_link_the_oracle():
    out = subprocess.run(["readelf", "-d", hr.LIB_PATH], check=True, capture_output=True,
                         text=True).stdout
    assert "oracle" not in out
    needed = re.findall(r"\(NEEDED\).*\[(.+)\]", out)
    assert any(n.startswith("libamdhip64") for n in needed)


def test_product_code_never_references_the_oracle():
    pkg = os.path.join(ROOT, "message_fp16_all_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, re.M), f
                assert "hr_oracle" not in text and "hro_" not in text, f


def test_status_strings():
    assert hr.hr_status_str(hr.HR_OK) == "HR_OK"
    assert hr.hr_status_str(hr.HR_ERR_TIMEOUT) == "HR_ERR_TIMEOUT"
    assert hr.hr_status_str(hr.HR_ERR_ABORTED) == "HR_ERR_ABORTED"
    assert hr.hr_status_str(99) == "HR_ERR_UNKNOWN"


FAKE = 0x7F0000000000   # never dereferenced: every case below fails validation


def test_reduce_validation_before_any_device_call():
    f = hr.hr_reduce_f16
    assert f([FAKE, FAKE + 4096], 0, FAKE + 8192, 16, 0) == hr.HR_ERR_INVALID_ARG
    assert f([FAKE] * 17, 17, FAKE + 8192, 16, 0) == hr.HR_ERR_INVALID_ARG
    assert f([FAKE, FAKE + 4096], 2, FAKE + 8192, 0, 0) == hr.HR_OK          # empty: no-op
    assert f([FAKE, 0], 2, FAKE + 8192, 16, 0) == hr.HR_ERR_INVALID_ARG       # null input
    assert f([FAKE, FAKE + 4096], 2, 0, 16, 0) == hr.HR_ERR_INVALID_ARG       # null out
    assert f([FAKE, FAKE + 4097], 2, FAKE + 8192, 16, 0) == hr.HR_ERR_ALIGNMENT
    assert f([FAKE, FAKE + 4096], 2, FAKE + 8193, 16, 0) == hr.HR_ERR_ALIGNMENT
    # out overlapping an input without being equal to it
    assert f([FAKE, FAKE + 4096], 2, FAKE + 16, 16, 0) == hr.HR_ERR_INVALID_ARG
    st = hr.load().hr_reduce_f16(None, 2, FAKE, 16, None)
    assert st == hr.HR_ERR_INVALID_ARG


def test_channel_validation_before_any_device_call():
    lib = hr.load()
    h = ctypes.c_void_p()
    assert lib.hr_create_channel(None, ctypes.byref(h)) == hr.HR_ERR_INVALID_ARG
    for ws in (0, 1, 9, 16):
        cfg = hr.hr_channel_config(0, ws, 0, 0, 0)
        assert lib.hr_create_channel(ctypes.byref(cfg), ctypes.byref(h)) == hr.HR_ERR_UNSUPPORTED
    cfg = hr.hr_channel_config(-1, 2, 0, 0, 0)
    assert lib.hr_create_channel(ctypes.byref(cfg), ctypes.byref(h)) == hr.HR_ERR_INVALID_ARG
    cfg = hr.hr_channel_config(0, 2, hr.HR_MAX_NUMEL_LIMIT + 1, 0, 0)
    assert lib.hr_create_channel(ctypes.byref(cfg), ctypes.byref(h)) == hr.HR_ERR_INVALID_ARG
    for algo in (-1, 4):
        cfg = hr.hr_channel_config(0, 2, 0, 0, 0, algo)
        assert lib.hr_create_channel(ctypes.byref(cfg), ctypes.byref(h)) == hr.HR_ERR_INVALID_ARG
    cfg = hr.hr_channel_config(0, 2, 0, -4, 0)
    assert lib.hr_create_channel(ctypes.byref(cfg), ctypes.byref(h)) == hr.HR_ERR_INVALID_ARG
    for rate in (1, hr.HR_MIN_LINK_MBPS - 1):
        cfg = hr.hr_channel_config(0, 2, 0, 0, 0, 0, rate)
        assert lib.hr_create_channel(ctypes.byref(cfg), ctypes.byref(h)) == hr.HR_ERR_INVALID_ARG
    assert hr.hr_allreduce_f16(None, 0, FAKE, FAKE, 16, 0) == hr.HR_ERR_INVALID_ARG
    assert hr.hr_allreduce_group_f16(None, [FAKE, FAKE], [FAKE, FAKE], 16, 0) == hr.HR_ERR_INVALID_ARG
    assert hr.hr_allreduce_group_bf16(None, [FAKE, FAKE], [FAKE, FAKE], 16, 0) == hr.HR_ERR_INVALID_ARG
    assert hr.hr_exchange_algorithm.__doc__
    assert lib.hr_exchange_algorithm(None, 16, None) == hr.HR_ERR_INVALID_ARG
    assert hr.hr_channel_status(None) == hr.HR_ERR_INVALID_ARG
    assert hr.hr_channel_abort(None) == hr.HR_ERR_INVALID_ARG
    assert lib.hr_channel_get_info(None, None) == hr.HR_ERR_INVALID_ARG
    r, m, c = ctypes.c_int(), ctypes.c_uint32(), ctypes.c_uint64()
    assert lib.hr_channel_timeout_info(None, ctypes.byref(r), ctypes.byref(m),
                                       ctypes.byref(c)) == hr.HR_ERR_INVALID_ARG
    assert hr.hr_destroy(None) == hr.HR_OK
    assert lib.hr_loopback_stream_create(-1, ctypes.byref(h)) == hr.HR_ERR_INVALID_ARG
    assert lib.hr_loopback_stream_create(0, None) == hr.HR_ERR_INVALID_ARG
    assert hr.hr_loopback_stream_destroy(None) == hr.HR_OK


def test_calls_past_validation_fail_cleanly_without_a_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert hr.hr_reduce_f16([FAKE, FAKE + 4096], 2, FAKE + 8192, 16, 0) == hr.HR_ERR_HIP
    with pytest.raises(hr.HrError) as ei:
        hr.hr_create_channel()
    assert ei.value.status in (hr.HR_ERR_HIP, hr.HR_ERR_INVALID_ARG)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(hr, "_lib", None)
    monkeypatch.setattr(hr, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        hr.load()


def test_noalloc_group_validation_before_any_device_call():
    f = hr.hr_allreduce_group_noalloc_f16
    two = [FAKE, FAKE + 65536]
    outs = [FAKE + 2 * 65536, FAKE + 3 * 65536]
    for ws in (0, 1, 9):
        assert f(two, outs, ws, 16, None, 0) == hr.HR_ERR_UNSUPPORTED
    assert f(two, outs, 2, 0, None, 0) == hr.HR_OK                              # empty: no-op
    assert f(two, outs, 2, hr.HR_NOALLOC_MAX_NUMEL + 1, None, 0) == hr.HR_ERR_TOO_LARGE
    assert f([FAKE, 0], outs, 2, 16, None, 0) == hr.HR_ERR_INVALID_ARG          # null input
    assert f(two, [outs[0], FAKE + 1], 2, 16, None, 0) == hr.HR_ERR_ALIGNMENT
    assert f(two, outs, 2, 16, FAKE + 2, 0) == hr.HR_ERR_ALIGNMENT              # status word
    assert f(two, [outs[0], outs[0] + 8], 2, 16, None, 0) == hr.HR_ERR_INVALID_ARG  # outputs overlap
    assert f(two, [two[1], outs[1]], 2, 16, None, 0) == hr.HR_ERR_INVALID_ARG   # out 0 is rank 1's input
    lib = hr.load()
    assert lib.hr_allreduce_group_noalloc_f16(None, None, 2, 16, None, None) == hr.HR_ERR_INVALID_ARG
