"""Admission policy (CPU only): which reductions take the host path, and the
named reason for every decline.

The default policy is the 1Cat-vLLM page's: FP16 payloads of two-rank groups
without peer access, up to 256 KiB, behind an on/off switch ("Purpose",
"Path coverage").  The decode-sized bound follows the SGLang page
("Modifications"): rows = max batch x tokens per request, times hidden.
"""
import pytest

from message_fp16_all_amd import hr

F16, BF16, OTHER = hr.HR_DTYPE_F16, hr.HR_DTYPE_BF16, hr.HR_DTYPE_OTHER


def admit(dtype=F16, world=2, peer=False, numel=4096, policy=None):
    return hr.hr_admit(policy, dtype, world, peer, numel)


def test_default_policy_admits_the_pages_case():
    assert admit() == hr.HR_ROUTE_HOST
    assert admit(numel=131_072) == hr.HR_ROUTE_HOST           # exactly 256 KiB
    assert admit(numel=0) == hr.HR_ROUTE_HOST


def test_default_policy_declines_everything_else_by_name():
    assert admit(numel=131_073) == hr.HR_DECLINE_TOO_LARGE
    assert admit(dtype=BF16) == hr.HR_DECLINE_DTYPE
    assert admit(dtype=OTHER) == hr.HR_DECLINE_DTYPE
    assert admit(world=4) == hr.HR_DECLINE_WORLD_SIZE
    assert admit(world=1) == hr.HR_DECLINE_WORLD_SIZE
    assert admit(peer=True) == hr.HR_DECLINE_PEER_ACCESS


def test_switch_off_declines_first():
    off = hr.hr_admit_policy(0, 0, 1, 8)
    assert admit(policy=off) == hr.HR_DECLINE_DISABLED
    assert admit(policy=off, dtype=OTHER, world=9, peer=True, numel=1 << 30) == hr.HR_DECLINE_DISABLED


def test_decline_order_names_the_first_failing_condition():
    # dtype before world size before peer access before size
    assert admit(dtype=OTHER, world=9, peer=True, numel=1 << 30) == hr.HR_DECLINE_DTYPE
    assert admit(world=9, peer=True, numel=1 << 30) == hr.HR_DECLINE_WORLD_SIZE
    assert admit(peer=True, numel=1 << 30) == hr.HR_DECLINE_PEER_ACCESS


def test_widened_policy():
    pol = hr.hr_admit_policy(1, 1 << 20, 1, 8)
    assert admit(policy=pol, dtype=BF16, world=8, numel=1 << 19) == hr.HR_ROUTE_HOST
    assert admit(policy=pol, world=8, numel=(1 << 19) + 1) == hr.HR_DECLINE_TOO_LARGE
    assert admit(policy=pol, world=9) == hr.HR_DECLINE_WORLD_SIZE
    too_wide = hr.hr_admit_policy(1, 0, 0, 16)                # never beyond HR_MAX_WORLD
    assert admit(policy=too_wide, world=16) == hr.HR_DECLINE_WORLD_SIZE


def test_route_names():
    assert hr.hr_route_str(hr.HR_ROUTE_HOST) == "HR_ROUTE_HOST"
    assert hr.hr_route_str(hr.HR_DECLINE_TOO_LARGE) == "HR_DECLINE_TOO_LARGE"
    assert hr.hr_route_str(42) == "HR_ROUTE_UNKNOWN"


def test_decode_sized_bound():
    # the SGLang page's default: 64 rows x hidden 6144 = 393216 values
    assert hr.hr_decode_numel(64, 1, 6144) == 393_216
    # its review thread: 32 requests with 4 draft tokens need 128 rows
    assert hr.hr_decode_numel(32, 4, 6144) == 128 * 6144
    assert hr.hr_decode_numel(64, 0, 6144) == 393_216          # 0 tokens counts as 1
    # the 1Cat-vLLM cap of 256 KiB is 32 decode tokens at hidden 4096
    assert hr.hr_decode_numel(32, 1, 4096) * 2 == 256 * 1024


def test_workspace_stride():
    mib2 = (2 << 20) // 2                        # 2 MiB in binary16 values
    assert hr.hr_workspace_stride(16_777_216) == 16_777_216 + 2048
    assert hr.hr_workspace_stride(1) == mib2 + 2048
    assert hr.hr_workspace_stride(mib2 + 1) == 2 * mib2 + 2048
    for n in (1, 4096, 393_216, 16_777_216, 9_000_001):
        s = hr.hr_workspace_stride(n)
        assert s >= n and (s * 2) % (2 << 20) == 4096
