"""The timeline tool's record analysis (message_fp16_all_amd/timeline.py) on
synthetic records whose phases, skews and poll counts are known, so the
figures it prints for the profiles are checked against values set by hand.
CPU only: no library is loaded."""
import numpy as np
import pytest

from message_fp16_all_amd import hr, timeline

TPU = 100.0   # ticks per microsecond


def ll_records(calls=200, nb=4, active=2, skew_us=None, polls=None):
    """Two-rank LL records: call k starts at k * 10 us on rank 0; rank 1
    starts skew_us[k] later; after entry, counter 1 us, publish 1 us, polls
    1 us, barrier 2 us, fold 0.5 us.
    Records are stored out of call order (the tool sorts by call number)."""
    rec = np.zeros((calls, 2, nb, timeline.WORDS), dtype=np.uint64)
    skew_us = np.zeros(calls) if skew_us is None else skew_us
    polls = np.ones((calls, 2), dtype=np.int64) if polls is None else polls
    for k in range(calls):
        slot = (k * 7) % calls                 # a permutation of the slots
        for r in range(2):
            t0 = 1_000_000 + k * 10 * TPU + (skew_us[k] * TPU if r == 1 else 0)
            steps = np.cumsum([0, 1, 1, 1, 2, 0.5]) * TPU
            for b in range(active):
                rec[slot, r, b, :6] = (t0 + steps[:6]).astype(np.uint64)
                rec[slot, r, b, 6] = polls[k, r]
                rec[slot, r, b, 7] = k + 1
    return rec


def test_ll_rank_analysis_reads_skew_and_second_polls():
    calls = 200
    skew = np.where(np.arange(calls) % 2 == 0, 0.8, -0.6)       # alternating, as the cycle does
    polls = np.ones((calls, 2), dtype=np.int64)
    polls[np.arange(calls) % 2 == 0, 0] = 2                    # rank 0 early -> its second poll
    polls[np.arange(calls) % 2 == 1, 1] = 2
    rec = ll_records(calls, skew_us=skew, polls=polls)
    (med, p10, p90), ranks = timeline.analyse_ll_ranks(rec, TPU)
    assert p10 == pytest.approx(-0.6, abs=1e-6)
    assert p90 == pytest.approx(0.8, abs=1e-6)
    assert ranks[0][0] == pytest.approx(0.5, abs=0.01)
    assert ranks[1][0] == pytest.approx(0.5, abs=0.01)
    assert ranks[0][1] == pytest.approx(0.8, abs=1e-6)          # rank 0 polled twice when it led
    assert ranks[1][1] == pytest.approx(-0.6, abs=1e-6)


def test_ll_phase_analysis_reads_the_last_ending_workgroup():
    calls = 100
    rec = ll_records(calls, skew_us=np.full(calls, 0.3))
    # the replay's span: first call's start to the last call's end (rank 1,
    # 0.3 us late, ends 5.5 us after its entry), which the tool's clock rate
    # is taken against
    elapsed = ((calls - 1) * 10 + 0.3 + 5.5) * 1e-6
    rows, per_call, tpu, nact, polls = timeline.analyse(rec, elapsed, hr.HR_ALGO_LL)
    got = {name: med for name, med, _ in rows}
    assert tpu == pytest.approx(TPU, rel=0.01)
    assert got["entry"] == pytest.approx(0.3, abs=0.01)          # rank 1 ends last, 0.3 us late
    assert got["counter"] == pytest.approx(1.0, abs=0.01)
    assert got["publish (issue words)"] == pytest.approx(1.0, abs=0.01)
    assert got["lane 0's hold and polls until its peer words match"] == pytest.approx(1.0, abs=0.01)
    assert got["rest of the workgroup (barrier)"] == pytest.approx(2.0, abs=0.01)
    assert got["fold + store"] == pytest.approx(0.5, abs=0.01)
    assert got["call period (start to next start)"] == pytest.approx(10.0, abs=0.01)
    assert nact == 4 and polls == 1
