"""The benchmark script's contract, checked without a GPU: it refuses more than
one GPU with a message, and its settling rule (untimed calls until the call time
stops falling) stops where it should.  (The freshness of the counter summaries it
reads is checked in test_profile_summary.py.)"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "one GPU" in r.stdout


def _fake_groups(medians):
    """time_group() stand-in returning groups whose median is the next value."""
    it = iter(medians)

    def time_group():
        m = next(it)
        return [m] * bench.SETTLE_GROUP
    return time_group


def test_settling_stops_once_the_call_time_stops_falling():
    # a card raising its clock: 1.10, 1.00, 0.94 ms, then flat within 0.5 %
    calls, med = bench.settle_groups(_fake_groups([1.10, 1.00, 0.94, 0.938, 0.5]), max_s=60)
    assert med == [1.1, 1.0, 0.94, 0.938]
    assert calls == 4 * bench.SETTLE_GROUP


def test_settling_takes_at_least_the_minimum_number_of_groups():
    calls, med = bench.settle_groups(_fake_groups([0.9, 0.9, 0.9, 0.9]), max_s=60)
    assert len(med) == bench.SETTLE_MIN_GROUPS
    assert calls == bench.SETTLE_MIN_GROUPS * bench.SETTLE_GROUP


def test_settling_stops_at_its_time_limit():
    ticks = iter(range(100))
    calls, med = bench.settle_groups(_fake_groups([3.0 - 0.1 * i for i in range(30)]),
                                     max_s=4.5, clock=lambda: float(next(ticks)))
    # the clock advances one second per reading: groups end once 4.5 s have passed
    assert len(med) == 5 and med[-1] < med[-2]


def test_settling_can_be_switched_off():
    assert bench.settle_groups(_fake_groups([]), max_s=0) == (0, [])


def test_settling_groups_span_a_fixed_call_time():
    # later groups hold enough calls for SETTLE_GROUP_MS of call time, within bounds
    assert bench.settle_group_size(5.0) == bench.SETTLE_GROUP
    assert bench.settle_group_size(0.0625) == 320   # 20 ms of 62.5 us calls
    assert bench.settle_group_size(1e-5) == bench.SETTLE_GROUP_MAX
    # the call count is the sum of the group sizes
    sizes = iter([10, 400, 400, 400])

    def time_group():
        return [0.05] * next(sizes)
    calls, med = bench.settle_groups(time_group, max_s=60)
    assert calls == 10 + 400 + 400 and len(med) == 3
