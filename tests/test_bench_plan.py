"""bench.py's warm-up and timed-region planning (host logic, no GPU).

Without --warmup / --steps each timed section warms up for at least SETTLE_S
seconds and times at least TIMED_S seconds (and at least MIN_STEPS steps),
from the duration of one step; given on the command line, the counts are used
exactly and the step is not timed first.  A stub stands in for torch's device
events: one step of the stub "takes" a fixed time.
"""
import argparse
import math

import pytest

import bench


class _Clock:
    def __init__(self, step_s):
        self.step_s = step_s
        self.t = 0.0
        self.calls = 0

    def step(self):
        self.t += self.step_s
        self.calls += 1


class _Event:
    def __init__(self, clock):
        self.clock = clock
        self.at = None

    def record(self):
        self.at = self.clock.t

    def elapsed_time(self, other):  # milliseconds, as torch.cuda.Event reports
        return (other.at - self.at) * 1e3


class _Torch:
    def __init__(self, clock):
        clock_ = clock

        class cuda:
            @staticmethod
            def Event(enable_timing=True):
                return _Event(clock_)

            @staticmethod
            def synchronize():
                pass

        self.cuda = cuda


def _args(warmup=None, steps=None):
    return argparse.Namespace(warmup=warmup, steps=steps)


@pytest.mark.parametrize("step_s", [1e-6, 170e-6, 1.4e-3, 85e-3, 2.0])
def test_default_counts_cover_the_durations(step_s):
    clock = _Clock(step_s)
    warmup, steps = bench.plan_steps(_args(), _Torch(clock), clock.step)
    assert clock.calls == 2  # one untimed call, one timed
    if step_s * bench.MIN_WARMUP < bench.SETTLE_S and math.ceil(bench.SETTLE_S / step_s) <= 100000:
        assert warmup * step_s >= bench.SETTLE_S * (1 - 1e-9)
        assert (warmup - 1) * step_s < bench.SETTLE_S
    assert warmup >= bench.MIN_WARMUP and warmup <= 100000
    assert steps >= bench.MIN_STEPS and steps <= 100000
    if step_s * bench.MIN_STEPS < bench.TIMED_S and math.ceil(bench.TIMED_S / step_s) <= 100000:
        assert steps * step_s >= bench.TIMED_S * (1 - 1e-9)


def test_explicit_counts_are_used_exactly():
    clock = _Clock(1e-3)
    assert bench.plan_steps(_args(3, 7), _Torch(clock), clock.step) == (3, 7)
    assert clock.calls == 0  # nothing run to plan


def test_one_explicit_count_keeps_it():
    clock = _Clock(1e-3)
    warmup, steps = bench.plan_steps(_args(warmup=2), _Torch(clock), clock.step)
    assert warmup == 2 and steps == max(bench.MIN_STEPS, math.ceil(bench.TIMED_S / 1e-3))
    clock = _Clock(1e-3)
    warmup, steps = bench.plan_steps(_args(steps=11), _Torch(clock), clock.step)
    assert steps == 11 and warmup == max(bench.MIN_WARMUP, math.ceil(bench.SETTLE_S / 1e-3))


def test_run_timed_runs_exactly_the_planned_steps():
    clock = _Clock(2e-3)
    ms, warmup, steps = bench.run_timed(_args(4, 9), _Torch(clock), clock.step, "stub")
    assert (warmup, steps) == (4, 9)
    assert clock.calls == 4 + 9
    assert ms == pytest.approx(2.0)


def test_sustained_figure_only_after_explicit_counts():
    # explicit counts: the line's value is the exact K-step timing, and the
    # same step is timed again after the default settling, as a second figure
    clock = _Clock(170e-6)
    ms, warmup, steps = bench.run_timed(_args(5, 20), _Torch(clock), clock.step, "stub")
    assert clock.calls == 25
    sus = bench.sustained_after(_args(5, 20), _Torch(clock), clock.step, ms)
    ms2, w2, s2 = sus
    assert w2 * 170e-6 >= bench.SETTLE_S * (1 - 1e-9) and s2 * 170e-6 >= bench.TIMED_S * (1 - 1e-9)
    assert clock.calls == 25 + w2 + s2
    assert ms2 == pytest.approx(0.17)
    obj = bench.sustained_obj(sus, 1.0, "GB/s", 8000.0)
    assert obj["value"] == pytest.approx(1.0 / 170e-6, rel=1e-4) and obj["warmup"] == w2 and obj["steps"] == s2
    # duration-based counts already: no second figure, nothing run
    clock = _Clock(170e-6)
    assert bench.sustained_after(_args(), _Torch(clock), clock.step, 0.17) is None
    assert bench.sustained_after(_args(warmup=5), _Torch(clock), clock.step, 0.17) is None
    assert clock.calls == 0
