"""Host logic of bench.py's timing loop, on the CPU: which steps carry HIP events.

An event record costs the stream a few microseconds, so the timed region may sample at most
every 10th step; when it is too short for 10 pairs of samples, the same schedule continues
after it.  The device calls are replaced by stand-ins that log what the loop does.
"""
import bench
import pytest

torch = pytest.importorskip("torch")


class _Log:
    def __init__(self):
        self.syncs = 0
        self.clock = 0.0
        self.steps = []      # (step index, sync count when launched, events passed)


@pytest.fixture
def fake_cuda(monkeypatch):
    log = _Log()

    class Event:
        def __init__(self, enable_timing=False):
            self.t = None

        def record(self, *a, **k):
            log.clock += 1.0
            self.t = log.clock

        def elapsed_time(self, other):
            return other.t - self.t

    def synchronize():
        log.syncs += 1

    monkeypatch.setattr(torch.cuda, "Event", Event)
    monkeypatch.setattr(torch.cuda, "synchronize", synchronize)
    return log


def _run(log, steps):
    n = {"i": 0}

    def step(S, ev):
        log.steps.append((n["i"], log.syncs, ev is not None))
        if ev is not None:
            ev[0].record()
            ev[1].record()
            ev[2].record()
        n["i"] += 1

    st = {}
    ms, ph1, ph2 = bench.time_loop(step, [None], steps, warmup=3, settle_ms=0.0, stats_out=st)
    return st, ph1, ph2


@pytest.mark.parametrize("steps", [5, 20, 200, 333])
def test_sampling_schedule(fake_cuda, steps):
    st, ph1, ph2 = _run(fake_cuda, steps)
    warm = st["warmup_steps_run"]
    launched = fake_cuda.steps[warm:]
    # the timed region is the `steps` launches after the warm-up; nothing sampled more often than
    # every EVENT_EVERY-th step, in it or after it
    sampled = [k for k, (_, _, ev) in enumerate(launched) if ev]
    assert all(k % bench.EVENT_EVERY == 0 for k in sampled)
    assert len(sampled) % 2 == 0 and len(sampled) // 2 >= bench.MIN_EVENT_PAIRS
    assert st["event_samples"] == len(sampled)
    assert st["event_samples_in_timed_region"] == sum(1 for k in sampled if k < steps)
    assert st["event_samples_after_timed_region"] == sum(1 for k in sampled if k >= steps)
    # the extra steps exist only to complete the pairs, and run after the timed region's closing sync
    extra = len(launched) - steps
    assert extra == max(0, 2 * bench.MIN_EVENT_PAIRS * bench.EVENT_EVERY - steps)
    closing = launched[steps - 1][1] + 1 if steps else None
    assert all(sync >= closing for (_, sync, _) in launched[steps:])
    assert len(ph1) == len(ph2) == len(sampled) // 2
