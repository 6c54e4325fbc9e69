"""bench.py's command line without a GPU: it runs on one GPU only, so any
other GPU count (or a distributed launch) exits with status 2 and a message
before anything touches a device; and its timing helpers follow the
protocol they state."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=e, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_distributed_launch_is_refused():
    r = _bench(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "WORLD_SIZE=4" in r.stderr


def test_time_steps_orders_flush_event_step():
    # the protocol on a fake torch: each timed step is preceded by a flush
    # and bracketed by its own events; the back-to-back run has no flushes
    sys.path.insert(0, ROOT)
    import bench
    log = []

    class Ev:
        def __init__(self, enable_timing=True):
            self.t = None

        def record(self):
            log.append("event")
            self.t = len(log)

        def elapsed_time(self, other):
            return float(other.t - self.t)

    class Cuda:
        Event = Ev

        @staticmethod
        def synchronize():
            log.append("sync")

    class FakeTorch:
        cuda = Cuda

    class Args:
        warmup, steps = 2, 3

    t = bench.time_steps(FakeTorch, lambda: log.append("step"), Args,
                         lambda: log.append("flush"))
    timed = log[log.index("sync") + 1:]
    timed = timed[:timed.index("sync")]
    assert timed == ["flush", "event", "step", "event"] * 3
    assert log[:4] == ["flush", "step", "flush", "step"]          # warm-up, flushed
    assert log[-4:] == ["step", "step", "step", "sync"]           # back to back
    assert t["mean"] == 2.0 and t["min"] == 2.0
