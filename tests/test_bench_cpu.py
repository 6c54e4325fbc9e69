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


def test_algorithmic_counts_of_the_configs():
    # bytes: q, k, v, out once in the input type (+ fp32 log-gates), plus the
    # final state (and z when normalised); flops: 2C(dk+dv) + 4 dk dv per
    # token-head -- the per-token-head figures of the workloads' definitions
    sys.path.insert(0, ROOT)
    import bench
    from recurrent_attention_amd import workloads
    W = workloads.WORKLOADS
    w1 = W["linear_elu1_L64_d16_fp32"]
    assert bench.prefill_bytes(w1) == 64 * 4 * 4 * 16 + 16 * 16 * 4 + 16 * 4
    assert bench.prefill_flops(w1) == 64 * 2048
    w2 = W["linear_elu1_B4H8_L2048_d64"]
    assert bench.prefill_bytes(w2) == 32 * 2048 * 512 + 32 * (64 * 64 * 4 + 64 * 4)
    assert bench.prefill_flops(w2) == 32 * 2048 * 32768
    w3 = W["retention_B2H16_L8192_d128"]
    assert bench.prefill_bytes(w3) == 32 * 8192 * 1024 + 32 * 128 * 128 * 4
    w4 = W["gla_B1H16_L32768_d128"]
    assert bench.prefill_bytes(w4) == 16 * 32768 * 1536 + 16 * 128 * 128 * 4
    assert bench.prefill_flops(w4) == 16 * 32768 * 98304
    # the headline's floor is its HBM time at 8 TB/s
    frac, floor_us = bench.attainable_frac(w4, 0.2016)
    assert abs(floor_us - bench.prefill_bytes(w4) / 8e12 * 1e6) < 1e-9
    assert abs(frac - floor_us / 201.6) < 1e-12
    # fp32 inputs take the fp32 matrix peak for their flop floor
    assert bench.attainable_frac(w1, 1.0)[1] == max(
        bench.prefill_bytes(w1) / 8e12, bench.prefill_flops(w1) / 157.3e12) * 1e6
