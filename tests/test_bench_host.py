"""Host-side checks of bench.py (no GPU): the one-GPU guard, the roofline arithmetic of the
21x30x52, 12-head, d128 workload, and the counter summary's copy calibration on synthetic
rocprofv3 csv output."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_roofline_arithmetic():
    N, d, h = 32760, 128, 12
    fr, br = bench.stage_work(N, d, h, 52)     # stage R: blocks of W = 52
    fl, bl = bench.stage_work(N, d, h, 630)    # stage L: groups of T*H = 630
    assert br == bl == 8 * N * d * h == 402554880
    assert fr == 4.0 * N * d * h * 52 and fl == 4.0 * N * d * h * 630
    # stage R is HBM-bound (50.32 us at 8 TB/s), stage L MFMA-bound (50.72 us at 2.5 PF)
    assert bench.roofline_us(fr, br) == pytest.approx(br / 8e12 * 1e6)
    assert bench.roofline_us(fl, bl) == pytest.approx(fl / 2.5e15 * 1e6)
    assert bench.roofline_us(fr, br) + bench.roofline_us(fl, bl) == pytest.approx(101.04, abs=0.01)


def _write_counters(d, rows):
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_counter_summary_scales_by_the_copy(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    kern = "void ma::group_attn_bf16<128, 4, false>(ma::AttnLaunch)"
    # a copy of one 100.6 MB tensor reads FETCH 49140 KiB and WRITE 98280 KiB per dispatch
    _write_counters(str(tmp_path / "cf"), [(copy, "FETCH_SIZE", 49140)] * 3 + [(kern, "FETCH_SIZE", 1)])
    _write_counters(str(tmp_path / "cw"), [(copy, "WRITE_SIZE", 98280)] * 3)
    _write_counters(str(tmp_path / "kf"), [(kern, "FETCH_SIZE", 150000), (kern, "FETCH_SIZE", 150002),
                                           ("other", "FETCH_SIZE", 7)])
    _write_counters(str(tmp_path / "kw"), [(kern, "WRITE_SIZE", 98280)] * 2)
    out = bench.summarize_counters(str(tmp_path / "kf"), str(tmp_path / "kw"), str(tmp_path / "cf"),
                                   str(tmp_path / "cw"), "stage_l", out_path=str(tmp_path / "t.json"))
    tensor = 12 * 32760 * 128 * 2
    assert out["fetch_scale"] == pytest.approx(tensor / (1024.0 * 49140))
    assert out["write_scale"] == pytest.approx(tensor / (1024.0 * 98280))
    assert out["fetch_bytes"] == pytest.approx(1024.0 * 150001 * out["fetch_scale"])
    assert out["write_bytes"] == pytest.approx(1024.0 * 98280 * out["write_scale"])
    assert out["bytes_per_launch"] == pytest.approx(out["fetch_bytes"] + out["write_bytes"])
    assert out["algorithmic_bytes"] == 8.0 * 32760 * 128 * 12
    assert os.path.exists(str(tmp_path / "t.json"))


class _FakeEvent:
    """Stands in for torch.cuda.Event on the host: elapsed_time in ms of wall clock."""

    def __init__(self, enable_timing=True):
        self.t = None

    def record(self, stream=None):
        import time
        self.t = time.perf_counter()

    def elapsed_time(self, other):
        return (other.t - self.t) * 1e3


def test_time_loop_warmup_does_not_count_the_first_call(monkeypatch):
    """A slow first call (on a fresh process the first launch loads code objects) must not
    stand in for the clock warm-up: steady calls still run until MIN_WARM_MS have passed."""
    import time
    import torch
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    monkeypatch.setattr(torch.cuda, "Event", _FakeEvent)
    calls = []

    def fn(i):
        calls.append(i)
        time.sleep(0.15 if len(calls) == 1 else 0.002)   # first call 150 ms, then 2 ms each

    info = {}
    bench.time_loop(fn, steps=3, warmup=2, min_warm_ms=40.0, info=info)
    # about 40 ms / 2 ms of steady calls after the first one, in batches of 8
    assert info["extra_warmup"] >= 8
    steady = len(calls) - 3 - 1          # untimed calls after the first, timed calls excluded
    assert steady * 2.0 >= 40.0 * 0.8    # they covered (nearly) the minimum warm-up time


def test_repeat_stats_quantiles(monkeypatch):
    import torch
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    monkeypatch.setattr(torch.cuda, "Event", _FakeEvent)
    r = bench.repeat_stats(lambda i: None, steps=2, first_ms=5.0, repeats=3)
    assert r["loops"] == 4 and r["steps_each"] == 2
    assert r["p10_ms"] <= r["median_ms"] <= r["p90_ms"] <= 5.0
