"""Host logic of bench.py (CPU only): the counter-to-bytes arithmetic of the
traffic record, its invalidation when a kernel source changes, and the one-GPU
exit."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def write_counters(d, counter, rows):
    """A rocprofv3 --pmc CSV with (kernel name, value) rows for `counter`."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, v in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})
            wr.writerow({"Kernel_Name": name, "Counter_Name": "OTHER", "Counter_Value": 1e9})


@pytest.fixture()
def sandbox(tmp_path, monkeypatch):
    """bench's paths pointed at a temporary tree holding one fake kernel source."""
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "traffic.json"))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"k": ["k.hip"]})
    monkeypatch.setattr(bench, "KERNEL_PATTERNS", {"k": ("my_kernel<8>",), "k2": ("my_kernel<8>", "their_kernel<1>")})
    return tmp_path


def test_traffic_record_scales_by_the_copy_calibration(sandbox, capsys):
    t = sandbox
    kib = 1024.0
    # the kernel: two dispatches per counter run, mean 1000 KiB fetched and 100 KiB written
    write_counters(t / "f", "FETCH_SIZE", [("void my_kernel<8>(Args)", 900.0), ("void my_kernel<8>(Args)", 1100.0),
                                          ("void other(Args)", 5.0)])
    write_counters(t / "w", "WRITE_SIZE", [("void my_kernel<8>(Args)", 100.0), ("void my_kernel<8>(Args)", 100.0)])
    # the copy reads half its known size in FETCH_SIZE and all of it in WRITE_SIZE
    copy = bench.COPYCAL_BYTES / kib
    write_counters(t / "cf", "FETCH_SIZE", [("copyBuffer", copy / 2)])
    write_counters(t / "cw", "WRITE_SIZE", [("copyBuffer", copy)])
    bench.record_traffic("k", str(t / "f"), str(t / "w"), str(t / "cf"), str(t / "cw"), ["cmd"])
    capsys.readouterr()
    rec = json.load(open(bench.TRAFFIC_JSON))["k"]
    assert rec["dispatches"] == [2, 2]
    assert rec["copy_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["copy_calibration"]["write_scale"] == pytest.approx(1.0)
    assert rec["bytes_per_launch"] == round(1000 * kib * 2.0 + 100 * kib * 1.0)
    assert bench.recorded_traffic("k") == rec["bytes_per_launch"]


def test_traffic_record_averages_over_its_kernels(sandbox, monkeypatch, capsys):
    t = sandbox
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"k2": ["k.hip"]})
    # one kernel twice at 1000 KiB, the other once at 400 KiB: each kernel counts once, 700 KiB
    write_counters(t / "f", "FETCH_SIZE", [("void my_kernel<8>(Args)", 1000.0), ("void my_kernel<8>(Args)", 1000.0),
                                          ("void their_kernel<1>(Args)", 400.0), ("void other(Args)", 5.0)])
    write_counters(t / "w", "WRITE_SIZE", [("void my_kernel<8>(Args)", 10.0), ("void their_kernel<1>(Args)", 10.0)])
    copy = bench.COPYCAL_BYTES / 1024.0
    write_counters(t / "cf", "FETCH_SIZE", [("copyBuffer", copy)])
    write_counters(t / "cw", "WRITE_SIZE", [("copyBuffer", copy)])
    bench.record_traffic("k2", str(t / "f"), str(t / "w"), str(t / "cf"), str(t / "cw"), ["cmd"])
    capsys.readouterr()
    rec = json.load(open(bench.TRAFFIC_JSON))["k2"]
    assert rec["dispatches"] == [3, 2]
    assert rec["fetch_kib_per_dispatch"] == pytest.approx(700.0)
    assert "my_kernel<8>" in rec["kernel_name"] and "their_kernel<1>" in rec["kernel_name"]
    assert "other" not in rec["kernel_name"]


def test_traffic_record_is_void_once_the_kernel_changes(sandbox, capsys):
    t = sandbox
    for d, c in (("f", "FETCH_SIZE"), ("w", "WRITE_SIZE")):
        write_counters(t / d, c, [("my_kernel<8>", 10.0)])
    for d, c in (("cf", "FETCH_SIZE"), ("cw", "WRITE_SIZE")):
        write_counters(t / d, c, [("copyBuffer", bench.COPYCAL_BYTES / 1024.0)])
    bench.record_traffic("k", str(t / "f"), str(t / "w"), str(t / "cf"), str(t / "cw"), ["cmd"])
    capsys.readouterr()
    assert bench.recorded_traffic("k") is not None
    (t / "k.hip").write_text("kernel v2\n")
    assert bench.recorded_traffic("k") is None
    assert bench.recorded_traffic("absent") is None


def test_committed_traffic_record_names_its_kernel():
    """The committed record covers the decode kernel, with the commands that made it."""
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    r = rec["decode_f16_step"]
    assert all(p in r["kernel_name"] for p in bench.KERNEL_PATTERNS["decode_f16_step"])
    assert any("FETCH_SIZE" in c for c in r["commands"]) and any("WRITE_SIZE" in c for c in r["commands"])
    assert r["bytes_per_launch"] > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


class _FakeGraph:
    def __init__(self, fn, calls, log):
        self.fn, self.calls, self.log = fn, calls, log

    def replay(self):
        for i in range(self.calls):
            self.fn(i)


@pytest.mark.parametrize("steps,warmup", [(20, 5), (2000, 200), (1, 0), (128, 128), (129, 3), (300, 7)])
def test_decode_steps_run_exactly_as_requested(monkeypatch, steps, warmup):
    """The timed region runs exactly --steps steps and the warm-up exactly --warmup
    steps, whatever the graph size (whole replays plus one remainder graph), and
    every replayed step continues the weight rotation from step 0."""
    ran = []
    monkeypatch.setattr(bench, "capture", lambda fn, calls, stream, torch: _FakeGraph(fn, calls, ran))
    period = 128
    runner = bench.StepRunner(lambda i: ran.append(i), period, None, None)
    runner.prepare(warmup, steps)
    ran.clear()
    runner.run(warmup)
    assert len(ran) == warmup
    ran.clear()
    runner.run(steps)
    assert len(ran) == steps
    q, r = bench.step_schedule(steps, period)
    assert q * period + r == steps and 0 <= r < period
    # whole replays each run steps 0 .. period-1, the remainder 0 .. r-1
    assert ran == list(range(period)) * q + list(range(r))


def test_bad_step_counts_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "0"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "--steps" in r.stderr
