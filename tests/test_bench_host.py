"""Host-side logic of bench.py (no GPU): the one-GPU guard, the choice of the
step loop's dispatches in counter runs, the counter scaling, and the per-call
percentiles."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_step_grid_is_the_most_dispatched():
    rows = [("realign_kernel<16>", 100.0, 4096)] * 23 + [("realign_kernel<16>", 5.0, 1024)] * 8 \
        + [("greedy_chunk_kernel<true>", 7.0, 2048)] * 22 + [("greedy_chunk_kernel<true>", 3.0, 1024)] * 24
    assert bench._per_kernel(rows, "realign", step_grid=True) == (100.0, 23)
    assert bench._per_kernel(rows, "greedy_chunk", step_grid=True) == (3.0, 24)
    mean, n = bench._per_kernel(rows, "realign")
    assert n == 31 and mean == pytest.approx((23 * 100 + 8 * 5) / 31)
    assert bench._per_kernel(rows, "absent") == (None, 0)
    tie = [("k", 1.0, 10)] * 3 + [("k", 2.0, 20)] * 3     # a tie goes to the larger grid
    assert bench._per_kernel(tie, "k", step_grid=True) == (2.0, 3)


def _counter_dir(tmp_path, name, counter, rows):
    d = tmp_path / name / "run"
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kname, grid, value in rows:
            w.writerow(dict(Kernel_Name=kname, Grid_Size=grid, Counter_Name=counter, Counter_Value=value))
    return str(tmp_path / name)


def test_traffic_scaled_by_the_copy_probe(tmp_path, monkeypatch):
    probe_kib = bench.PROBE_BYTES / 1024
    fetch = _counter_dir(tmp_path, "f", "FETCH_SIZE",
                         [("neg_kernel", 1, 0.5 * probe_kib)] + [("realign_kernel<16>", 7, 1000.0)] * 3
                         + [("greedy_verify_kernel<true>", 9, 40.0)] * 2)
    write = _counter_dir(tmp_path, "w", "WRITE_SIZE",
                         [("neg_kernel", 1, probe_kib)] + [("realign_kernel<16>", 7, 3000.0)] * 3
                         + [("greedy_verify_kernel<true>", 9, 1.0)] * 2)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out))
    bench.record_traffic(fetch, write)
    t = json.loads(out.read_text())
    assert t["probe"]["fetch_factor"] == pytest.approx(0.5) and t["probe"]["write_factor"] == pytest.approx(1.0)
    # bytes = 1024 * (FETCH / 0.5 + WRITE / 1.0)
    assert bench.traffic_bytes("realign_kernel") == pytest.approx(1024 * (2000.0 + 3000.0))
    assert bench.traffic_bytes("greedy_verify_kernel") == pytest.approx(1024 * (80.0 + 1.0))
    t["sources_sha256"] = "stale"
    out.write_text(json.dumps(t))
    assert bench.traffic_bytes("realign_kernel") is None      # counters of other sources are not used


def test_per_call_spread_nearest_rank():
    ts = [0.005, 0.001, 0.004, 0.002, 0.003]             # seconds, unsorted
    sp = bench._spread(ts, 1e3)                          # in ms
    assert sp == {"p10": pytest.approx(1.0), "median": pytest.approx(3.0), "p90": pytest.approx(5.0)}
    many = [i * 1e-6 for i in range(1, 21)]              # 1 .. 20 us
    sp = bench._spread(many, 1e6)
    assert sp["p10"] == pytest.approx(3.0) and sp["p90"] == pytest.approx(18.0)
    assert sp["median"] == pytest.approx(10.5)
    assert bench._spread([2e-3], 1e3) == {"p10": pytest.approx(2.0), "median": pytest.approx(2.0),
                                          "p90": pytest.approx(2.0)}
