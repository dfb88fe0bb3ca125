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


def _counter_dir(tmp_path, name, rows):
    """rows: (kernel name, grid, counter, value)."""
    d = tmp_path / name / "run"
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kname, grid, counter, value in rows:
            w.writerow(dict(Kernel_Name=kname, Grid_Size=grid, Counter_Name=counter, Counter_Value=value))
    return str(tmp_path / name)


def _bench_log(tmp_path, rea_bytes, ver_bytes):
    p = tmp_path / "pmc1.log"
    p.write_text("[bench] warmup\n" + json.dumps({
        "roofline": {"algorithmic_bytes_all_dispatches": rea_bytes},
        "roofline_verify": {"algorithmic_bytes_per_launch": ver_bytes}}) + "\n")
    return str(p)


def _passes(tmp_path, probe, kernels):
    """One directory per counter pass; probe and kernels map counter -> value."""
    dirs = []
    for i, names in enumerate(bench.COUNTER_PASSES):
        rows = []
        for c in names:
            rows.append(("neg_kernel", 1, c, probe[c]))
            for kname, grid, n, vals in kernels:
                rows += [(kname, grid, c, vals[c])] * n
        dirs.append(_counter_dir(tmp_path, f"pmc{i + 1}", rows))
    return dirs


def test_traffic_scaled_by_the_copy_probe_and_from_request_sizes(tmp_path, monkeypatch):
    P = bench.PROBE_BYTES
    probe = {"FETCH_SIZE": 0.5 * P / 1024, "WRITE_SIZE": P / 1024,
             "TCC_EA0_RDREQ_sum": P / 128, "TCC_EA0_RDREQ_32B_sum": 0, "TCC_EA0_RDREQ_64B_sum": 0,
             "TCC_EA0_RDREQ_128B_sum": P / 128, "TCC_EA0_WRREQ_sum": P / 64, "TCC_EA0_WRREQ_64B_sum": P / 64,
             "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum": 100.0, "TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum": 50.0}
    rea = dict(probe, FETCH_SIZE=1000.0, WRITE_SIZE=3000.0, TCC_EA0_RDREQ_sum=20, TCC_EA0_RDREQ_32B_sum=4,
               TCC_EA0_RDREQ_64B_sum=6, TCC_EA0_RDREQ_128B_sum=10, TCC_EA0_WRREQ_sum=30, TCC_EA0_WRREQ_64B_sum=25)
    ver = dict(rea, FETCH_SIZE=40.0, WRITE_SIZE=1.0)
    # the step loop's grids are the most dispatched ones; a smaller grid of the same kernel is ignored
    kernels = [("realign_kernel<16, int>", 7, 3, rea), ("realign_kernel<16, int>", 5, 1, probe),
               ("greedy_verify_kernel<true>", 9, 2, ver)]
    dirs = _passes(tmp_path, probe, kernels)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out))
    monkeypatch.setattr(bench, "TRAFFIC_MD", str(tmp_path / "traffic.md"))
    bench.record_traffic(_bench_log(tmp_path, 5000 * 1024, 81 * 1024), *dirs)
    t = json.loads(out.read_text())
    assert t["probe"]["fetch_factor"] == pytest.approx(0.5) and t["probe"]["write_factor"] == pytest.approx(1.0)
    assert t["probe"]["request_read_bytes"] == P and t["probe"]["request_write_bytes"] == P
    # scaled: bytes = 1024 * (FETCH / 0.5 + WRITE / 1.0)
    assert bench.traffic_bytes("realign_kernel") == pytest.approx(1024 * (2000.0 + 3000.0))
    assert bench.traffic_bytes("greedy_verify_kernel") == pytest.approx(1024 * (80.0 + 1.0))
    # requests: 4 x 32 + 6 x 64 + 10 x 128 read, 25 x 64 + 5 x 32 written
    assert bench.traffic_bytes("realign_kernel", requests=True) == 4 * 32 + 6 * 64 + 10 * 128 + 25 * 64 + 5 * 32
    assert t["kernels"]["realign_kernel"]["dispatches"] == 3
    assert t["kernels"]["realign_kernel"]["algorithmic_bytes"] == 5000 * 1024
    md = (tmp_path / "traffic.md").read_text()
    assert "TCC_EA0_RDREQ_128B_sum" in md and "| `realign_kernel` | 3 |" in md
    t["sources_sha256"] = "stale"
    out.write_text(json.dumps(t))
    assert bench.traffic_bytes("realign_kernel") is None      # counters of other sources are not used
    assert bench.traffic_bytes("realign_kernel", requests=True) is None


def test_request_bytes_needs_every_count():
    c = {"TCC_EA0_RDREQ_32B_sum": 1, "TCC_EA0_RDREQ_64B_sum": 1, "TCC_EA0_RDREQ_128B_sum": 1,
         "TCC_EA0_WRREQ_sum": 3, "TCC_EA0_WRREQ_64B_sum": 1}
    assert bench.request_bytes(c) == (32 + 64 + 128, 64 + 2 * 32)
    del c["TCC_EA0_RDREQ_128B_sum"]
    assert bench.request_bytes(c) is None


def test_trace_summary(tmp_path, monkeypatch):
    d = tmp_path / "trace" / "run"
    d.mkdir(parents=True)
    names = ["void specv::(anonymous namespace)::realign_kernel<16, int>(specv::(anonymous namespace)::RealignParams)",
             "void specv::(anonymous namespace)::greedy_verify_kernel<true>(specv::(anonymous namespace)::GreedyParams)",
             "void at::native::neg_kernel_cuda(at::TensorIteratorBase&)", "some_other_kernel"]
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i, n in enumerate(names):                 # the probe (i = 2) starts at 10^6
            for j in range(2):
                t0 = 1000 * j + (10 ** 6 if i >= 2 else 0) + (10 ** 7 if i == 1 and j == 1 else 0)
                w.writerow(dict(Kernel_Name=n, Grid_Size_X=64 * (i + 1), Start_Timestamp=t0,
                                End_Timestamp=t0 + 2000 * (i + 1) + 1000 * j))
    logp = tmp_path / "trace.log"
    logp.write_text(json.dumps({"value": 1.0, "ms_per_step": 2.0, "realign_ms_per_call": 3.0,
                                "verify_us_per_launch": 18.0, "copy_probe_GBps": 6000.0,
                                "roofline": {"achieved": 5000.0, "frac": 0.625},
                                "roofline_verify": {"achieved": 4000.0, "frac": 0.5}}) + "\n")
    monkeypatch.setattr(bench, "TRACE_MD", str(tmp_path / "k.md"))
    bench.summarize_trace(str(tmp_path / "trace"), str(logp))
    md = (tmp_path / "k.md").read_text()
    assert "| `realign_kernel<16, int>` | 64 | 2 | 2.50 | 2.00 | 3.00 | **step** |" in md
    # one launch after the probe: not only the step workload's
    assert "| `greedy_verify_kernel<true>` | 128 | 2 | 4.50 | 4.00 | 5.00 |  |" in md
    assert "torch neg (copy probe)" in md and "some_other_kernel" not in md


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
