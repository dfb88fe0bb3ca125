#!/usr/bin/env python3
"""Benchmark of the verify-and-commit step on one MI355X.

Workload: large-batch greedy, realign-heavy -- B=32 sequences, k=8 drafts,
V=128256 bf16 logits ~N(0, 2), per-sequence acceptance rate alpha_b in
[0.3, 0.95], bf16 KV cache of 32 layers x 8 KV heads x head_dim 128,
contiguous and left-padded, prefix lengths in [512, 4096] (~18 GB).

One step = greedy verify of the batch's 288 logit rows (spec_verify_greedy)
followed by the commit that realigns the KV cache, position ids and mask in
place (spec_commit_realign_kv), chained on the device (the end column and
lengths never visit the host).  Logits rotate over 8 distinct buffers
(~590 MB, more than the 256 MB last-level cache) so every verify reads HBM.

Prints one JSON line.  `value` is whole-step throughput (verified rows per
second, verify + commit).  `roofline` is for the dominant kernel (the KV
realign); `roofline_verify` for the verify call, which is one launch (its
streaming workgroups and the workgroup that commits them); both use
algorithmic bytes (verify: every logit byte plus ids; realign: 2 x bytes of
every moved KV row plus the position-id and mask rows) over the kernel's
average duration from HIP events on the launch stream (for verify, events
around back-to-back launches: one call's events add microseconds of their own).  `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W]
    python bench.py --record-traffic LOG DIR1 DIR2 DIR3 DIR4   (after the four rocprofv3 --pmc passes)
    python bench.py --summarize-trace TRACE_DIR LOG            (after a rocprofv3 --kernel-trace run)
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import itertools
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified rows/s + KV-realign HBM GB/s (% of peak) at B=32 k=8 V=128256"
PEAK_HBM = 8.0e12            # MI355X HBM3E, bytes/s (published)
WORKLOAD = 3
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic_verify_realign_B32_k8_V128256.json")
KERNEL_SOURCES = ["speculative_decoding_verification_04_amd/csrc/verify_greedy.hip",
                  "speculative_decoding_verification_04_amd/csrc/commit_realign.hip",
                  "speculative_decoding_verification_04_amd/csrc/common.h"]
PROBE_BYTES = 2 << 30


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def sources_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# ------------------------------------------------------------ counters ----
def _counter_rows(directory: str, counter: str):
    import csv
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r.get("Kernel_Name", ""), float(r["Counter_Value"]), int(r.get("Grid_Size", 0))))
    return rows


def _per_kernel(rows, key, step_grid=False):
    """Mean counter value per dispatch of the kernels named like key.  With
    step_grid, only the dispatches of the grid launched most often (the
    largest on a tie): the step loop's, not a secondary call or a smaller
    batch-size run of the same kernel."""
    sel = [(v, g) for name, v, g in rows if key in name]
    if step_grid and sel:
        count = {}
        for _, g in sel:
            count[g] = count.get(g, 0) + 1
        top = max(count, key=lambda g: (count[g], g))
        sel = [(v, g) for v, g in sel if g == top]
    vals = [v for v, _ in sel]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


# Counter passes (one rocprofv3 --pmc run each; at most 4 TCC counters a run).
# FETCH_SIZE and WRITE_SIZE are rocprofv3's derived KiB per dispatch; the
# request passes count the L2-to-memory requests by size, which gives the
# bytes without any scale fitted to a probe.
COUNTER_PASSES = [
    ["FETCH_SIZE"],
    ["WRITE_SIZE"],
    ["TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum"],
    ["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum",
     "TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum"],
]
TRAFFIC_KERNELS = ("greedy_verify_kernel", "realign_kernel")
TRAFFIC_MD = TRAFFIC_JSON[:-len(".json")] + ".md"
TRACE_MD = os.path.join(ROOT, "profiles", "kernels_verify_realign_B32_k8_V128256.md")
COUNTER_BENCH_ARGS = "--steps 3 --warmup 1 --step-only --no-cpu-baseline"


def request_bytes(c: dict):
    """(read, write) bytes over the L2-to-memory interface from request counts
    and their sizes: reads of 32, 64 or 128 bytes, writes of 64 bytes or
    else 32.  None if a count is missing."""
    need = ["TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum",
            "TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum"]
    if any(c.get(x) is None for x in need):
        return None
    rd = 32 * c["TCC_EA0_RDREQ_32B_sum"] + 64 * c["TCC_EA0_RDREQ_64B_sum"] + 128 * c["TCC_EA0_RDREQ_128B_sum"]
    wr = 64 * c["TCC_EA0_WRREQ_64B_sum"] + 32 * (c["TCC_EA0_WRREQ_sum"] - c["TCC_EA0_WRREQ_64B_sum"])
    return rd, wr


def _bench_line(log_path: str) -> dict:
    with open(log_path) as f:
        return json.loads([x for x in f if x.startswith("{")][-1])


def record_traffic(bench_log: str, *dirs: str) -> None:
    """Turn the counter passes of this benchmark (COUNTER_PASSES, in order,
    each run as `bench.py COUNTER_BENCH_ARGS` under rocprofv3 --pmc) into the
    committed traffic summary (JSON and markdown).  Each counter's mean per
    dispatch is taken over the step loop's dispatches of each kernel and over
    the copy probe (torch int32 negation of PROBE_BYTES: that many bytes read
    and as many written).  bench_log: the output of one of those runs, for
    the algorithmic bytes of the same dispatches."""
    rows = {}
    for d, names in zip(dirs, COUNTER_PASSES):
        for c in names:
            r = _counter_rows(d, c)
            if r:
                rows[c] = r

    def per(c, key, probe=False):
        if c not in rows:
            return None
        sel = [r for r in rows[c] if "neg" in r[0].lower()] if probe else rows[c]
        v, _ = _per_kernel(sel, "" if probe else key, step_grid=True)
        return v

    probe = {"kernel": "torch int32 negation (one 4-byte read and one 4-byte write per element)",
             "bytes_read": PROBE_BYTES, "bytes_written": PROBE_BYTES}
    for c in rows:
        probe[c] = per(c, "", probe=True)
    pf, pw = probe.get("FETCH_SIZE"), probe.get("WRITE_SIZE")
    probe["fetch_factor"] = (pf * 1024 / PROBE_BYTES) if pf else None
    probe["write_factor"] = (pw * 1024 / PROBE_BYTES) if pw else None
    rb = request_bytes(probe)
    probe["request_read_bytes"], probe["request_write_bytes"] = rb if rb else (None, None)
    bl = _bench_line(bench_log)
    alg = {"greedy_verify_kernel": bl["roofline_verify"]["algorithmic_bytes_per_launch"],
           "realign_kernel": bl["roofline"]["algorithmic_bytes_all_dispatches"]}
    out = {"probe": probe, "kernels": {}, "sources_sha256": sources_digest(),
           "counter_bench_args": COUNTER_BENCH_ARGS}
    for key in TRAFFIC_KERNELS:
        kk = {c: per(c, key) for c in rows}
        kk["fetch_kib_per_dispatch"] = kk.pop("FETCH_SIZE", None)
        kk["write_kib_per_dispatch"] = kk.pop("WRITE_SIZE", None)
        kk["dispatches"] = _per_kernel(rows["FETCH_SIZE"], key, step_grid=True)[1] if "FETCH_SIZE" in rows else 0
        rb = request_bytes(kk)
        kk["request_read_bytes"], kk["request_write_bytes"] = rb if rb else (None, None)
        kk["algorithmic_bytes"] = alg[key]
        out["kernels"][key] = kk
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(out, f, indent=1)
    with open(TRAFFIC_MD, "w") as f:
        f.write(_traffic_md(out))
    print(json.dumps(out))


def _traffic_md(t: dict) -> str:
    p = t["probe"]
    fk = lambda v: "n/a" if v is None else f"{v:.4g}"
    cmds = [f"timeout -s KILL 120 rocprofv3 --pmc {' '.join(c)} -f csv -d $R/gpurun_out/pmc{i + 1} -o run "
            f"-- python3 $R/bench.py {COUNTER_BENCH_ARGS} > $R/gpurun_out/pmc{i + 1}.log"
            for i, c in enumerate(COUNTER_PASSES)]
    out = ["# HBM traffic per dispatch: verify + realign, B=32 k=8 V=128256", "",
           "Four counter passes of the step loop (3 timed steps after 1 warm-up step, then the copy probe). "
           "Each pass is its own run (R is the repository root):", "", "```",
           "cd /tmp && export TMPDIR=/tmp", *cmds,
           "python3 $R/bench.py --record-traffic $R/gpurun_out/pmc1.log " +
           " ".join(f"$R/gpurun_out/pmc{i + 1}" for i in range(len(COUNTER_PASSES))), "```", "",
           "Two independent byte counts:", "",
           "- **scaled**: FETCH_SIZE and WRITE_SIZE, each divided by what it reads for the copy probe per byte "
           f"moved (FETCH {fk(p['fetch_factor'])}, WRITE {fk(p['write_factor'])}).",
           "- **requests**: the L2-to-memory requests counted by size (reads of 32, 64 and 128 bytes; "
           "writes of 64 bytes, the rest 32), times their size. No scale is fitted.", "",
           f"The copy probe moves {PROBE_BYTES} bytes each way. Its read requests give "
           f"{fk(p.get('request_read_bytes'))} bytes and its write requests {fk(p.get('request_write_bytes'))}. "
           "FETCH_SIZE counts every read request that is not 32 bytes as 64 bytes; its 128-byte term rests on "
           "TCC_BUBBLE, which reads 0 here, while TCC_EA0_RDREQ_128B counts every read. That is why FETCH_SIZE "
           "reads half.", "",
           "| kernel | dispatches | algorithmic bytes | scaled bytes | request bytes (read + write) | "
           "request / algorithmic |", "|---|---|---|---|---|---|"]
    for key, k in t["kernels"].items():
        sc = (1024 * (k["fetch_kib_per_dispatch"] / p["fetch_factor"] + k["write_kib_per_dispatch"] / p["write_factor"])
              if k.get("fetch_kib_per_dispatch") is not None and p.get("fetch_factor") else None)
        rq = (k["request_read_bytes"] + k["request_write_bytes"]) if k.get("request_read_bytes") is not None else None
        ratio = f"{rq / k['algorithmic_bytes']:.4f}" if rq else "n/a"
        out.append(f"| `{key}` | {k['dispatches']} | {k['algorithmic_bytes']:.6g} | {fk(sc)} | "
                   f"{fk(k.get('request_read_bytes'))} + {fk(k.get('request_write_bytes'))} | {ratio} |")
    out += ["", "DRAM credit stalls (cycles summed over the L2 channels) per memory request:", "",
            "| kernel | read-credit stalls / read request | write-credit stalls / write request |", "|---|---|---|"]
    for name, k in [("copy probe", p)] + list(t["kernels"].items()):
        rs, ws_ = k.get("TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum"), k.get("TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum")
        rr, wr = k.get("TCC_EA0_RDREQ_sum"), k.get("TCC_EA0_WRREQ_sum")
        a = f"{rs / rr:.3f}" if rs is not None and rr else "n/a"
        b = f"{ws_ / wr:.3f}" if ws_ is not None and wr else "n/a"
        out.append(f"| {name} | {a} | {b} |")
    out += ["", f"Kernel sources hash: `{t['sources_sha256'][:16]}` (bench.py reports `traffic` only while the "
            "sources match).", ""]
    return "\n".join(out)


def _trace_rows(directory: str):
    """(kernel label, grid) -> (durations in us, start times) from a rocprofv3
    kernel trace, for the library's kernels and the copy probe."""
    import csv
    import re
    acc = {}
    for path in glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                n = r["Kernel_Name"]
                m = re.search(r"::(\w+_kernel)(<.*?>)?\(", n)
                if "specv" in n and m:
                    label = m.group(1) + (m.group(2) or "").replace("specv::(anonymous namespace)::", "")
                elif "neg_kernel" in n:
                    label = "torch neg (copy probe)"
                elif "floor_max_kernel" in n:
                    label = "floor_max_kernel (read floor, bench_floor.hip)"
                else:
                    continue
                t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
                grid = int(r["Grid_Size_X"] if "Grid_Size_X" in r else r.get("Grid_Size", 0))
                d = acc.setdefault((label, grid), ([], []))
                d[0].append((t1 - t0) / 1e3)
                d[1].append(t0)
    return acc


def summarize_trace(trace_dir: str, bench_log: str) -> None:
    """Write the committed kernel-duration summary from a rocprofv3
    --kernel-trace run of the default bench and that run's output.  Launches
    before the copy probe are the step workload's own (the timed steps, the
    back-to-back verify launches and the parity check); they are marked."""
    acc = _trace_rows(trace_dir)
    b = _bench_line(bench_log)
    probe = [min(v[1]) for (k, _), v in acc.items() if k.startswith("torch neg")]
    t_probe = min(probe) if probe else None
    out = ["# Kernel durations: verify + realign, B=32 k=8 V=128256, bf16 KV 32x8x128 (~18 GB)", "",
           "Command (MI355X, one GPU; R is the repository root):", "", "```",
           "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -f csv -d $R/gpurun_out/trace -o run "
           "-- python3 $R/bench.py > $R/gpurun_out/trace.log",
           "python3 $R/bench.py --summarize-trace $R/gpurun_out/trace $R/gpurun_out/trace.log", "```", "",
           "Every launch of the library's kernels in that run, grouped by kernel and grid size. Rows marked "
           "**step** hold only launches of the B=32 k=8 V=128256 step workload: the warm-up and timed steps, "
           "the back-to-back verify launches and the parity check, all before the copy probe. The other rows "
           "are the secondary measurements and the batch-size sweeps.", "",
           "| kernel | grid | calls | avg (us) | min (us) | max (us) | |", "|---|---|---|---|---|---|---|"]
    for (k, g), (v, starts) in sorted(acc.items(), key=lambda x: -sum(x[1][0])):
        step = (t_probe is not None and max(starts) < t_probe and not k.startswith("torch neg")
                and not k.startswith("floor_max"))
        out.append(f"| `{k}` | {g} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                   f"{'**step**' if step else ''} |")
    rf, rv = b["roofline"], b["roofline_verify"]
    out += ["", "From the bench line of the same run (HIP events on the launch stream):", "",
            f"- value {b['value']:.0f} rows/s, {b['ms_per_step']:.3f} ms per step",
            f"- `realign_kernel`: {b['realign_ms_per_call']:.3f} ms per call, {rf['achieved']:.0f} GB/s, "
            f"{rf['frac']:.3f} of 8 TB/s",
            f"- `greedy_verify_kernel` (the whole verify call): {b['verify_us_per_launch']:.2f} us per launch, "
            f"{rv['achieved']:.0f} GB/s, {rv['frac']:.3f} of 8 TB/s",
            f"- copy probe (torch int32 negation, 2 GiB each way): {b['copy_probe_GBps']:.0f} GB/s",
            (f"- read floor (`floor_max_kernel`, one pass over the verify call's logits): "
             f"{b['verify_read_floor']['us_per_launch']:.2f} us per launch, "
             f"{b['verify_read_floor']['frac_of_peak']:.3f} of 8 TB/s" if b.get("verify_read_floor") else
             "- read floor: not measured"), "",
            "Under the tracer every dispatch carries the tracer's own overhead, so the bench's back-to-back "
            "timings in a traced run are slower than untraced ones; the kernel rows above are the kernels' own "
            "durations, to set beside an untraced bench line.", ""]
    with open(TRACE_MD, "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))


def traffic_bytes(key: str, requests: bool = False):
    """Measured HBM bytes per dispatch, None if stale or absent: FETCH_SIZE and
    WRITE_SIZE scaled by the copy probe's per-byte readings, or (requests)
    the request counts times their sizes."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256") != sources_digest():
        return None
    k = t["kernels"].get(key, {})
    if requests:
        if k.get("request_read_bytes") is None:
            return None
        return k["request_read_bytes"] + k["request_write_bytes"]
    p = t["probe"]
    if not k.get("fetch_kib_per_dispatch") or not p.get("fetch_factor") or not p.get("write_factor"):
        return None
    return 1024 * (k["fetch_kib_per_dispatch"] / p["fetch_factor"] + k["write_kib_per_dispatch"] / p["write_factor"])


# --------------------------------------------------------------- bench ----
def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--buffers", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step only: no secondary calls or batch-size sweeps (for counter runs)")
    ap.add_argument("--record-traffic", nargs=len(COUNTER_PASSES) + 1, metavar="PATH",
                    help="the log of one counter run, then the output directory of each counter pass")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"))
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return 0
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the step shards "
              "by sequence with no exchange); run it with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import speculative_decoding_verification_04_amd as sv
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.workload(WORKLOAD)
    R = args.warmup + args.steps
    g = W.kv_geometry(WORKLOAD, rounds=R)
    L, H, D, B, k, n, E, C = (g[x] for x in ("L", "H", "D", "B", "k", "n", "E", "C"))
    V = cfg["V"]
    nbuf = args.buffers

    log(f"generating {nbuf} rounds of logits [{B}, {k + 1}, {V}] bf16")
    rounds = [W.greedy_round(WORKLOAD, round_=r) for r in range(nbuf)]
    logits = [torch.from_numpy(r["logits"].view(np.int16)).to(dev).view(torch.bfloat16) for r in rounds]
    drafts = [torch.from_numpy(r["drafts"]).to(dev) for r in rounds]
    log(f"allocating and filling KV [{L}, 2, {B}, {H}, {C}, {D}] bf16 "
        f"({L * 2 * B * H * C * D * 2 / 1e9:.1f} GB)")
    kv = torch.empty((L, 2, B, H, C, D), dtype=torch.bfloat16, device=dev)
    tokens = W.prefix_tokens(WORKLOAD, B, E + 1)
    W.fill_kv_torch(kv, E, n, torch.as_tensor(tokens, device=dev), "bf16")

    i32 = dict(dtype=torch.int32, device=dev)
    acc, emit = torch.empty(B, **i32), torch.empty(B, **i32)
    toks, offs = torch.empty(B, k + 1, **i32), torch.empty(B + 1, **i32)
    ws = sv.workspace(sv.spec_verify_greedy_workspace_bytes(B, k, V, sv.SPEC_BF16), dev)
    Ebuf = [torch.tensor([E], **i32), torch.empty(1, **i32)]
    Nbuf = [torch.as_tensor(n, **i32), torch.empty(B, **i32)]
    pos, mask = torch.empty(B, C, **i32), torch.empty(B, C, **i32)
    moved = torch.zeros(R, dtype=torch.int64, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(R)]
    torch.cuda.synchronize()

    def step(r: int) -> None:
        s = r % nbuf
        evs[r][0].record()
        sv.spec_verify_greedy(logits[s], drafts[s], acc, emit, toks, ws, emit_offsets=offs)
        evs[r][1].record()
        sv.spec_commit_realign_kv(kv, k, Ebuf[r % 2], Nbuf[r % 2], emit, Ebuf[(r + 1) % 2],
                                  Nbuf[(r + 1) % 2], pos, mask, bytes_moved=moved[r:r + 1])
        evs[r][2].record()

    log(f"warmup {args.warmup} steps")
    for r in range(args.warmup):
        step(r)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for r in range(args.warmup, R):
        step(r)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    timed = range(args.warmup, R)
    t_ver = [evs[r][0].elapsed_time(evs[r][1]) * 1e-3 for r in timed]
    t_rea = [evs[r][1].elapsed_time(evs[r][2]) * 1e-3 for r in timed]
    moved_h = moved.cpu().numpy()
    rows = B * (k + 1)
    ver_bytes = rows * V * 2 + B * k * 4 + rows * 4 + (3 * B + 1) * 4
    rea_bytes = [int(moved_h[r]) + 8 * B * C for r in timed]
    ver_GBps = ver_bytes * len(t_ver) / sum(t_ver)
    rea_GBps = sum(rea_bytes) / sum(t_rea)
    log(f"verify {statistics.mean(t_ver) * 1e6:.1f} us/call, realign {statistics.mean(t_rea) * 1e3:.3f} ms/call")

    # The verify launch alone: HIP events around one call add a few
    # microseconds of their own, so the kernel's duration is taken from
    # back-to-back launches over the rotating buffers between two events.
    n_back = 6 * nbuf
    for i in range(nbuf):
        sv.spec_verify_greedy(logits[i], drafts[i], acc, emit, toks, ws, emit_offsets=offs)
    a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_ev.record()
    for i in range(n_back):
        sv.spec_verify_greedy(logits[i % nbuf], drafts[i % nbuf], acc, emit, toks, ws, emit_offsets=offs)
    b_ev.record()
    torch.cuda.synchronize()
    t_launch = a_ev.elapsed_time(b_ev) * 1e-3 / n_back
    log(f"verify launch {t_launch * 1e6:.2f} us (back-to-back)")

    # The verify call's floor: one plain pass over the same logits in the same
    # chunks (bench_floor.hip, built beside this file by __graft_entry__.build),
    # the same back-to-back timing.  Not part of the step.
    read_floor = None
    if not args.step_only:
        read_floor = measure_read_floor(torch, logits, rows, V, n_back)
        if read_floor:
            log(f"read floor {read_floor['us_per_launch']:.2f} us per launch")

    # Reference for the verify call's floor: the framework's own reductions
    # over the same bytes (every logit of the same rotating buffers, the same
    # back-to-back timing).  Not part of the step.
    stream_ref = None
    if not args.step_only:
        stream_ref = {}
        flat = [x.view(rows, V) for x in logits]
        for name, fn in (("torch.amax", lambda x: torch.amax(x, dim=-1)),
                         ("torch.argmax", lambda x: torch.argmax(x, dim=-1))):
            for i in range(nbuf):
                fn(flat[i])
            torch.cuda.synchronize()
            a_r, b_r = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_r.record()
            for i in range(n_back):
                fn(flat[i % nbuf])
            b_r.record()
            torch.cuda.synchronize()
            t_r = a_r.elapsed_time(b_r) * 1e-3 / n_back
            stream_ref[name] = {"us_per_call": t_r * 1e6, "GBps": rows * V * 2 / t_r / 1e9,
                                "frac_of_peak": rows * V * 2 / t_r / PEAK_HBM}
        log("stream reference: " + ", ".join(f"{k} {v['us_per_call']:.2f} us" for k, v in stream_ref.items()))

    # parity guard: one more verify of buffer 0 against the oracle (outside the timed region)
    import oracle
    sv.spec_verify_greedy(logits[0], drafts[0], acc, emit, toks, ws, emit_offsets=offs)
    torch.cuda.synchronize()
    ref = oracle.greedy_verify(rounds[0]["logits"], "bf16", rounds[0]["drafts"])
    parity = bool(np.array_equal(toks.cpu().numpy(), ref["out_tokens"]) and
                  np.array_equal(emit.cpu().numpy(), ref["emit_count"]))

    probe = None
    if not args.no_probe:
        log("copy probe")
        src = torch.ones(PROBE_BYTES // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        ts = []
        for _ in range(5):
            a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            torch.neg(src, out=dst)
            b_.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b_) * 1e-3)
        probe = 2 * PROBE_BYTES / min(ts)
        del src, dst

    secondary = None
    if not args.step_only:
        log("secondary: stochastic verify, tree verify, paged commit, same-length grouping")
        secondary = secondary_measurements(dev, np, torch, sv, W)
        log("batch scaling: realign cost and grouping rate against batch size")
        secondary.update(batch_scaling(dev, np, torch, sv, W))
        cpu_side = not args.no_cpu_baseline
        for c in (0, 1, 2):
            log(f"workload {c}: verify + commit step")
            secondary[f"workload_{c}_step"] = config_step(dev, np, torch, sv, W, c, cpu=cpu_side)
        log("workload 4: grouping, per-batch verify, realign-based commit")
        secondary["workload_4_grouped"] = grouped_workload(dev, np, torch, sv, W, cpu=cpu_side)
        log("draft-cache re-sync")
        secondary["draft_resync"] = draft_resync(dev, np, torch, sv, W)
        log("EQSPEC vs EXSPEC loop")
        secondary["policy_loop"] = policy_loop(dev, np, torch, sv, W)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on host cores)")
        cpu = cpu_baseline(rounds[0], ref, g, np)

    tr_rea = traffic_bytes("realign_kernel")
    tr_ver = traffic_bytes("greedy_verify_kernel")
    avg_rea_bytes = sum(rea_bytes) / len(rea_bytes)
    # every dispatch of the step loop, warm-up included: what the counter runs average over
    all_rea_bytes = sum(int(moved_h[r]) + 8 * B * C for r in range(R)) / R
    result = {
        "metric": METRIC,
        "value": rows * args.steps / wall,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generators; logits N(0,2), planted drafts, hashed KV contents)",
        "config": {"workload": "large-batch greedy verify + realign-heavy commit",
                   "B": B, "k": k, "V": V, "kv": f"{L} layers x {H} KV heads x {D} bf16",
                   "prefix": "512-4096", "capacity_columns": C, "logit_buffers": nbuf},
        "roofline": {"bound": "hbm", "kernel": "realign_kernel", "achieved": rea_GBps / 1e9,
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": rea_GBps / PEAK_HBM,
                     "traffic": tr_rea, "traffic_requests": traffic_bytes("realign_kernel", requests=True),
                     "algorithmic_bytes_per_launch": avg_rea_bytes,
                     "algorithmic_bytes_all_dispatches": all_rea_bytes},
        "roofline_verify": {"bound": "hbm", "kernel": "greedy_verify_kernel (the whole spec_verify_greedy call: one launch)",
                            "achieved": ver_bytes / t_launch / 1e9,
                            "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": ver_bytes / t_launch / PEAK_HBM,
                            "traffic": tr_ver,
                            "traffic_requests": traffic_bytes("greedy_verify_kernel", requests=True),
                            "algorithmic_bytes_per_launch": ver_bytes,
                            "timing": f"HIP events around {n_back} back-to-back launches over the rotating buffers"},
        "verify_read_floor": read_floor,
        "verify_stream_reference": stream_ref,
        "verify_rows_per_s": rows / t_launch,
        "verify_us_per_launch": t_launch * 1e6,
        "verify_us_per_call_in_step": statistics.mean(t_ver) * 1e6,
        "verify_GBps_in_step": ver_GBps / 1e9,
        "realign_GBps": rea_GBps / 1e9,
        "realign_ms_per_call": statistics.mean(t_rea) * 1e3,
        "per_call_spread": {"verify_us": _spread(t_ver, 1e6), "realign_ms": _spread(t_rea, 1e3)},
        "copy_probe_GBps": None if probe is None else probe / 1e9,
        "parity_checked": parity,
        "secondary": secondary,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result))
    return 0


def measure_read_floor(torch, logits, rows: int, V: int, n_back: int):
    """Per-launch time of bench_floor.so's one-pass chunk maximum over the
    verify call's rotating logit buffers (HIP events around n_back
    back-to-back launches), or None when the probe is not built."""
    import ctypes
    path = os.path.join(ROOT, "bench_floor.so")
    if not os.path.exists(path):
        log("read floor: bench_floor.so is not built (run __graft_entry__.build())")
        return None
    lib = ctypes.CDLL(path)
    fn = lib.floor_chunk_max_bf16
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    nb = len(logits)
    out = torch.empty(rows * ((V + 16383) // 16384), dtype=torch.float32, device=logits[0].device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call(i):
        if fn(ctypes.c_void_p(logits[i % nb].data_ptr()), rows, V, ctypes.c_void_p(out.data_ptr()), stream) < 0:
            raise RuntimeError("floor_chunk_max_bf16 rejected its arguments")

    call(0)
    torch.cuda.synchronize()
    if float(out.max()) != float(logits[0].float().max()):
        raise RuntimeError("read floor: chunk maxima disagree with the buffer's maximum")
    t = _back_to_back(torch, call, n_back)
    nbytes = rows * V * 2
    return {"kernel": "floor_max_kernel (bench_floor.hip: chunk maxima only, no argmax, no commit)",
            "us_per_launch": t * 1e6, "GBps": nbytes / t / 1e9, "frac_of_peak": nbytes / t / PEAK_HBM,
            "bytes": nbytes, "timing": f"HIP events around {n_back} back-to-back launches over the rotating buffers"}


def _spread(ts, scale: float) -> dict:
    """p10, median and p90 of per-call times (HIP events), scaled."""
    q = sorted(ts)

    def pct(f: float) -> float:                  # nearest rank
        return q[min(len(q) - 1, max(0, int(round(f * (len(q) - 1)))))] * scale

    return {"p10": pct(0.1), "median": statistics.median(q) * scale, "p90": pct(0.9)}


def _time_calls(torch, fn, reps: int, inner: int = 24):
    """Seconds per call: (GPU time, host-inclusive time).

    GPU time: `inner` calls captured in one HIP graph (the calls launch kernels
    only), replayed `reps` times between HIP events on the replay stream; the
    median replay divided by `inner`.  Host-inclusive: HIP events around single
    eager calls, median; for calls of a few microseconds this is mostly the
    Python binding and launch latency."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    eager = statistics.median(ts[2:])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(inner):
            fn()
    torch.cuda.synchronize()
    gs = []
    for _ in range(max(5, reps // 4)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        gs.append(a.elapsed_time(b) * 1e-3 / inner)
    del g
    fn()                                    # outputs read afterwards come from an eager call
    torch.cuda.synchronize()
    return statistics.median(gs), eager


def _rates(t: float, th: float, nbytes: int) -> dict:
    return {"us_per_call": t * 1e6, "us_per_call_host": th * 1e6, "algorithmic_bytes": nbytes,
            "GBps": nbytes / t / 1e9, "frac_of_peak": nbytes / t / PEAK_HBM}


def secondary_measurements(dev, np, torch, sv, W) -> dict:
    """The other calls at their workload shapes (not part of `value`)."""
    out = {}
    r = W.sample_round(2)
    B, k, V = r["B"], r["k"], r["V"]
    p, q = torch.from_numpy(r["p"]).to(dev), torch.from_numpy(r["q"]).to(dev)
    d, u = torch.from_numpy(r["drafts"]).to(dev), torch.from_numpy(r["uniforms"]).to(dev)
    i32 = dict(dtype=torch.int32, device=dev)
    acc, emit, toks = torch.empty(B, **i32), torch.empty(B, **i32), torch.empty(B, k + 1, **i32)
    offs, mass = torch.empty(B + 1, **i32), torch.empty(B, dtype=torch.float64, device=dev)
    ws = sv.workspace(sv.spec_verify_sample_workspace_bytes(B, k, V), dev)
    # 6 copies of p and q (262 MB, more than the 256 MB last-level cache), used in turn
    pq = [(p, q)] + [(p.clone(), q.clone()) for _ in range(5)]
    ip = itertools.count()

    def call():
        pc, qc = pq[next(ip) % len(pq)]
        sv.spec_verify_sample(pc, qc, d, u, acc, emit, toks, ws, emit_offsets=offs, final_mass=mass)

    t, th = _time_calls(torch, call, 22)
    m, e = acc.cpu().numpy(), emit.cpu().numpy()
    # realized algorithmic bytes: the row drawn from (p_j and q_j after a rejection,
    # p_k after full acceptance) plus two gathered scalars per examined draft
    row_bytes = sum(8 * V if (e[b] > m[b] and m[b] < k) else (4 * V if e[b] > m[b] else 0) for b in range(B))
    gathers = 8 * int(sum(min(int(m[b]) + 1, k) for b in range(B)))
    nbytes = row_bytes + gathers + 4 * B * (k + 1) * 2
    out["sample_verify"] = {"workload": f"stochastic verify, B={B} k={k} V={V} f32, 6 rotating p/q copies",
                            **_rates(t, th, nbytes), "rows_per_s": B * (k + 1) / t}
    del pq
    # stochastic verification from bf16 logits with temperature 0.7, top-k 50, top-p 0.9
    g = W.sample_logits(2)
    T, K, TP = g["temperature"], 50, 0.9
    zt = torch.from_numpy(g["zt"]).to(dev).to(torch.bfloat16)
    zd = torch.from_numpy(g["zd"]).to(dev).to(torch.bfloat16)
    # drafting (outside the step): draw from the processed draft rows by inverse CDF
    qproc = torch.empty(zd.shape, dtype=torch.float32, device=dev)
    wsp = sv.workspace(sv.spec_process_workspace_bytes(B * k, V), dev)
    sv.spec_process_logits(zd, T, wsp, top_k=K, top_p=TP, probs=qproc)
    gen = torch.Generator(device=dev).manual_seed(7)
    ud = torch.rand(B, k, 1, device=dev, generator=gen, dtype=torch.float64)
    cq = torch.cumsum(qproc.double(), dim=-1)
    dl = torch.searchsorted(cq, ud * cq[..., -1:]).clamp_(max=V - 1).squeeze(-1).to(torch.int32).contiguous()
    ul = torch.from_numpy(g["uniforms"]).to(dev)
    wsl = sv.workspace(sv.spec_verify_sample_logits_workspace_bytes(B, k, V), dev)
    # 12 copies of the two logit tensors (267 MB), used in turn
    zz = [(zt, zd)] + [(zt.clone(), zd.clone()) for _ in range(11)]
    iz = itertools.count()

    def call():
        a, b = zz[next(iz) % len(zz)]
        sv.spec_verify_sample_logits(a, b, dl, ul, acc, emit, toks, wsl, temperature=T, top_k=K,
                                     top_p=TP, emit_offsets=offs, final_mass=mass)

    t, th = _time_calls(torch, call, 22)
    m, e = acc.cpu().numpy(), emit.cpu().numpy()
    rows_read = B * (2 * k + 1) * V * 2                       # the statistics pass reads every row once
    redraw = sum(4 * V if (e[b] > m[b] and m[b] < k) else (2 * V if e[b] > m[b] else 0) for b in range(B))
    nbytes = rows_read + redraw
    out["sample_verify_logits"] = {"workload": f"stochastic verify from bf16 logits, B={B} k={k} V={V}, "
                                               f"T={T} top_k={K} top_p={TP}, 12 rotating logit copies",
                                   **_rates(t, th, nbytes), "rows_per_s": B * (k + 1) / t}
    # the same call with top-p alone (no top-k): the slice path with exact row weights
    iz2 = itertools.count()

    def call2():
        a, b = zz[next(iz2) % len(zz)]
        sv.spec_verify_sample_logits(a, b, dl, ul, acc, emit, toks, wsl, temperature=T, top_k=0, top_p=TP,
                                     emit_offsets=offs, final_mass=mass)

    t2, th2 = _time_calls(torch, call2, 22)
    m, e = acc.cpu().numpy(), emit.cpu().numpy()
    redraw = sum(4 * V if (e[b] > m[b] and m[b] < k) else (2 * V if e[b] > m[b] else 0) for b in range(B))
    nbytes = rows_read + redraw
    out["sample_verify_logits_top_p"] = {"workload": f"stochastic verify from bf16 logits, B={B} k={k} V={V}, "
                                                     f"T={T} top_p={TP} (no top-k), 12 rotating logit copies",
                                         **_rates(t2, th2, nbytes), "rows_per_s": B * (k + 1) / t2}
    del zz
    # paged layout: the commit is a rollback of lengths and pages, no KV bytes move
    g3 = W.kv_geometry(3)
    B3, k3, page = g3["B"], g3["k"], 16
    n3 = torch.as_tensor(g3["n"], dtype=torch.int32, device=dev)
    e3 = torch.as_tensor(W.accept_counts(3, 0), dtype=torch.int32, device=dev)
    maxp = (int(g3["n"].max()) + k3 + 1 + page - 1) // page
    bt = torch.arange(B3 * maxp, dtype=torch.int32, device=dev).view(B3, maxp)
    per = (k3 + page) // page
    kl, pk = torch.empty(B3, **i32), torch.empty(B3, **i32)
    fr, fo = torch.empty(B3 * per, **i32), torch.empty(B3 + 1, **i32)
    call = lambda: sv.spec_commit_paged(k3, page, n3, e3, bt, kl, pk, fr, fo)
    t, th = _time_calls(torch, call, 52)
    out["paged_commit"] = {"workload": f"paged rollback, B={B3} k={k3} page {page} rows, prefixes 512-4096",
                           "us_per_call": t * 1e6, "us_per_call_host": th * 1e6,
                           "pages_released": int(fo[-1].item()),
                           "kv_bytes_moved": 0}
    # tree verification: a 16-node candidate tree per sequence (parents among the
    # 3 nodes just below), bf16 logits over the large-batch vocabulary, rotating
    # over 3 logit buffers (394 MB, more than the 256 MB last-level cache); then
    # the compaction of the accepted path's KV slots in the large-batch cache
    cfg3 = W.workload(3)
    NT, Vt, nbt = 16, cfg3["V"], 3
    trees = []
    for i in range(nbt):
        gt = W.planted_tree(W.stream(3, "logits", i, 1), W.stream(3, "drafts", i, 1), B3, NT, Vt,
                            cfg3["logit_sd"], "bf16", W.alphas(3), 3)
        trees.append([torch.from_numpy(gt["logits"].view(np.int16)).to(dev).view(torch.bfloat16)] +
                     [torch.from_numpy(gt[key]).to(dev) for key in ("draft", "first_child", "next_sibling")])
        del gt
    acct, emitt, tokt = torch.empty(B3, **i32), torch.empty(B3, **i32), torch.empty(B3, NT, **i32)
    patht, offt = torch.empty(B3, NT, **i32), torch.empty(B3 + 1, **i32)
    wst = sv.workspace(sv.spec_verify_tree_workspace_bytes(B3, NT, Vt, sv.SPEC_BF16), dev)
    it = itertools.count()

    def tree_call():
        z, dtr, fct, nst = trees[next(it) % nbt]
        sv.spec_verify_tree(z, dtr, fct, nst, acct, emitt, tokt, patht, wst, emit_offsets=offt)

    reps = 22
    t, th = _time_calls(torch, tree_call, reps, inner=3 * nbt)
    nbytes = B3 * NT * Vt * 2
    accs = []
    for i in range(nbt):                                 # mean accept length over the buffers
        tree_call()
        accs.append(float(acct.float().mean().item()))
    out["tree_verify"] = {"workload": f"greedy tree verify, B={B3} N={NT} nodes (parents among the 3 below), "
                                      f"V={Vt} bf16, {nbt} rotating logit buffers",
                          **_rates(t, th, nbytes), "rows_per_s": B3 * NT / t,
                          "mean_accept_len": sum(accs) / nbt}
    del trees, wst
    # stochastic tree verification: 16-node trees whose siblings are draws
    # from the parent's q, float32 p and q over the stochastic workload's
    # vocabulary, rotating over 3 input sets (467 MB)
    Bs, Ns, Vs, nbs = 8, 16, W.workload(2)["V"], 3
    rng_s = W.stream(2, "tree", 0, 0)
    sets = []
    for i in range(nbs):
        gs_ = W.sampled_tree(rng_s, Bs, Ns, Vs)
        sets.append([torch.from_numpy(gs_["p"]).to(dev), torch.from_numpy(gs_["q"]).to(dev)] +
                    [torch.from_numpy(gs_[key]).to(dev) for key in ("draft", "first_child", "next_sibling",
                                                                   "uniforms")])
        del gs_
    accs_, emits_ = torch.empty(Bs, **i32), torch.empty(Bs, **i32)
    toks_, paths_, offs_ = torch.empty(Bs, Ns, **i32), torch.empty(Bs, Ns, **i32), torch.empty(Bs + 1, **i32)
    its = itertools.count()
    ws_s = sv.workspace(sv.spec_verify_tree_sample_workspace_bytes(Bs, Ns, Vs), dev)

    def tree_sample_call():
        ps, qs, ds, fcs, nss, us = sets[next(its) % nbs]
        sv.spec_verify_tree_sample(ps, qs, ds, fcs, nss, us, accs_, emits_, toks_, paths_, ws_s,
                                   emit_offsets=offs_)

    t, th = _time_calls(torch, tree_sample_call, 22, inner=3 * nbs)
    acc_s, emit_s = [], []
    for i in range(nbs):
        tree_sample_call()
        acc_s.append(float(accs_.float().mean().item()))
        emit_s.append(float(emits_.float().mean().item()))
    out["tree_sample_verify"] = {
        "workload": f"stochastic tree verify, B={Bs} N={Ns} nodes (parents among the 3 below, siblings drawn "
                    f"from the parent's q), V={Vs} f32 p/q, {nbs} rotating input sets",
        "us_per_call": t * 1e6, "us_per_call_host": th * 1e6,
        "mean_accept_len": sum(acc_s) / nbs, "mean_emit_count": sum(emit_s) / nbs,
        "workgroups_per_sequence": "several (workspace given)" if ws_s.numel() > 256 else 1}
    del sets
    # compaction of the last buffer's paths; successive calls use end columns
    # NT apart, so 48 calls touch 48 disjoint column ranges (more than the
    # last-level cache holds) and each call moves cold bytes
    Et = g3["E"]
    nE = 48
    kvt = torch.empty((g3["L"], 2, B3, g3["H"], Et + NT, g3["D"]), dtype=torch.bfloat16, device=dev)
    ends = [torch.tensor([Et - i * NT], **i32) for i in range(nE)]
    stt = torch.empty(B3, **i32)
    ic = itertools.count()
    call = lambda: sv.spec_compact_tree_kv(kvt, NT, ends[next(ic) % nE], patht, emitt, status=stt)
    t, th = _time_calls(torch, call, 52, inner=nE)
    ph, eh = patht.cpu().numpy(), emitt.cpu().numpy()
    moved = sum(int((ph[b, :eh[b]] != np.arange(eh[b])).sum()) for b in range(B3))
    col = g3["L"] * 2 * g3["H"] * g3["D"] * 2                  # one slot of one sequence, all planes
    nbytes = 2 * moved * col
    out["tree_compact"] = {"workload": f"tree slot compaction, B={B3} N={NT}, KV L={g3['L']} H={g3['H']} "
                                       f"D={g3['D']} bf16, end columns {Et - (nE - 1) * NT}..{Et}",
                           **_rates(t, th, nbytes), "slots_moved": moved,
                           "status_ok": bool((stt == 0).all().item())}
    del kvt
    P = W.pool_lengths()
    L = torch.as_tensor(P, dtype=torch.int32, device=dev)
    N = P.size
    perm, bstart, blen = torch.empty(N, **i32), torch.empty(N + 1, **i32), torch.empty(N, **i32)
    nb, ng = torch.empty(1, **i32), torch.empty(1, **i32)
    cfg = W.workload(4)
    call = lambda: sv.spec_group_same_length(L, cfg["B"], cfg["min_group"], perm, bstart, blen, nb, ng)
    t, th = _time_calls(torch, call, 52)
    out["group_same_length"] = {"workload": f"same-length grouping, pool {N}, batch {cfg['B']}, min_group {cfg['min_group']}",
                                "us_per_call": t * 1e6, "us_per_call_host": th * 1e6, "num_batches": int(nb.item()),
                                "grouped_fraction": int(ng.item()) / N}
    return out


def _dev_logits(torch, dev, np, arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev)


def _back_to_back(torch, fn, n: int) -> float:
    """Seconds per launch of n back-to-back calls between two HIP events."""
    fn(0)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / n


def config_step(dev, np, torch, sv, W, c: int, steps: int = 12, warm: int = 3, nbuf: int = 4,
                cpu: bool = True) -> dict:
    """One workload's whole step (verify + commit, chained on the device over
    `steps` rounds) and its parts; the oracle's step on the host beside it."""
    import oracle
    cfg = W.workload(c)
    R = warm + steps
    g = W.kv_geometry(c, rounds=R)
    L, H, D, B, k, n, E, C = (g[x] for x in ("L", "H", "D", "B", "k", "n", "E", "C"))
    V = cfg["V"]
    mode = cfg["mode"]
    i32 = dict(dtype=torch.int32, device=dev)
    kvdt = g["dtype"]
    kv = torch.empty((L, 2, B, H, C, D), dtype=torch.bfloat16 if kvdt == "bf16" else torch.float32, device=dev)
    tokens = torch.as_tensor(W.prefix_tokens(c, B, E + 1), device=dev)
    W.fill_kv_torch(kv, E, n, tokens, kvdt)
    acc, emit, toks = torch.empty(B, **i32), torch.empty(B, **i32), torch.empty(B, k + 1, **i32)
    offs = torch.empty(B + 1, **i32)
    if mode == "greedy":
        rounds = [W.greedy_round(c, round_=r) for r in range(nbuf)]
        ins = [(_dev_logits(torch, dev, np, r["logits"], r["dtype"]), torch.as_tensor(r["drafts"]).to(dev))
               for r in rounds]
        ws = sv.workspace(sv.spec_verify_greedy_workspace_bytes(B, k, V, sv.SPEC_BF16 if cfg["logit_dtype"] == "bf16"
                                                                else sv.SPEC_F32), dev)

        def verify(i):
            z, d = ins[i % nbuf]
            sv.spec_verify_greedy(z, d, acc, emit, toks, ws, emit_offsets=offs)
        elt = 2 if cfg["logit_dtype"] == "bf16" else 4
        ver_bytes = B * (k + 1) * V * elt + B * k * 4 + B * (k + 1) * 4 + (3 * B + 1) * 4
    else:
        rounds = [W.sample_round(c, round_=r) for r in range(nbuf)]
        ins = [tuple(torch.from_numpy(r[x]).to(dev) for x in ("p", "q", "drafts", "uniforms")) for r in rounds]
        mass = torch.empty(B, dtype=torch.float64, device=dev)
        ws = sv.workspace(sv.spec_verify_sample_workspace_bytes(B, k, V), dev)

        def verify(i):
            p_, q_, d, u = ins[i % nbuf]
            sv.spec_verify_sample(p_, q_, d, u, acc, emit, toks, ws, emit_offsets=offs, final_mass=mass)
        ver_bytes = None                        # realized per call (rows drawn from), below
    Eb = [torch.tensor([E], **i32), torch.empty(1, **i32)]
    Nb = [torch.as_tensor(n, **i32), torch.empty(B, **i32)]
    pos, mask = torch.empty(B, C, **i32), torch.empty(B, C, **i32)
    moved = torch.zeros(R, dtype=torch.int64, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(R)]

    def commit(r):
        sv.spec_commit_realign_kv(kv, k, Eb[r % 2], Nb[r % 2], emit, Eb[(r + 1) % 2], Nb[(r + 1) % 2], pos, mask,
                                  bytes_moved=moved[r:r + 1])

    def step(r):
        evs[r][0].record()
        verify(r)
        evs[r][1].record()
        commit(r)
        evs[r][2].record()

    for r in range(warm):
        step(r)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(warm, R):
        step(r)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_rea = [evs[r][1].elapsed_time(evs[r][2]) * 1e-3 for r in range(warm, R)]
    rea_bytes = [int(moved[r].item()) + 8 * B * C for r in range(warm, R)]
    # the same R rounds from the initial state, captured in one HIP graph and
    # replayed once: the steps' GPU time with no host launches between calls;
    # the replay must leave the cache and end column the eager rounds left
    kv_eager, e_eager = kv.clone(), int(Eb[R % 2].item())
    W.fill_kv_torch(kv, E, n, tokens, kvdt)
    Eb[0].fill_(E)
    Nb[0].copy_(torch.as_tensor(n, **i32))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(R):
            verify(r)
            commit(r)
    ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ga.record()
    graph.replay()
    gb.record()
    torch.cuda.synchronize()
    t_graph = ga.elapsed_time(gb) * 1e-3 / R
    graph_same = bool(torch.equal(kv, kv_eager)) and int(Eb[R % 2].item()) == e_eager
    del graph, kv_eager
    t_eager = _back_to_back(torch, verify, 6 * nbuf)
    ctr = [0]

    def verify_next():
        verify(ctr[0])
        ctr[0] += 1
    t_launch, _ = _time_calls(torch, verify_next, 12, inner=6 * nbuf)
    if ver_bytes is None:                       # stochastic: one verify of each buffer, realized bytes
        vb = []
        for i in range(nbuf):
            verify(i)
            m_, e_ = acc.cpu().numpy(), emit.cpu().numpy()
            rowb = sum(8 * V if (e_[b] > m_[b] and m_[b] < k) else (4 * V if e_[b] > m_[b] else 0) for b in range(B))
            vb.append(rowb + 8 * int(sum(min(int(m_[b]) + 1, k) for b in range(B))) + 4 * B * (k + 1) * 2)
        ver_bytes = sum(vb) / nbuf
    rows = B * (k + 1)
    out = {"workload": f"{cfg['name']}: B={B} k={k} V={V} {cfg.get('logit_dtype', 'f32 p/q')}, KV {L}x{H}x{D} {kvdt}, "
                       f"{nbuf} rotating inputs",
           "rows_per_s": rows * steps / wall, "ms_per_step": wall / steps * 1e3,
           "step_timing": "eager launches through the Python binding, host clock around the timed steps "
                          "(for small workloads the host's launch rate bounds it)",
           "rows_per_s_graph": rows / t_graph, "ms_per_step_graph": t_graph * 1e3,
           "step_timing_graph": f"all {R} rounds (warm-up included) captured in one HIP graph from the initial "
                                "state and replayed once, HIP events around the replay",
           "graph_equals_eager": graph_same,
           "verify_us_per_launch": t_launch * 1e6,
           "verify_timing": f"GPU time: {6 * nbuf} calls over the rotating inputs captured in one HIP graph, "
                            "median replay / calls",
           "verify_us_per_launch_eager": t_eager * 1e6, "verify_algorithmic_bytes": ver_bytes,
           "verify_GBps": ver_bytes / t_launch / 1e9, "verify_frac_of_peak": ver_bytes / t_launch / PEAK_HBM,
           "realign_ms_per_call": statistics.mean(t_rea) * 1e3,
           "realign_GBps": sum(rea_bytes) / sum(t_rea) / 1e9,
           "realign_frac_of_peak": sum(rea_bytes) / sum(t_rea) / PEAK_HBM,
           "realign_bytes_per_call": sum(rea_bytes) / len(rea_bytes)}
    # parity guard (outside the timed region): round 0 against the oracle
    verify(0)
    torch.cuda.synchronize()
    r0 = rounds[0]
    if mode == "greedy":
        ref = oracle.greedy_verify(r0["logits"], r0["dtype"], r0["drafts"])
    else:
        ref = oracle.sample_verify(r0["p"], r0["q"], r0["drafts"], r0["uniforms"])
    out["parity_checked"] = bool(np.array_equal(emit.cpu().numpy(), ref["emit_count"]) and
                                 np.array_equal(toks.cpu().numpy(), ref["out_tokens"]))
    del kv
    torch.cuda.empty_cache()
    if cpu:
        out["cpu_baseline"] = _cpu_step(np, oracle, W, c, r0, ref, g)
    return out


def _cpu_step(np, oracle, W, c, r0, ref, g) -> dict:
    """The oracle's verify + commit of one round on the host (median of 3),
    on the workload's full KV (random contents: the oracle's cost does not
    depend on them); at most 4 layers are copied, scaled to all."""
    L, H, D, B, k, n, E, C = (g[x] for x in ("L", "H", "D", "B", "k", "n", "E", "C"))
    tv = []
    for _ in range(3):
        t = time.perf_counter()
        if "p" in r0:
            oracle.sample_verify(r0["p"], r0["q"], r0["drafts"], r0["uniforms"])
        else:
            oracle.greedy_verify(r0["logits"], r0["dtype"], r0["drafts"])
        tv.append(time.perf_counter() - t)
    layers = min(L, 4)
    u = np.uint16 if g["dtype"] == "bf16" else np.uint32
    kv = np.random.default_rng(0).integers(0, 1 << 16, size=(layers, 2, B, H, C, D), dtype=u)
    tr = []
    for _ in range(3):
        t = time.perf_counter()
        oracle.commit_realign(kv, E, n, ref["emit_count"], k)
        tr.append(time.perf_counter() - t)
    step = statistics.median(tv) + statistics.median(tr) * L / layers
    return {"value": B * (k + 1) / step, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"verify of one round's {B * (k + 1)} rows + realign of {layers} of {L} layers scaled to "
                      f"{L}; median of 3; single-threaded numpy"}


def grouped_workload(dev, np, torch, sv, W, batches: int = 4, cpu: bool = True) -> dict:
    """The grouped workload: same-length grouping of the 256-sequence pool,
    then, per batch, stochastic verification (k=4, V=256000, p/q as the
    stochastic workload's) and the realign-based commit of the batch's
    left-padded rectangle (28 layers x 4 KV heads x 128 bf16), each timed on
    its own."""
    import oracle
    cfg = W.workload(4)
    Bm, k, V, mg = cfg["B"], cfg["k"], cfg["V"], cfg["min_group"]
    L, H, D = cfg["L"], cfg["H"], cfg["D"]
    P = W.pool_lengths()
    N = P.size
    i32 = dict(dtype=torch.int32, device=dev)
    lens = torch.as_tensor(P, **i32)
    perm, bs, bl = torch.empty(N, **i32), torch.empty(N + 1, **i32), torch.empty(N, **i32)
    nb, ng = torch.empty(1, **i32), torch.empty(1, **i32)
    t_g, th_g = _time_calls(torch, lambda: sv.spec_group_same_length(lens, Bm, mg, perm, bs, bl, nb, ng), 52)
    perm_h, bs_h, bl_h = perm.cpu().numpy(), bs.cpu().numpy(), bl.cpu().numpy()
    nbat = int(nb.item())
    # batches to time: mixed ones (the realign has something to move), at most `batches`
    chosen = [b for b in range(nbat) if bl_h[b] < 0 and bs_h[b + 1] - bs_h[b] == Bm][:batches]
    acc, emit, toks = torch.empty(Bm, **i32), torch.empty(Bm, **i32), torch.empty(Bm, k + 1, **i32)
    offs, mass = torch.empty(Bm + 1, **i32), torch.empty(Bm, dtype=torch.float64, device=dev)
    ws = sv.workspace(sv.spec_verify_sample_workspace_bytes(Bm, k, V), dev)
    vt, vbytes, rt, rbytes, cpu_t = [], [], [], [], []
    for j, b in enumerate(chosen):
        r = W.sample_round(4, batch=j, B=Bm)
        ins = [torch.from_numpy(r[x]).to(dev) for x in ("p", "q", "drafts", "uniforms")]
        copies = [ins[:2]] + [[ins[0].clone(), ins[1].clone()] for _ in range(2)]     # 3 x 74 MB, rotated
        it = itertools.count()

        def call():
            p_, q_ = copies[next(it) % len(copies)]
            sv.spec_verify_sample(p_, q_, ins[2], ins[3], acc, emit, toks, ws, emit_offsets=offs, final_mass=mass)
        t, _ = _time_calls(torch, call, 12, inner=6)
        m_, e_ = acc.cpu().numpy(), emit.cpu().numpy()
        rowb = sum(8 * V if (e_[q] > m_[q] and m_[q] < k) else (4 * V if e_[q] > m_[q] else 0) for q in range(Bm))
        vt.append(t)
        vbytes.append(rowb + 8 * int(sum(min(int(m_[q]) + 1, k) for q in range(Bm))) + 4 * Bm * (k + 1) * 2)
        # the batch's rectangle: its members' cached rows, right-aligned at the longest
        n = (P[perm_h[bs_h[b]:bs_h[b + 1]]] - 1).astype(np.int64)
        E = int(n.max())
        C = E + (k + 1) * 2
        kv = torch.empty((L, 2, Bm, H, C, D), dtype=torch.bfloat16, device=dev)
        W.fill_kv_torch(kv, E, n, torch.as_tensor(W.prefix_tokens(4, Bm, E + 1), device=dev), "bf16")
        Eb, Eo = torch.tensor([E], **i32), torch.empty(1, **i32)
        Nb, No = torch.as_tensor(n, **i32), torch.empty(Bm, **i32)
        pos, mask = torch.empty(Bm, C, **i32), torch.empty(Bm, C, **i32)
        mv = torch.zeros(1, dtype=torch.int64, device=dev)
        # the same in-place move repeated: every call moves the same ranges
        call = lambda: sv.spec_commit_realign_kv(kv, k, Eb, Nb, emit, Eo, No, pos, mask, bytes_moved=mv)
        t, _ = _time_calls(torch, call, 8, inner=4)
        rt.append(t)
        rbytes.append(int(mv.item()) + 8 * Bm * C)
        if cpu and j == 0:
            ref = oracle.sample_verify(r["p"], r["q"], r["drafts"], r["uniforms"])
            g4 = dict(L=L, H=H, D=D, B=Bm, k=k, n=n, E=E, C=C, dtype="bf16")
            t0 = time.perf_counter()
            oracle.group_same_length(P, Bm, mg)
            tg_cpu = time.perf_counter() - t0
            cpu_t.append((tg_cpu, _cpu_step(np, oracle, W, 4, r, ref, g4)))
        del kv, copies, ins
        torch.cuda.empty_cache()
    out = {"workload": f"{cfg['name']}: pool {N}, batches of {Bm}, min_group {mg}; stochastic verify k={k} V={V} f32 "
                       f"p/q; realign of a mixed batch's rectangle, KV {L}x{H}x{D} bf16",
           "grouping_us": t_g * 1e6, "grouping_us_host": th_g * 1e6, "num_batches": nbat,
           "grouped_fraction": int(ng.item()) / N, "batches_timed": len(chosen),
           "verify_us_per_batch": statistics.mean(vt) * 1e6,
           "verify_GBps": sum(vbytes) / sum(vt) / 1e9, "verify_frac_of_peak": sum(vbytes) / sum(vt) / PEAK_HBM,
           "commit_ms_per_batch": statistics.mean(rt) * 1e3,
           "commit_GBps": sum(rbytes) / sum(rt) / 1e9, "commit_frac_of_peak": sum(rbytes) / sum(rt) / PEAK_HBM}
    if cpu_t:
        tg_cpu, cb = cpu_t[0]
        out["cpu_baseline"] = dict(cb, grouping_us=tg_cpu * 1e6)
    return out


def draft_resync(dev, np, torch, sv, W) -> dict:
    """spec_resync_draft_kv at a small draft model's cache geometry (24 layers,
    2 KV heads, head_dim 64, bf16), 64-token prefixes, k = 4."""
    i32 = dict(dtype=torch.int32, device=dev)
    L, H, D, k, P = 24, 2, 64, 4, 64
    out = {"workload": f"draft-cache re-sync, KV {L}x{H}x{D} bf16, {P}-token prefixes, k={k} (the draft wrote k slots)"}
    for B in (1, 8):
        n = np.full(B, P - 1, np.int64)
        E = P - 1
        C = E + k + 1
        kv = torch.empty((L, 2, B, H, C, D), dtype=torch.bfloat16, device=dev)
        W.fill_kv_torch(kv, E, n, torch.as_tensor(W.prefix_tokens(4, B, E + 1), device=dev), "bf16")
        e = torch.as_tensor(np.arange(B) % (k + 1) + 1, **i32)          # emitted counts 1 .. k+1
        Eb, Eo = torch.tensor([E], **i32), torch.empty(1, **i32)
        Nb, No = torch.as_tensor(n, **i32), torch.empty(B, **i32)
        pos, mask = torch.empty(B, C, **i32), torch.empty(B, C, **i32)
        mv = torch.zeros(1, dtype=torch.int64, device=dev)
        call = lambda: sv.spec_resync_draft_kv(kv, k, Eb, Nb, e, Eo, No, pos_ids=pos, mask=mask, bytes_moved=mv)
        t, th = _time_calls(torch, call, 22)
        out[f"B{B}"] = {"us_per_call": t * 1e6, "us_per_call_host": th * 1e6, "bytes_moved": int(mv.item())}
        del kv
    return out


def policy_loop(dev, np, torch, sv, W, rounds: int = 8) -> dict:
    """EQSPEC against EXSPEC over several rounds on the grouped workload's pool
    at its full KV geometry (28 layers x 4 KV heads x 128 bf16), greedy
    verification of planted drafts (V = 256000 bf16 logits made on the
    device each round), on the drifted pool and on a four-length pool.  Per
    policy: verification calls, KV bytes moved, GPU time of grouping,
    verification and commit, and GPU time per emitted token (the simulated
    forward's slot writes are not timed)."""
    from speculative_decoding_verification_04_amd.scheduler import EqspecPool, ExspecPool
    cfg = W.workload(4)
    L, H, D, V, k, B, mg = cfg["L"], cfg["H"], cfg["D"], cfg["V"], cfg["k"], cfg["B"], cfg["min_group"]
    fw = lambda kv, rows, seq, c0, p0, tk: W.write_rows_torch(kv, rows, seq, c0, p0, tk, "bf16")
    out = {"workload": f"pool 256, batches of {B}, k={k}, {rounds} rounds, greedy verify V={V} bf16, "
                       f"KV {L}x{H}x{D} bf16; EQSPEC: fixed rectangles realigned every round; EXSPEC: ragged "
                       f"caches regrouped every round, same-length batches by a length update, mixed batches "
                       f"by repad / unpad"}
    for kind in ("drifted", "four"):
        pp = W.policy_pool(kind)
        N, P = pp["N"], pp["P"]
        rng = np.random.default_rng(7)
        tokens = [list(rng.integers(0, V, size=int(x))) for x in P]
        T = np.zeros((N, int(P.max()) + 1), np.int64)
        for s in range(N):
            T[s, :len(tokens[s])] = tokens[s]
        T_d = torch.as_tensor(T).to(dev)
        Cs = int((P - 1).max()) + (k + 1) * (rounds + 1)
        gen = torch.Generator(device=dev).manual_seed(11)
        alpha = torch.as_tensor(pp["alpha"], device=dev, dtype=torch.float32)
        res = {}
        for name in ("eqspec", "exspec"):
            if name == "eqspec":
                pol = EqspecPool(torch, tokens, L, H, D, "bf16", k, B, Cs, V, dev,
                                 lambda kv, E, nn, seq: W.fill_kv_torch(kv, E, nn, T_d[torch.as_tensor(seq).to(dev)],
                                                                        "bf16", seq=seq))
            else:
                pol = ExspecPool(torch, tokens, L, H, D, "bf16", k, B, mg, Cs, V, dev,
                                 lambda pool, nn: W.fill_kv_torch(pool, nn, nn, T_d, "bf16"))
            gen.manual_seed(11)
            tot = dict(verify_calls=0, bytes_moved=0, emitted=0, mixed_batches=0, grouped=0)
            times = {}
            for r in range(rounds):
                z = (torch.randn((N, k + 1, V), device=dev, generator=gen) * 2).to(torch.bfloat16)
                am = z[:, :k].float().argmax(-1).to(torch.int32)
                other = torch.randint(0, V, (N, k), device=dev, generator=gen, dtype=torch.int32)
                keep = torch.rand((N, k), device=dev, generator=gen) < alpha[:, None]
                dr = torch.where(keep, am, torch.where(other == am, (other + 1) % V, other)).contiguous()
                st = pol.round(z, dr, dr.cpu().numpy(), fw)
                tot["verify_calls"] += st["verify_calls"]
                tot["bytes_moved"] += st["bytes_moved"]
                tot["emitted"] += int(st["emit_count"].sum())
                tot["mixed_batches"] += st.get("mixed_batches", 0)
                tot["grouped"] += st.get("num_grouped", 0)
                for kk, v in st["times"].items():
                    times[kk] = times.get(kk, 0.0) + v
                del z
            gpu = sum(times.values())
            res[name] = dict(tot, **{f"{kk}_ms": v * 1e3 for kk, v in times.items()},
                             gpu_ms=gpu * 1e3, gpu_ms_per_emitted_token=gpu * 1e3 / tot["emitted"],
                             commit_GBps=tot["bytes_moved"] / times.get("commit", 1e-30) / 1e9)
            del pol
            torch.cuda.empty_cache()
        res["grouping_rate"] = res["exspec"]["grouped"] / (N * rounds)
        out[kind] = res
    return out


def batch_scaling(dev, np, torch, sv, W) -> dict:
    """How the commit's cost and the grouping rate move with batch size.

    Realign: the bench workload's per-sequence geometry (prefixes 512-4096,
    8 KV heads x 128 bf16) with 4 layers instead of 32 (bytes scale with the
    layer count; the trend does not), 8 chained rounds per batch size with
    synthetic emitted counts from the workload's acceptance law.  Grouping: a
    pool of 256 with the grouped workload's drifted lengths, and a pool of 256
    drawn from 4 lengths only (a near-identical-length subset).
    """
    c, Lr, R = 3, 4, 8
    cfg = W.workload(c)
    k, H, D = cfg["k"], cfg["H"], cfg["D"]
    i32 = dict(dtype=torch.int32, device=dev)
    rows = []
    for B in (1, 2, 4, 8, 16, 32):
        g = W.kv_geometry(c, rounds=R, B=B)
        n, E, C = g["n"], g["E"], g["C"]
        kv = torch.empty((Lr, 2, B, H, C, D), dtype=torch.bfloat16, device=dev)
        W.fill_kv_torch(kv, E, n, torch.as_tensor(W.prefix_tokens(c, B, E + 1), device=dev), "bf16")
        Eb = [torch.tensor([E], **i32), torch.empty(1, **i32)]
        Nb = [torch.as_tensor(n, **i32), torch.empty(B, **i32)]
        pos, mask = torch.empty(B, C, **i32), torch.empty(B, C, **i32)
        moved = torch.zeros(R, dtype=torch.int64, device=dev)
        es = [torch.as_tensor(W.accept_counts(c, r, B), **i32) for r in range(R)]
        torch.cuda.synchronize()
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for r in range(R):
            sv.spec_commit_realign_kv(kv, k, Eb[r % 2], Nb[r % 2], es[r], Eb[(r + 1) % 2], Nb[(r + 1) % 2],
                                      pos, mask, bytes_moved=moved[r:r + 1])
        b_.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b_) * 1e-3 / R
        mv = moved.cpu().numpy().astype(np.float64)
        pad = float(np.mean([np.mean(e.max() - e) for e in (x.cpu().numpy() for x in es)]))
        rows.append({"B": B, "bytes_moved_per_round": float(mv.mean()),
                     "bytes_moved_per_sequence": float(mv.mean() / B),
                     "padding_columns_per_sequence": pad, "ms_per_round": t * 1e3,
                     "GBps": float(mv.mean()) / t / 1e9 if mv.mean() > 0 else 0.0})
        del kv
    torch.cuda.empty_cache()
    P = W.pool_lengths()
    same = W.stream(4, "pool", 99).choice(np.array([512, 513, 900, 1500]), size=P.size)
    grouping = []
    for B in (2, 4, 8, 16, 32):
        out = {"B": B}
        for name, lens in (("drifted_pool", P), ("four_lengths_pool", same)):
            L = torch.as_tensor(lens, **i32)
            N = L.numel()
            perm, bs, bl = torch.empty(N, **i32), torch.empty(N + 1, **i32), torch.empty(N, **i32)
            nb, ng = torch.empty(1, **i32), torch.empty(1, **i32)
            for tag, mg in (("2", 2), ("B", B)):   # partial same-length batches allowed / full batches only
                sv.spec_group_same_length(L, B, mg, perm, bs, bl, nb, ng)
                out[f"{name}_min_group_{tag}"] = int(ng.item()) / N
        grouping.append(out)
    return {"realign_vs_batch": {"workload": f"bench geometry with {Lr} layers, {R} rounds per batch size",
                                 "rows": rows,
                                 # (k+1) - E[e], E[e] = (1 - a^(k+1)) / (1 - a) averaged over the workload's a_b
                                 "padding_limit_columns": float((k + 1) - np.mean(
                                     (1 - W.alphas(c) ** (k + 1)) / (1 - W.alphas(c))))},
            "grouping_rate_vs_batch": grouping}


def cpu_baseline(r0: dict, ref_verify: dict, g: dict, np) -> dict:
    """The oracle as it stands, on the host: verify of all rows of one round
    plus the realign of two of the cache's layers, scaled to all layers."""
    import oracle
    L, H, D, B, k, n, E, C = (g[x] for x in ("L", "H", "D", "B", "k", "n", "E", "C"))
    rows = B * (k + 1)
    tv = []
    for _ in range(3):
        t = time.perf_counter()
        oracle.greedy_verify(r0["logits"], "bf16", r0["drafts"])
        tv.append(time.perf_counter() - t)
    layers = 2
    kv = np.random.default_rng(0).integers(0, 1 << 16, size=(layers, 2, B, H, C, D), dtype=np.uint16)
    tr = []
    for _ in range(3):
        t = time.perf_counter()
        oracle.commit_realign(kv, E, n, ref_verify["emit_count"], k)
        tr.append(time.perf_counter() - t)
    step = statistics.median(tv) + statistics.median(tr) * L / layers
    return {"value": rows / step, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"verify of all {rows} rows of one round + realign of {layers} of {L} layers "
                      f"scaled x{L // layers}; median of 3; single-threaded numpy",
            "host_cpus": os.cpu_count(), "host_model": _cpu_model()}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    sys.exit(main())
