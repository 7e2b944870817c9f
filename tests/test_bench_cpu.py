"""bench.py's host logic on the CPU: the one-GPU guard, the rocprofv3 kernel
trace and counter summaries (on synthetic CSV files of rocprofv3's columns),
and the digest gate that keeps a stale counter record out of the bench line."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

HEAD = "void xsymv::symv_strip<float, false, 16, 1, 16, true, 256, false>(xsymv::StripArgs<float>)"
MERGE = "void xsymv::symv_strip_merge<float, 16, false>(xsymv::StripMergeArgs<float>)"
OTHER = "void xsymv::symv_strip<double, true, 16, 1, 16, true, 256, false>(xsymv::StripArgs<double>)"
SHARD = "void xsymv::symv_strip<float, false, 16, 1, 16, true, 256, true>(xsymv::StripArgs<float>)"


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_message(argv, env):
    r = subprocess.run([sys.executable, "bench.py", *argv], cwd=ROOT, capture_output=True,
                       text=True, timeout=120, env={**os.environ, **env})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def write_csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_trace_summary_runs_and_headline(tmp_path):
    """Launch order: the headline kernel (5 launches of 100 us, each followed
    by a merge), another workload, the headline's kernel and grid again for a
    later workload (3 x 200 us), then a kernel launched more often than the
    headline's (10 x 50 us).  The runs table keeps the two runs of the same
    kernel and grid apart, and the headline section takes the first kernel
    launched, not the most launched one."""
    trace, t = [], 0

    def launch(name, grid, us):
        nonlocal t
        trace.append({"Kernel_Name": name, "Grid_Size_X": grid, "Workgroup_Size_X": 1024,
                      "Start_Timestamp": t, "End_Timestamp": t + int(us * 1000)})
        t += int(us * 1000) + 500

    for _ in range(5):
        launch(HEAD, 262144, 100)
        launch(MERGE, 32768, 7)
    for _ in range(2):
        launch(OTHER, 262144, 600)
    for _ in range(3):
        launch(HEAD, 262144, 200)
        launch(MERGE, 32768, 7)
    for _ in range(10):
        launch(SHARD, 262144, 50)
    stats = []
    for name in (HEAD, MERGE, OTHER, SHARD):
        d = [(r["End_Timestamp"] - r["Start_Timestamp"]) for r in trace if r["Kernel_Name"] == name]
        stats.append({"Name": name, "Calls": len(d), "TotalDurationNs": sum(d),
                      "AverageNs": sum(d) / len(d), "MinNs": min(d), "MaxNs": max(d)})
    write_csv(tmp_path / "trace.csv", trace)
    write_csv(tmp_path / "stats.csv", stats)
    md = bench.summarize_trace(str(tmp_path / "trace.csv"), str(tmp_path / "stats.csv"),
                               "rocprofv3 ... -- python3 bench.py --steps 2 --warmup 1")
    runs = [line for line in md.splitlines() if line.startswith("| ") and "`" in line
            and line.split("|")[1].strip().isdigit()]
    got = [(int(r.split("|")[1]), r.split("|")[2].strip().strip("`"), int(r.split("|")[5]),
            float(r.split("|")[6])) for r in runs]
    assert got == [(0, HEAD[:90], 5, 100.0), (1, OTHER[:90], 2, 600.0),
                   (2, HEAD[:90], 3, 200.0), (3, SHARD[:90], 10, 50.0)]
    head = md.split("## Headline workload")[1]
    # warmup + 2 * steps = 5 launches of the first kernel launched
    assert f"The first 5 launches of `{HEAD[:90]}`: mean 100.0 us" in head


def pmc_rows(values):
    """Dispatch rows of a --pmc-workloads run: per workload `calls` streaming
    launches (each followed by a merge, whose readings must be ignored), then
    the calibration kernel; values[k] = the k-th workload's streaming
    readings (FETCH, WRITE)."""
    neg = "void at::native::vectorized_elementwise_kernel<neg_kernel_cuda>(...)"
    fetch, write, did = [], [], 0
    for (fv, wv) in values:
        for _ in range(bench.PMC_CALLS):
            for name, f, w in ((HEAD, fv, wv), (MERGE, 9.0e6, 100.0)):
                did += 1
                fetch.append({"Dispatch_Id": did, "Kernel_Name": name, "Grid_Size": 262144,
                              "Counter_Value": f})
                write.append({"Dispatch_Id": did, "Kernel_Name": name, "Grid_Size": 262144,
                              "Counter_Value": w})
    did += 1
    fetch.append({"Dispatch_Id": did, "Kernel_Name": neg, "Grid_Size": 4096,
                  "Counter_Value": 524288.0})
    write.append({"Dispatch_Id": did, "Kernel_Name": neg, "Grid_Size": 4096,
                  "Counter_Value": 1048576.0})
    return fetch, write


def test_counter_summary_scales_by_the_calibration_kernel(tmp_path):
    """FETCH_SIZE reads 524288 KiB and WRITE_SIZE 1048576 KiB for the 1 GiB
    calibration kernel (scales 2 and 1); each workload's streaming launches
    are scaled by them, in launch order, and the merge kernels are left out."""
    from blas_symmetric_mat_amd import roofline as R
    vals = [(1000000.0 + k, 4000.0 + k) for k in range(len(bench.PMC_WORKLOADS))]
    fetch, write = pmc_rows(vals)
    fetch.reverse()  # the summary orders dispatches by id
    write_csv(tmp_path / "f.csv", fetch)
    write_csv(tmp_path / "w.csv", write)
    out = bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "cmd")
    assert list(out) == bench.PMC_WORKLOADS
    for k, name in enumerate(bench.PMC_WORKLOADS):
        rec = out[name]
        assert rec["kernel"] == HEAD
        assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
        assert rec["fetch_bytes_per_launch"] == (1000000 + k) * 1024 * 2
        assert rec["write_bytes_per_launch"] == (4000 + k) * 1024
        assert rec["bytes_per_launch"] == (1000000 + k) * 2048 + (4000 + k) * 1024
        prec, n = name[0], int(name.split("-")[2][1:])
        assert rec["algorithmic_bytes_per_launch"] == R.tile_kernel_bytes(prec, n)
        assert rec["launches"] == bench.PMC_CALLS and rec["grid_threads"] == 262144
        assert rec["kernel_source_digest"] == bench.kernel_source_digest()


def test_counter_summary_needs_every_launch_and_the_calibration_kernel(tmp_path):
    vals = [(1.0, 1.0)] * len(bench.PMC_WORKLOADS)
    fetch, write = pmc_rows(vals)
    write_csv(tmp_path / "f.csv", fetch[:-1])
    write_csv(tmp_path / "w.csv", write[:-1])
    with pytest.raises(ValueError, match="calibration"):
        bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "cmd")
    write_csv(tmp_path / "f.csv", fetch[2:])
    write_csv(tmp_path / "w.csv", write[2:])
    with pytest.raises(ValueError, match="streaming launches"):
        bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "cmd")


def test_profile_workload_names():
    from blas_symmetric_mat_amd import workloads as W

    class P:
        pass
    for name in bench.PMC_WORKLOADS:
        parts = name.split("-")
        q = P()
        q.prec, q.uplo, q.n = parts[0], parts[1], int(parts[2][1:])
        q.lda = next((int(x[3:]) for x in parts[3:] if x.startswith("lda")), q.n)
        q.beta = 0.0 if "beta0" in parts else 1.0
        assert bench.workload_key(q) == name
    assert bench.workload_key(W.dsymv_upper_n8192_lda8200_beta0()) == "d-U-n8192-lda8200-beta0"
    for bad in ("x-L-n10", "s-Q-n10", "s-L-10", "s-L-n10-foo"):
        with pytest.raises(SystemExit):
            bench.profile_problem(bad)


def test_traffic_record_only_for_current_source_and_configuration(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.traffic_record("ssymv-L-n32768", "cfg") is None  # no file
    rec = {"kernel_config": "cfg", "kernel_source_digest": bench.kernel_source_digest(),
           "bytes_per_launch": 5}
    path.write_text(json.dumps({"ssymv-L-n32768": rec}))
    assert bench.traffic_record("ssymv-L-n32768", "cfg")["bytes_per_launch"] == 5
    assert bench.traffic_record("ssymv-L-n32768", "another cfg") is None
    assert bench.traffic_record("dsymv-L-n32768", "cfg") is None
    path.write_text(json.dumps({"ssymv-L-n32768": {**rec, "kernel_source_digest": "0" * 16}}))
    assert bench.traffic_record("ssymv-L-n32768", "cfg") is None



def test_call_breakdown(tmp_path):
    """A --profile-workload --calls 3 --flush run: 2 warm-up calls (no gap),
    3 mode-1 calls and 3 mode-2 calls (a 5 us gap before the merge) and 3
    calls of the per-call protocol (no gap), flush kernels between them, then
    two layouts of the read probe.  The breakdown keeps the four groups
    apart, takes kernel, gap, merge and span per group, the fastest probe
    layout, and quotes what the timings measured."""
    from blas_symmetric_mat_amd import roofline as R
    kern = "void xsymv::symv_strip<double, true, 16, 1, 8, true, 256, false>(xsymv::StripArgs<double>)"
    merge = "void xsymv::symv_strip_merge<double, 16, false, 32>(xsymv::StripMergeArgs<double>)"
    fill = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>(...)"
    probe4 = "void read_probe<4>(unsigned int __vector(4) const*, long long, unsigned int*)"
    probe8 = "void read_probe<8>(unsigned int __vector(4) const*, long long, unsigned int*)"
    trace, t = [], 0

    def launch(name, grid, wg, us, gap=0.0):
        nonlocal t
        trace.append({"Kernel_Name": name, "Grid_Size_X": grid, "Workgroup_Size_X": wg,
                      "Start_Timestamp": t, "End_Timestamp": t + int(us * 1000)})
        t += int(us * 1000) + int(gap * 1000)

    for _ in range(2):
        launch(kern, 262144, 1024, 54.0)
        launch(merge, 262144, 1024, 5.0)
    for gap in (5.0, 5.0, 0.0):
        for _ in range(3):
            launch(fill, 1 << 26, 256, 150.0)
            launch(kern, 262144, 1024, 47.0, gap=gap)
            launch(merge, 262144, 1024, 4.0)
        if gap == 0.0:
            launch(fill, 1 << 26, 256, 150.0)  # flush alone
    for _ in range(4):
        launch(probe4, 2048 * 256, 256, 42.0)
        launch(probe8, 2048 * 256, 256, 40.0)
    write_csv(tmp_path / "trace.csv", trace)
    (tmp_path / "ev.json").write_text(json.dumps({
        "calls": 3, "kernel_us_median": 51.0, "call_us_median": 58.5,
        "call_us_differential": 51.5, "flush_us_median": 450.0}))
    name = "d-U-n8192-lda8200-beta0"
    md = bench.summarize_calls(str(tmp_path / "trace.csv"), name,
                               f"rocprofv3 ... -- python3 bench.py --profile-workload {name} "
                               "--calls 3 --flush --read-probe",
                               events_json=str(tmp_path / "ev.json"))
    assert "| warm-up, no timing, no flush | 2 | 54.0 | 0.0 | 5.0 | 59.0 |" in md
    assert "| flushed, events bound to each kernel (mode 1) | 3 | 47.0 | 5.0 | 4.0 | 56.0 |" in md
    assert "| flushed, events bound to the call (mode 2) | 3 | 47.0 | 5.0 | 4.0 | 56.0 |" in md
    assert "| flushed, no library events (per-call protocol) | 3 | 47.0 | 0.0 | 4.0 | 51.0 |" in md
    kb = R.tile_kernel_bytes("d", 8192)
    assert f"the kernel moves {kb / 47.0 / 1e3:.0f} GB/s" in md
    assert "Fastest layout: 40.0 us; the streaming kernel (last group) takes 1.175 x that." in md
    assert "flush 450.0 us), 51.5 us." in md


def test_call_ms_differential_protocol(monkeypatch):
    """call_ms on a simulated clock: (flush + call) - (flush alone) gives the
    call's own time; without a flush, calls back to back over their count; a
    call lost in the flush falls back to more pairs, then to the events'
    whole-call span."""
    import torch
    clock = {"t": 0.0}

    class Ev:
        def __init__(self, enable_timing=True):
            self.t = None

        def record(self):
            self.t = clock["t"]

        def synchronize(self):
            pass

        def elapsed_time(self, other):
            return other.t - self.t

    monkeypatch.setattr(torch.cuda, "Event", Ev)
    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)

    def flush():
        clock["t"] += 0.45

    class D:
        def __init__(self, ms):
            self.ms = ms

        def call(self):
            clock["t"] += self.ms

    c, f = bench.call_ms(D(0.054), 20, flush)
    assert abs(c - 0.054) < 1e-9 and abs(f - 0.45) < 1e-9
    c, f = bench.call_ms(D(0.33), 20)
    assert abs(c - 0.33) < 1e-9 and f is None
    seen = []
    monkeypatch.setattr(bench, "time_kernels",
                        lambda d, reps, fl=None, mode=1: seen.append(mode) or [(0.06, 0.0)] * reps)
    c, f = bench.call_ms(D(0.0), 20, flush)
    assert seen == [2] and abs(c - 0.06) < 1e-9


@pytest.mark.parametrize("passes", [1, 2, 3])
def test_rule_check_averages_every_pass(monkeypatch, passes):
    """The rule check averages each configuration's medians over all the
    autotuner passes it asked for, whatever their number."""
    import blas_symmetric_mat_amd as X
    # configuration 1 is the built-in choice; per pass, configuration 0 is
    # faster in the first pass only, configuration 2 on average
    times = [[1.0, 2.0, 1.5], [3.0, 2.0, 1.5], [3.0, 2.0, 1.5]]
    calls = []

    def autotune(prec, uplo, n, reps=20, lda=None):
        calls.append((prec, uplo, n, reps, lda))
        return 0, list(times[len(calls) - 1])

    monkeypatch.setattr(X, "clear_config", lambda: None)
    monkeypatch.setattr(X, "current_config", lambda prec, uplo, n, lda: 1)
    monkeypatch.setattr(X, "autotune", autotune)
    out = bench.rule_check([("s", "L", 4096)], reps=7, passes=passes)
    assert calls == [("s", "L", 4096, 7, 4096)] * passes
    avg = [sum(t[i] for t in times[:passes]) / passes for i in range(3)]
    best = min(range(3), key=lambda i: avg[i])
    assert out == {"s-L-n4096": [round(avg[1] / avg[best], 4), 1, best]}
