"""bench.py's measurement plumbing on the CPU: the rocprofv3 summaries it writes from
counter and kernel-statistics CSV files, the traffic it reads back (and refuses when the
kernel sources or the workload differ), and the one-GPU guard."""
import argparse
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

N215 = 215_000_000


def _counter_csv(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, counter, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def _pmc_args(tmp_path, out):
    upd = "void nz1::flat_update_kernel<1, 0>(nz1::FlatSpan, unsigned int const*)"
    copy = "void at::native::MulFunctor<float>(float)"
    _counter_csv(tmp_path / "f", [(upd, "FETCH_SIZE", 1000.0), (upd, "FETCH_SIZE", 1002.0),
                                  ("void nz1::norm_kernel<1>()", "FETCH_SIZE", 5.0)])
    _counter_csv(tmp_path / "w", [(upd, "WRITE_SIZE", 3000.0), (upd, "WRITE_SIZE", 3000.0)])
    _counter_csv(tmp_path / "cf", [(copy, "FETCH_SIZE", 512.0)])      # 1 MiB read, counted as 512 KiB
    _counter_csv(tmp_path / "cw", [(copy, "WRITE_SIZE", 1024.0)])
    return argparse.Namespace(pmc_fetch=str(tmp_path / "f"), pmc_write=str(tmp_path / "w"),
                              pmc_copy_fetch=str(tmp_path / "cf"),
                              pmc_copy_write=str(tmp_path / "cw"), copy_bytes=1 << 20,
                              workload="neox20b_shard_215m", out=str(out))


def test_pmc_summary_and_traffic_readback(tmp_path, monkeypatch, capsys):
    out = tmp_path / "summary.txt"
    bench.summarize_pmc(_pmc_args(tmp_path, out))
    text = out.read_text()
    vals = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and not line.startswith("#"))
    assert vals["kernel"] == "nz1::flat_update_kernel<1, 0>"
    assert float(vals["fetch_kib_per_dispatch"]) == 1001.0 and vals["update_dispatches"] == "2"
    assert float(vals["copy_factor_fetch"]) == 2.0 and float(vals["copy_factor_write"]) == 1.0
    want = 1024.0 * (1001.0 * 2.0 + 3000.0 * 1.0)
    assert float(vals["traffic_bytes_per_dispatch"]) == round(want)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    os.replace(out, bench.pmc_summary("neox20b_shard_215m", "flat_update_kernel"))
    assert bench.read_traffic("neox20b_shard_215m", N215) == want
    assert bench.read_traffic("tiny_1m", 1 << 20) is None              # no summary for it
    # a summary filed under another workload's or kernel's name is not used
    os.replace(bench.pmc_summary("neox20b_shard_215m", "flat_update_kernel"),
               bench.pmc_summary("tiny_1m", "flat_update_kernel"))
    assert bench.read_traffic("tiny_1m", 1 << 20) is None
    os.replace(bench.pmc_summary("tiny_1m", "flat_update_kernel"),
               bench.pmc_summary("neox20b_shard_215m", "update_kernel"))
    assert bench.read_traffic("neox20b_shard_215m", N215, "update_kernel") is None
    os.replace(bench.pmc_summary("neox20b_shard_215m", "update_kernel"),
               bench.pmc_summary("neox20b_shard_215m", "flat_update_kernel"))
    assert bench.read_traffic("neox20b_shard_215m", N215) == want
    monkeypatch.setattr(bench, "kernel_sha", lambda: "0" * 64)
    assert bench.read_traffic("neox20b_shard_215m", N215) is None      # other kernel sources


def test_pmc_summary_needs_the_update_kernel(tmp_path):
    args = _pmc_args(tmp_path, tmp_path / "s.txt")
    _counter_csv(tmp_path / "w", [("void nz1::norm_kernel<1>()", "WRITE_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(args)


def test_trace_summary(tmp_path):
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "t_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                          "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow(dict(Name="void nz1::flat_update_kernel<1, 0>(nz1::FlatSpan)", Calls=43,
                        TotalDurationNs=43 * 1_050_000, AverageNs=1_050_000.0, Percentage=90,
                        MinNs=1_000_000, MaxNs=1_100_000, StdDev=1))
        w.writerow(dict(Name="void nz1::norm_kernel<1>(nz1::Chunk const*)", Calls=43,
                        TotalDurationNs=43 * 66_000, AverageNs=66_000.0, Percentage=6,
                        MinNs=60_000, MaxNs=70_000, StdDev=1))
        w.writerow(dict(Name="void at::native::normal_kernel()", Calls=5, TotalDurationNs=10,
                        AverageNs=2.0, Percentage=0, MinNs=1, MaxNs=3, StdDev=0))
    log = tmp_path / "bench.log"
    log.write_text("[bench] noise\n" + json.dumps({"ms_per_step": 1.12, "kernel_avg_ms": {
        "norm": 0.066, "finalize": 0.005, "update": 1.05}}) + "\n")
    out = tmp_path / "trace.txt"
    bench.summarize_trace(argparse.Namespace(trace=str(d), workload="neox20b_shard_215m",
                                             trace_steps=20, bench_log=str(log), out=str(out)))
    text = out.read_text()
    assert "normal_kernel" not in text
    assert f"nz1::flat_update_kernel: {28 * N215} algorithmic bytes per launch / 1050.0 us" in text
    assert f"= {28 * N215 / 1050e-6 / 1e9:.1f} GB/s" in text
    assert f"nz1::norm_kernel: {2 * N215} algorithmic bytes per launch / 66.0 us" in text
    assert "update avg 1050.0 us" in text and "step 1120.0 us wall" in text


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_summaries_record_extra_bench_flags(tmp_path):
    """A profile taken with extra bench flags (e.g. --chunked-update) states them in the
    commands its header gives, so the summary names the run that reproduces it."""
    args = _pmc_args(tmp_path, tmp_path / "s.txt")
    args.bench_flags = "--chunked-update"
    bench.summarize_pmc(args)
    head = [ln for ln in (tmp_path / "s.txt").read_text().splitlines() if ln.startswith("#")]
    assert any("--no-extra-workloads --chunked-update" in ln for ln in head)
    assert any("--bench-flags='--chunked-update'" in ln for ln in head)
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "t_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                          "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow(dict(Name="void nz1::update_kernel<1, 2, 0>(nz1::Chunk const*)", Calls=23,
                        TotalDurationNs=23, AverageNs=1.0, Percentage=90, MinNs=1, MaxNs=1,
                        StdDev=0))
    out = tmp_path / "trace.txt"
    bench.summarize_trace(argparse.Namespace(trace=str(d), workload="neox20b_shard_215m",
                                             trace_steps=10, bench_log=None, out=str(out),
                                             bench_flags="--chunked-update"))
    text = out.read_text()
    assert ("--steps 10 --warmup 3 --no-cpu-baseline --skip-steps 0 --no-ceiling "
            "--no-extra-workloads --chunked-update") in text
    assert "+ 10 steps" in text and "--trace-steps 10" in text


def test_sgd_summary_is_kept_apart(tmp_path, monkeypatch):
    """A counter summary of the momentum-SGD step (20 B/param, its own file name) is read
    for SGD runs only, and an AdamW summary never serves an SGD run."""
    args = _pmc_args(tmp_path, tmp_path / "s.txt")
    args.bench_flags = "--optimizer sgd"
    bench.summarize_pmc(args)
    vals = dict(line.split(": ", 1) for line in (tmp_path / "s.txt").read_text().splitlines()
                if ": " in line and not line.startswith("#"))
    assert vals["optimizer"] == "sgd" and vals["algorithmic_bytes_per_dispatch"] == str(20 * N215)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    sgd_path = bench.pmc_summary("neox20b_shard_215m", "flat_update_kernel", "sgd")
    assert sgd_path.endswith("flat_update_kernel_sgd_neox20b_shard_215m_pmc.txt")
    os.replace(tmp_path / "s.txt", sgd_path)
    want = 1024.0 * (1001.0 * 2.0 + 3000.0 * 1.0)
    assert bench.read_traffic("neox20b_shard_215m", N215, "flat_update_kernel", "sgd") == want
    assert bench.read_traffic("neox20b_shard_215m", N215, "flat_update_kernel") is None
    # an AdamW summary filed under the SGD name is refused
    args.bench_flags = ""
    bench.summarize_pmc(args)
    os.replace(tmp_path / "s.txt", sgd_path)
    assert bench.read_traffic("neox20b_shard_215m", N215, "flat_update_kernel", "sgd") is None


def test_skipped_step_timing_restores_the_gradient(monkeypatch):
    """bench.time_skipped_steps plants an inf at gradient element 0, runs the skipped steps
    (two untimed, K timed, K with events), restores the element, and refuses a run in
    which the steps were not skipped.  A fake library stands in for the GPU here."""
    import torch
    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)
    grad = torch.full((16,), 3.0, dtype=torch.float16)

    class FakeState:
        def __init__(self, skipped, last):
            self.skipped_total, self.last_skipped = skipped, last

    class FakeLib:
        def __init__(self, skips):
            self.skips, self.skipped, self.events = skips, 0, None

        def neox_scaler_state(self, h):
            return FakeState(self.skipped, 1 if self.skipped else 0)

        def neox_zero1_timing_begin(self, h, k):
            self.events = k

        def neox_zero1_timing_end(self, h):
            return [0.06 * self.events, 0.004 * self.events, 0.02 * self.events], self.events

    def make_step(lib):
        def step():
            assert torch.isinf(grad[0]) and grad[1] == 3.0      # the inf is in place
            if lib.skips:
                lib.skipped += 1
        return step

    lib = FakeLib(skips=True)
    ms, kernels = bench.time_skipped_steps(lib, 0, grad, make_step(lib), 5, events=True)
    assert lib.skipped == 2 + 5 + 5 and ms >= 0.0
    assert kernels == pytest.approx({"norm": 0.06, "finalize": 0.004, "update": 0.02})
    assert torch.equal(grad, torch.full((16,), 3.0, dtype=torch.float16))   # restored
    lib = FakeLib(skips=False)
    with pytest.raises(AssertionError):
        bench.time_skipped_steps(lib, 0, grad, make_step(lib), 3, events=False)


def test_split_step_timing_writes_the_local_slot(monkeypatch):
    """bench.time_split_steps: step_local writes into the rank array at the rank's slot,
    step_apply gets the whole array and the rank count every step, the other slots are
    filled once, and a skipped split step is refused.  A fake library stands in for the
    GPU here."""
    import torch
    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)

    class FakeLib:
        def __init__(self, skip):
            self.calls, self.skip, self.skipped = [], skip, 0

        def neox_zero1_step_local(self, h, ptr, stream):
            self.calls.append(("local", ptr))
            self.local_ptr = ptr
            # the library writes 2.0 at ptr
            self.array.view(-1)[(ptr - self.array.data_ptr()) // 8] = 2.0

        def neox_zero1_step_apply(self, h, ptr, lr, stream, nranks):
            self.calls.append(("apply", ptr, nranks))
            if self.skip:
                self.skipped += 1

        def neox_scaler_state(self, h):
            class S:
                pass
            st = S()
            st.skipped_total = self.skipped
            return st

    real_zeros = torch.zeros

    def zeros(*a, **k):
        t = real_zeros(*a, **k)
        lib.array = t
        return t

    monkeypatch.setattr(torch, "zeros", zeros)
    lib = FakeLib(skip=False)
    ms = bench.time_split_steps(lib, 0, 1e-3, 0, 4, ranks=8, rank=3, device="cpu")
    assert ms >= 0.0
    base = lib.array.data_ptr()
    assert lib.calls[0] == ("local", base + 24)
    assert lib.calls[1:] == [("local", base + 24), ("apply", base, 8)] * 7
    assert float(lib.array[3]) == 2.0
    assert torch.allclose(lib.array[[0, 7]], torch.tensor([1.8, 2.2], dtype=torch.float64))
    lib = FakeLib(skip=True)
    with pytest.raises(AssertionError):
        bench.time_split_steps(lib, 0, 1e-3, 0, 2, ranks=4, rank=0, device="cpu")


def test_stall_summary_table(tmp_path):
    """bench.summarize_stalls: per-kernel averages of the memory-side counters, turned into
    the duration, effective clock, latencies (LEVEL / REQ), requests in flight (LEVEL /
    cycles) and credit-stall percentages the table reports; torch kernels are left out."""
    upd = "void nz1::flat_update_kernel<1, 0>(nz1::FlatSpan, unsigned int const*)"
    cpy = "void (anonymous namespace)::copy_kernel<true>(unsigned int __vector(4) const*)"
    torch_k = "void at::native::vectorized_elementwise_kernel<4, at::native::float16_copy_kernel_cuda>()"
    vals = {  # per dispatch
        upd: dict(GRBM_GUI_ACTIVE=8 * 2_000_000, TCC_EA0_RDREQ_sum=1000, TCC_EA0_RDREQ_LEVEL_sum=2_000_000,
                  TCC_EA0_WRREQ_sum=500, TCC_EA0_WRREQ_LEVEL_sum=250_000,
                  TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum=128 * 20_000,
                  TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum=128 * 40_000,
                  TCP_TCC_READ_REQ_LATENCY_sum=3000, TCP_TCC_READ_REQ_sum=10,
                  TCC_HIT_sum=3, TCC_MISS_sum=1),
        cpy: dict(GRBM_GUI_ACTIVE=8 * 500_000, TCC_EA0_RDREQ_sum=10, TCC_EA0_RDREQ_LEVEL_sum=50,
                  TCC_EA0_WRREQ_sum=10, TCC_EA0_WRREQ_LEVEL_sum=20,
                  TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum=0, TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum=0,
                  TCP_TCC_READ_REQ_LATENCY_sum=100, TCP_TCC_READ_REQ_sum=1, TCC_HIT_sum=1, TCC_MISS_sum=1),
        torch_k: dict(GRBM_GUI_ACTIVE=1.0),
    }
    d = tmp_path / "stalls" / "p1"
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for k, cs in vals.items():
            dur = 1_000_000 if k == upd else 200_000           # ns: 2.0 and 2.5 GHz
            for c, v in cs.items():
                w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v,
                            "Start_Timestamp": 10, "End_Timestamp": 10 + dur})
    with open(d / "run_agent_info.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Agent_Type", "Num_Xcc"])
        w.writeheader()
        w.writerow({"Agent_Type": "CPU", "Num_Xcc": 1})
        w.writerow({"Agent_Type": "GPU", "Num_Xcc": 8})
    out = tmp_path / "stalls.txt"
    bench.summarize_stalls(argparse.Namespace(stalls=str(tmp_path / "stalls"),
                                              workload="neox20b_shard_215m", out=str(out)))
    rows = {ln.split()[0]: ln.split() for ln in out.read_text().splitlines()
            if ln.startswith(("nz1::", "copy_kernel"))}
    assert set(rows) == {"nz1::flat_update_kernel<1,", "copy_kernel<true>"}
    u = rows["nz1::flat_update_kernel<1,"][2:]          # after the split name
    # n, us, GHz, rd_req, wr_req, rd_lat, rd_infl, wr_lat, wr_infl, rdstl%, wrstl%, tcp, hit
    assert u[0] == "1" and float(u[1]) == 1000.0 and float(u[2]) == 2.0
    assert float(u[5]) == 2000 and float(u[6]) == 1 and float(u[7]) == 500
    assert float(u[9]) == 1.0 and float(u[10]) == 2.0 and float(u[11]) == 300 and float(u[12]) == 75.0
    assert "GRBM_GUI_ACTIVE" in out.read_text() and "rocprofv3 --pmc" in out.read_text()


def test_windowed_cpu_baseline_covers_runs_and_the_whole_norm():
    """The windowed CPU step (used for the 6e9 shard): every run lies inside one segment
    with that segment's decay flag, every segment's ends are covered, and the squared
    norm streamed piece by piece on several threads is the oracle's scan of the whole
    gradient up to summation order."""
    import numpy as np

    import bench
    import workloads as W
    from oracle import oracle as O
    w = W.Workload("windowed", 9, [(300_000, True), (5, False), (1_000_000, True),
                                   (9_000, False)], W.Hyper(), steps=1)
    g = W.host_grads(w, 0, w.hyper.init_scale)
    runs = bench.windowed_runs(w, windows=6, win=50_000, edge=512)
    starts = np.cumsum([0] + [k for k, _ in w.segments])
    for a, k, d in runs:
        seg = int(np.searchsorted(starts, a, side="right")) - 1
        assert k >= 1 and a + k <= starts[seg + 1] and d == w.segments[seg][1]
    covered = {(a, k) for a, k, _ in runs}
    for s, (n, _) in zip(starts, w.segments):
        if n <= 1024:
            assert (int(s), n) in covered
        else:
            assert (int(s), 512) in covered and (int(s) + n - 512, 512) in covered
    assert len(runs) == 2 * 3 + 1 + 6

    calls = []

    def fetch(lo, k):
        calls.append(k)
        return g[lo:lo + k]

    scan_s, upd_s, n_upd, d, sumsq = bench.oracle_windowed_step(w, fetch, runs, threads=3,
                                                                piece=100_000)
    assert max(calls) <= 100_000 and sum(calls[:14]) == w.numel
    cfg, st = bench._oracle_config(w)
    inv, inv32 = O.unscale_factor(cfg, st)
    want, of = O.scan(cfg.dtype, g, inv, inv32)
    assert of == 0 and abs(sumsq - want) <= 1e-12 * want
    assert d.skip == 0 and n_upd == sum(k for _, k, _ in runs)
    assert scan_s > 0 and upd_s > 0


def test_committed_profiles_were_taken_on_the_current_kernels():
    """Every rocprofv3 summary under profiles/ records the hash of the kernel sources it
    was taken on; all of them must match the sources in the tree."""
    import glob
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt")))
    assert paths
    want = bench.kernel_sha()
    for p in paths:
        with open(p) as f:
            shas = [line.split(":", 1)[1].strip() for line in f
                    if line.startswith("kernel_source_sha256:")]
        assert shas == [want], (os.path.basename(p), shas)
