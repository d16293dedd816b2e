#!/usr/bin/env python3
"""Throughput of the ZeRO-1 mixed-precision Adam step on one MI355X.

One step = the whole hot path on the shard: norm/overflow pass, finalize, fused
unscale + clip + AdamW + cast update.  Inputs are synthetic and already resident in
HBM.  Prints one JSON line:
  value     params/s over the timed steps (wall clock between synchronizations);
            ms_per_step_median / ms_per_step_min from per-step dispatch events
  hbm       the step's algorithmic bytes (30 B/param) and their rate against 8 TB/s
  roofline  the update kernel (the dominant one): algorithmic bytes per launch over its
            average duration from HIP events its own dispatch stamps, against 8 TB/s,
            and against a plain copy timed on the same GPU (frac_of_copy);
            traffic = HBM bytes per launch from the committed rocprofv3 counter summary
            of this workload and kernel (null when there is none for the current sources)
  kernel_avg_ms  norm / finalize / update durations (a short all-kernel pass after)
  split_step     the step a data-parallel rank runs (step_local, step_apply over 96
                 ranks' values; the exchange between them is not timed)
  skipped_step   the cost of a step with an inf in the gradient (timed last)
  probes    a plain copy and a kernel with the update's access pattern and trivial
            arithmetic, swept over launch shapes, on this GPU right after the timed steps
  workloads the 6e9-parameter OPT-style shard and the 5,000-tensor layout, each with its
            own timing, roofline and kernel split
  cpu_baseline  the CPU oracle on the host's cores (all threads, static contiguous
            pieces, per-thread double partials added in thread order) and on one thread,
            on the whole shard; the smaller shards in full, the 5,000-tensor layout in
            full and the 6e9 shard windowed; the host's CPU count, model and memory
Other modes: --summarize-trace / --summarize-pmc write the profiles/ summaries from
rocprofv3 output; --copy-probe-only is the counters' calibration copy.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
UPDATE_BYTES_PER_PARAM = 28      # grad 2 + master/m/v 12 read; master/m/v 12 + half 2 written
SGD_UPDATE_BYTES_PER_PARAM = 20  # momentum SGD keeps no second moment
STEP_BYTES_PER_PARAM = 30        # + the norm pass's 2-byte gradient read
# the sources that fix the kernels' code and launch shapes
KERNEL_SRCS = tuple(os.path.join(ROOT, "mixed_precision_zero_amd", "csrc", f)
                    for f in ("zero1_kernels.hip", "zero1_internal.h", "zero1_api.hip"))
PROFILES = os.path.join(ROOT, "profiles")


PYTHIA_RANKS = {f"pythia410m_dp8_rank{r}": r for r in (0, 1)}


def workload_names():
    import workloads as W
    return sorted(list(W.BENCH_WORKLOADS) + list(PYTHIA_RANKS))


def make_workload(name, partition="library"):
    """The named workload; a Pythia-410M rank takes its segments from the library's ZeRO-1
    partition (partition="oracle": the oracle's, for the CPU baseline)."""
    import workloads as W
    if name in PYTHIA_RANKS:
        t = W.pythia410m_tensors()
        numel, decay = [n for n, _ in t], [d for _, d in t]
        r = PYTHIA_RANKS[name]
        if partition == "oracle":
            from oracle import oracle as O
            segs, _ = O.partition(numel, decay, 8, r, 64)
            return W.pythia410m(r, [(g["numel"], g["flags"]) for g in segs])
        import mixed_precision_zero_amd as Z
        segs, _ = Z.neox_zero1_partition(numel, decay, 8, r, 64)
        return W.pythia410m(r, [(g.numel, g.flags) for g in segs])
    if name not in W.BENCH_WORKLOADS:
        sys.exit(f"unknown workload {name}; one of {workload_names()}")
    return W.BENCH_WORKLOADS[name]()


def pmc_summary(workload, kernel, optimizer="adamw"):
    """The committed counter summary of one update kernel on one workload."""
    tag = "" if optimizer == "adamw" else f"_{optimizer}"
    return os.path.join(PROFILES, f"{kernel}{tag}_{workload}_pmc.txt")


def flags_optimizer(args):
    """The optimizer a profiled run used, from the bench flags it recorded."""
    fl = getattr(args, "bench_flags", "") or ""
    return "sgd" if re.search(r"--optimizer[ =]sgd", fl) else "adamw"


def update_bytes(optimizer):
    return SGD_UPDATE_BYTES_PER_PARAM if optimizer == "sgd" else UPDATE_BYTES_PER_PARAM


def kernel_sha():
    h = hashlib.sha256()
    for p in KERNEL_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic(workload, n, kernel="flat_update_kernel", optimizer="adamw"):
    """HBM bytes per launch of the update kernel `kernel` from the committed rocprofv3 PMC
    summary for this workload and optimizer, scaled by its copy-kernel calibration
    factors; None if there is none, or it was taken on other kernel code, workload,
    kernel or optimizer."""
    path = pmc_summary(workload, kernel, optimizer)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    try:
        if vals.get("kernel_source_sha256") != kernel_sha() or vals.get("workload") != workload:
            return None
        if kernel not in re.findall(r"nz1::(\w+)<", vals.get("kernel", "")):
            return None
        if vals.get("optimizer", "adamw") != optimizer:
            return None
        return 1024.0 * (float(vals["fetch_kib_per_dispatch"]) * float(vals["copy_factor_fetch"])
                         + float(vals["write_kib_per_dispatch"]) * float(vals["copy_factor_write"]))
    except (KeyError, ValueError):
        return None


def bench_flags_arg(args):
    """The --bench-flags argument as it appears in a summary's own command line."""
    fl = getattr(args, "bench_flags", "")
    return f" --bench-flags='{fl}'" if fl else ""


def summarize_trace(args):
    """Write the kernel-time summary (profiles/...) from a rocprofv3 --kernel-trace --stats
    run of this program, with the algorithmic bandwidth of the step's kernels and, given
    that run's bench log, the HIP-event averages bench.py measured in the same process."""
    import csv
    import glob

    files = glob.glob(os.path.join(args.trace, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {args.trace}")
    with open(files[0]) as fh:
        rows = [r for r in csv.DictReader(fh) if "nz1::" in r["Name"]]
    n = make_workload(args.workload).numel
    flags = f" {args.bench_flags}" if getattr(args, "bench_flags", "") else ""
    per_param = {"update_kernel": update_bytes(flags_optimizer(args)), "norm_kernel": 2}
    lines = [
        f"# rocprofv3 kernel trace of the ZeRO-1 step on {args.workload} ({n} params), MI355X (gfx950).",
        "# Commands (from the repository root, on an MI355X):",
        f"#   rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o trace -- python3 bench.py "
        f"--workload {args.workload} --steps {args.trace_steps} --warmup 3 --no-cpu-baseline --skip-steps 0 "
        f"--no-ceiling --no-extra-workloads{flags} > <log>",
        f"#   python3 bench.py --summarize-trace <dir> --workload {args.workload} "
        f"--trace-steps {args.trace_steps} --bench-log <log>{bench_flags_arg(args)}",
        f"# Calls = 3 warm-up + {args.trace_steps} timed steps (update-kernel events only) + "
        f"{args.trace_steps} steps",
        "# with events around every kernel (a shard whose norm pass has at most 256 blocks has no",
        "# finalize launch); the torch kernels that draw the synthetic inputs are left out.  Durations in ns.",
        f"kernel_source_sha256: {kernel_sha()}",
        f"{'kernel':44s} {'calls':>6s} {'avg_ns':>10s} {'min_ns':>10s} {'max_ns':>10s}",
    ]
    rates = []
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].replace("void ", "").split("(")[0]
        lines.append(f"{name:44s} {int(r['Calls']):6d} {float(r['AverageNs']):10.0f} "
                     f"{int(r['MinNs']):10d} {int(r['MaxNs']):10d}")
        for k, bpp in per_param.items():
            if name.split("<")[0].endswith(k):
                us = float(r["AverageNs"]) / 1e3
                rates.append(f"{name.split('<')[0]}: {bpp * n} algorithmic bytes per launch / "
                             f"{us:.1f} us = {bpp * n / (us * 1e-6) / 1e9:.1f} GB/s")
    lines += [""] + rates
    if args.bench_log:
        with open(args.bench_log) as fh:
            last = [ln for ln in fh if ln.startswith("{")][-1]
        b = json.loads(last)
        k = b.get("kernel_avg_ms", {})
        lines.append(f"bench.py in the same run (dispatch-stamped HIP events): update avg "
                     f"{k.get('update', 0) * 1e3:.1f} us, norm {k.get('norm', 0) * 1e3:.1f} us, "
                     f"finalize {k.get('finalize', 0) * 1e3:.1f} us, step "
                     f"{b['ms_per_step'] * 1e3:.1f} us wall")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text, end="")


def summarize_pmc(args):
    """Write the traffic summary bench.py reads (profiles/...) from rocprofv3 --pmc
    output: FETCH_SIZE and WRITE_SIZE of the update kernel, each scaled by what the same
    counter reads for a plain streaming copy of known size (--copy-probe-only run)."""
    import csv
    import glob

    def rows(d):
        out = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                out += list(csv.DictReader(fh))
        if not out:
            raise SystemExit(f"no counter_collection.csv under {d}")
        return out

    names = set()

    def avg(d, counter, name_part):
        sel = [r for r in rows(d) if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]]
        if not sel:
            raise SystemExit(f"no {counter} rows for kernels matching {name_part!r} in {d}")
        if name_part == "update_kernel":
            names.update(r["Kernel_Name"].replace("void ", "").split("(")[0] for r in sel)
        return sum(float(r["Counter_Value"]) for r in sel) / len(sel), len(sel)

    fetch, nf = avg(args.pmc_fetch, "FETCH_SIZE", "update_kernel")
    write, nw = avg(args.pmc_write, "WRITE_SIZE", "update_kernel")
    cfetch, _ = avg(args.pmc_copy_fetch, "FETCH_SIZE", "MulFunctor")
    cwrite, _ = avg(args.pmc_copy_write, "WRITE_SIZE", "MulFunctor")
    known_kib = args.copy_bytes / 1024.0
    ff, fw = known_kib / cfetch, known_kib / cwrite
    n = make_workload(args.workload).numel
    traffic = (fetch * ff + write * fw) * 1024.0
    flags = f" {args.bench_flags}" if getattr(args, "bench_flags", "") else ""
    opt = flags_optimizer(args)
    bpp = update_bytes(opt)
    lines = [
        f"# HBM traffic of the update on {args.workload} ({n} params), from rocprofv3 PMC.",
        "# Commands (from the repository root, on an MI355X):",
        f"#   rocprofv3 --pmc FETCH_SIZE --kernel-include-regex 'nz1::' -d <fetch_dir> --output-format csv "
        f"-- python3 bench.py --workload {args.workload} --steps 5 --warmup 1 --no-cpu-baseline "
        f"--no-timing-events --skip-steps 0 --no-ceiling --no-extra-workloads{flags}",
        "#   rocprofv3 --pmc WRITE_SIZE -d <write_dir> ... (same program)",
        f"#   rocprofv3 --pmc FETCH_SIZE --kernel-include-regex 'MulFunctor' -d <copy_fetch_dir> "
        f"--output-format csv -- python3 bench.py --copy-probe-only {args.copy_bytes}",
        "#   rocprofv3 --pmc WRITE_SIZE -d <copy_write_dir> ... (same program)",
        f"#   python3 bench.py --summarize-pmc --workload {args.workload} --copy-bytes "
        f"{args.copy_bytes} --pmc-fetch <fetch_dir> --pmc-write <write_dir> "
        f"--pmc-copy-fetch <copy_fetch_dir> --pmc-copy-write <copy_write_dir>{bench_flags_arg(args)}",
        "# The copy probe reads and writes copy_bytes once per dispatch; its counter readings",
        "# give the factors that turn counter KiB into bytes.  Counters count traffic leaving",
        "# the L2 (Infinity Cache hits included).",
        f"workload: {args.workload}",
        f"optimizer: {opt}",
        f"kernel: {', '.join(sorted(names))}",
        f"kernel_source_sha256: {kernel_sha()}",
        f"update_dispatches: {nf}",
        f"fetch_kib_per_dispatch: {fetch:.1f}",
        f"write_kib_per_dispatch: {write:.1f}",
        f"copy_bytes: {args.copy_bytes}",
        f"copy_fetch_kib_per_dispatch: {cfetch:.1f}",
        f"copy_write_kib_per_dispatch: {cwrite:.1f}",
        f"copy_factor_fetch: {ff:.5f}",
        f"copy_factor_write: {fw:.5f}",
        f"traffic_bytes_per_dispatch: {traffic:.0f}",
        f"algorithmic_bytes_per_dispatch: {bpp * n}",
        f"traffic_over_algorithmic: {traffic / (bpp * n):.4f}",
    ]
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text, end="")


# per pass: at most 4 TCC, 4 TCP and 2 GRBM counters (one hardware pass each)
STALL_PASSES = (
    "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum TCC_EA0_WRREQ_STALL_sum GRBM_GUI_ACTIVE",
    "TCC_EA0_RDREQ_LEVEL_sum TCC_EA0_WRREQ_LEVEL_sum TCC_EA0_RDREQ_sum TCC_EA0_WRREQ_sum",
    "TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_WRITE_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum TCP_TCC_WRITE_REQ_sum",
    "TCC_BUSY_sum TCC_TAG_STALL_sum TCP_PENDING_STALL_CYCLES_sum GRBM_GUI_ACTIVE",
    "TCC_EA0_RDREQ_DRAM_sum TCC_EA0_WRREQ_DRAM_sum TCC_HIT_sum TCC_MISS_sum",
)
# gfx950: 8 XCDs of 16 L2 channels each
L2_CHANNELS = 128


def _kernel_key(name):
    return name.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0]


def summarize_stalls(args):
    """The memory-side counter table of the step's kernels next to the copy and access-
    pattern probes, from the rocprofv3 --pmc runs of STALL_PASSES (one sub-directory per
    pass under args.stalls): duration, effective shader clock, L2-to-memory request
    counts, latencies and requests in flight, credit stalls."""
    import csv
    import glob
    rows = {}
    durs = {}
    nxcc = 8
    for f in sorted(glob.glob(os.path.join(args.stalls, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                k = _kernel_key(r["Kernel_Name"])
                if not (k.startswith("nz1::") or "copy_kernel<" in k and "at::" not in k
                        or k.startswith("pattern_kernel")):
                    continue
                rows.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    durs.setdefault(k, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    for f in glob.glob(os.path.join(args.stalls, "**", "*agent_info.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Agent_Type") == "GPU":
                    nxcc = int(r["Num_Xcc"])
    if not rows:
        raise SystemExit(f"no step or probe kernels in counter files under {args.stalls}")
    lines = [
        "# Memory-side counters of the step's kernels and of the bandwidth probes, MI355X (gfx950).",
        "# Commands (from the repository root, on an MI355X), one run per counter pass:",
    ]
    for i, ps in enumerate(STALL_PASSES):
        lines.append(f"#   rocprofv3 --pmc {ps} -d <dir>/p{i + 1} --output-format csv -- python3 bench.py "
                     f"--workload {args.workload} --steps 3 --warmup 1 --no-cpu-baseline "
                     f"--no-timing-events --skip-steps 0 --no-extra-workloads")
    lines += [
        f"#   python3 bench.py --summarize-stalls <dir> --workload {args.workload}",
        "# Per dispatch (averages).  cycles = GRBM_GUI_ACTIVE / XCDs; clock = cycles / duration.",
        "# rd/wr req: L2-to-memory requests (TCC_EA0_*REQ_sum); B/req = algorithmic bytes / requests",
        "# (update kernels only).  lat = LEVEL_sum / REQ_sum (cycles a request waits for memory);",
        "# inflight = LEVEL_sum / cycles (chip-wide requests outstanding, x B/req = bytes in flight).",
        f"# stall% = credit-stall channel-cycles / (cycles x {L2_CHANNELS} L2 channels).",
        "# tcp_rd_lat = TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum (CU to L2 round trip).",
        f"kernel_source_sha256: {kernel_sha()}",
        f"{'kernel':34s} {'n':>4s} {'us':>8s} {'GHz':>6s} {'rd_req':>9s} {'wr_req':>9s} "
        f"{'rd_lat':>7s} {'rd_infl':>8s} {'wr_lat':>7s} {'wr_infl':>8s} {'rdstl%':>7s} {'wrstl%':>7s} "
        f"{'tcp_rd_lat':>10s} {'L2hit%':>7s}",
    ]
    def a(c, k):
        v = c.get(k)
        return sum(v) / len(v) if v else float("nan")
    for k in sorted(rows, key=lambda x: (not x.startswith("nz1::"), x)):
        c = rows[k]
        cyc = a(c, "GRBM_GUI_ACTIVE") / nxcc
        us = sum(durs[k]) / len(durs[k]) / 1e3 if k in durs else float("nan")
        rd, wr = a(c, "TCC_EA0_RDREQ_sum"), a(c, "TCC_EA0_WRREQ_sum")
        rl, wl = a(c, "TCC_EA0_RDREQ_LEVEL_sum"), a(c, "TCC_EA0_WRREQ_LEVEL_sum")
        hit, miss = a(c, "TCC_HIT_sum"), a(c, "TCC_MISS_sum")
        lines.append(
            f"{k[:34]:34s} {len(durs.get(k, [])):4d} {us:8.1f} {cyc / (us * 1e3):6.3f} {rd:9.0f} {wr:9.0f} "
            f"{rl / rd:7.0f} {rl / cyc:8.0f} {wl / wr:7.0f} {wl / cyc:8.0f} "
            f"{100 * a(c, 'TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum') / (cyc * L2_CHANNELS):7.2f} "
            f"{100 * a(c, 'TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum') / (cyc * L2_CHANNELS):7.2f} "
            f"{a(c, 'TCP_TCC_READ_REQ_LATENCY_sum') / a(c, 'TCP_TCC_READ_REQ_sum'):10.0f} "
            f"{100 * hit / (hit + miss):7.1f}")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text, end="")


def copy_probe(nbytes):
    """A plain streaming copy of known size for counter calibration: reads and writes
    nbytes once per dispatch, three dispatches."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(f"[bench] copy probe: 3 x {nbytes} bytes", file=sys.stderr, flush=True)


# threads per block x vectors per thread / blocks per CU (0 = unlimited) / non-temporal
# stores
PATTERN_SHAPES = ((256, 2, 0, 0), (256, 2, 1, 0), (256, 1, 1, 0), (128, 2, 2, 0),
                  (256, 2, 1, 1), (256, 1, 1, 1), (256, 1, 2, 1), (128, 2, 2, 1), (64, 2, 4, 1))


def measure_ceiling(bufs, n, reps=20):
    """GB/s of the stream probes on the workload's own arrays (contents are clobbered)."""
    import torch

    from mixed_precision_zero_amd import probe as P
    stream = torch.cuda.current_stream()
    ptr = {k: t.data_ptr() for k, t in bufs.items()}

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps

    # the pattern at several launch shapes (threads, vectors per thread, blocks per CU);
    # the ceiling is the best of them
    sweep = {}
    for t, u, c, nts in PATTERN_SHAPES:
        ms = timed(lambda: P.neox_probe_update_pattern(ptr["grad"], ptr["half"], ptr["master"],
                                                       ptr["m"], ptr["v"], n, t, u, c, nts,
                                                       stream.cuda_stream))
        sweep[f"{t}x{u}/cu{c}" + ("/nt" if nts else "")] = \
            UPDATE_BYTES_PER_PARAM * n / (ms * 1e-3) / 1e9
    best = max(sweep, key=sweep.get)
    copy = max(8 * n / (timed(lambda: P.neox_probe_copy(ptr["master"], ptr["m"], 4 * n, nts,
                                                        stream.cuda_stream)) * 1e-3) / 1e9
               for nts in (0, 1))
    return {"update_pattern_gbps": sweep[best], "update_pattern_shape": best,
            "update_pattern_sweep": {k: round(v, 1) for k, v in sweep.items()},
            "copy_gbps": copy}


def host_info():
    """The host the CPU baseline ran on: logical CPUs, the ones this process may use, the
    CPU model and the RAM."""
    info = {"nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": None, "ram_gb": None}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    info["ram_gb"] = round(int(line.split()[1]) / 2 ** 20, 1)
                    break
    except OSError:
        pass
    return info


# the machine's CPU share for one GPU: at most this many oracle threads
CPU_THREADS_MAX = 16


def _oracle_config(w):
    """The oracle's configuration and initial scaler for workload w."""
    from oracle import oracle as O
    h = w.hyper
    cfg = O.Config(beta1=h.beta1, beta2=h.beta2, eps=h.eps, weight_decay=h.weight_decay,
                   clip_norm=h.clip_norm, predivide_factor=h.predivide_factor,
                   dp_world_size=h.dp_world_size, dtype=h.dtype, scaler_mode=h.scaler_mode,
                   growth_interval=h.growth_interval, growth_factor=h.growth_factor,
                   backoff_factor=h.backoff_factor, min_scale=h.min_scale,
                   optimizer=h.optimizer)
    return cfg, O.Scaler(loss_scale=h.init_scale)


def _oracle_setup(w, n=None):
    """Host inputs of workload w (its first n params) for the oracle: config, scaler and
    the segment list over freshly drawn arrays (the step-0 gradient)."""
    import workloads as W

    n = w.numel if n is None else min(n, w.numel)
    segs, left = [], n
    for k, d in w.segments:
        if left == 0:
            break
        segs.append((min(k, left), d))
        left -= segs[-1][0]
    st0 = W.host_init(w, n=n)
    g = W.host_grads(w, 0, w.hyper.init_scale, n=n)
    h = w.hyper
    cfg, scaler = _oracle_config(w)
    osegs, off = [], 0
    for k, d in segs:
        sl = slice(off, off + k)
        osegs.append(dict(grad=g[sl], half=st0["half"][sl], master=st0["master"][sl],
                          m=st0["m"][sl], v=None if h.optimizer else st0["v"][sl], decay=d))
        off += k
    return cfg, scaler, osegs, n


def _time_oracle(cfg, st, segs, n, threads, budget_s, max_steps):
    """Steps of the oracle as it stands (one thread: its own whole-step routine; more:
    its routines over static contiguous pieces, partials added in thread order) until
    the budget is spent; returns (params/s, steps, seconds)."""
    import numpy as np

    from oracle import oracle as O
    lr = np.float32(6e-4)
    spent, steps = 0.0, 0
    while steps < 1 or (spent < budget_s and steps < max_steps):
        t0 = time.perf_counter()
        if threads == 1:
            O.step(cfg, st, lr, segs)
        else:
            O.step_parallel(cfg, st, lr, segs, threads)
        spent += time.perf_counter() - t0
        steps += 1
    return n * steps / spent, steps, spent


def cpu_baseline(w, budget_s=10.0, dev=None):
    """The CPU oracle on this host: the bench workload in full, on all the cores this
    process may use (up to the box's share) and on one thread, plus the two small
    workloads on all cores and on one thread; with dev, also the two large workloads (the 5,000-tensor
    shard in full, the 6e9 shard windowed), their inputs drawn on that device.  Inputs
    follow each workload's recipe (seeded host draws unless stated)."""
    info = host_info()
    threads = max(1, min(CPU_THREADS_MAX, info["affinity_cpus"]))
    cfg, st, segs, n = _oracle_setup(w)
    rate_t, steps_t, sec_t = _time_oracle(cfg, st, segs, n, threads, budget_s / 2, 20)
    # the same arrays, carried on: every step does the same work whatever their values
    rate_1, steps_1, sec_1 = _time_oracle(cfg, st, segs, n, 1, budget_s, 3)
    del segs
    small = {}
    for name in ("tiny_1m", "pythia410m_dp8_rank0"):
        sw = make_workload(name, partition="oracle")
        c, s2, sg, k = _oracle_setup(sw)
        r, ns, sec = _time_oracle(c, s2, sg, k, threads, 1.0, 20)
        r1, ns1, sec1 = _time_oracle(c, s2, sg, k, 1, 1.0, 20)
        small[name] = {"value": r, "params": k, "steps": ns, "seconds": round(sec, 2),
                       "cores": threads,
                       "single_thread": {"value": r1, "steps": ns1, "seconds": round(sec1, 2),
                                         "cores": 1}}
    large = {}
    if dev is not None:
        for name, fn in (("multi_tensor_5000_bf16", cpu_multi_tensor_in_full),
                         ("opt_style_6b", cpu_opt_style_windowed)):
            print(f"[bench] cpu baseline (oracle): {name}", file=sys.stderr, flush=True)
            try:
                large[name] = fn(dev, threads)
            except Exception as e:      # a reported baseline: never lose the bench line to it
                large[name] = {"error": repr(e)}
    what = (f"{w.name} in full ({n} params, {len(w.segments)} segments), step-0 gradient; "
            f"all-core: {steps_t} steps on {threads} threads in {sec_t:.1f} s (static contiguous "
            f"pieces, per-thread double partial sums added in thread order); one thread: "
            f"{steps_1} steps in {sec_1:.1f} s; fp64 scalar C, gcc -O2")
    return {"value": rate_t, "unit": "params/s", "cores": threads, "kind": "oracle",
            "sample": what,
            "gbps": STEP_BYTES_PER_PARAM * rate_t / 1e9,
            "single_thread": {"value": rate_1, "cores": 1, "steps": steps_1,
                              "seconds": round(sec_1, 2),
                              "gbps": STEP_BYTES_PER_PARAM * rate_1 / 1e9},
            "other_workloads_in_full": small,
            **({"large_workloads": large} if large else {}),
            "host": info}


def _host_bits(t):
    """Host (numpy) copy of a CUDA tensor; 16-bit formats as their uint16 bits."""
    import numpy as np
    import torch
    a = t.cpu()
    return a.view(torch.int16).numpy().view(np.uint16) if a.element_size() == 2 else a.numpy()


def cpu_multi_tensor_in_full(dev, threads, budget_s=5.0):
    """The oracle on all cores over the whole 5,000-tensor shard (1e9 params): the
    step-0 inputs drawn by the workload's seeded device generators and copied to host
    memory, then whole steps as for the bench workload."""
    import gc

    import torch
    w = make_workload("multi_tensor_5000_bf16")
    keep, _ = alloc_shard(w, dev, sgd=False)
    segs = [dict(grad=_host_bits(a["grad"]), half=_host_bits(a["half"]),
                 master=_host_bits(a["master"]), m=_host_bits(a["m"]), v=_host_bits(a["v"]),
                 decay=decay) for a, (_, decay) in zip(keep, w.segments)]
    del keep
    gc.collect()
    torch.cuda.empty_cache()
    cfg, st = _oracle_config(w)
    rate, steps, sec = _time_oracle(cfg, st, segs, w.numel, threads, budget_s, 3)
    return {"value": rate, "unit": "params/s", "params": w.numel, "segments": len(w.segments),
            "steps": steps, "seconds": round(sec, 2), "cores": threads,
            "gbps": STEP_BYTES_PER_PARAM * rate / 1e9,
            "sample": "in full: device-drawn step-0 inputs copied to host, whole steps on all "
                      "cores (static contiguous pieces, thread-order partial sums)"}


def windowed_runs(w, windows=64, win=1 << 20, edge=4096, seed=7):
    """The elements the windowed CPU update covers: `windows` seeded windows of `win`
    elements (each clipped to the end of the segment it starts in) and the first and last
    `edge` elements of every segment.  Returns (start, length, decay) runs in shard order;
    runs may overlap one another."""
    import numpy as np
    sizes = [k for k, _ in w.segments]
    starts = np.concatenate([[0], np.cumsum(sizes)])
    runs = []
    for k, (n, d) in enumerate(w.segments):
        s0 = int(starts[k])
        if n <= 2 * edge:
            runs.append((s0, n, d))
        else:
            runs.append((s0, edge, d))
            runs.append((s0 + n - edge, edge, d))
    rng = np.random.default_rng([w.wid, seed])
    for a in rng.integers(0, max(1, w.numel - win), size=windows):
        k = int(np.searchsorted(starts, a, side="right")) - 1
        end = min(int(a) + win, int(starts[k + 1]))
        runs.append((int(a), end - int(a), w.segments[k][1]))
    return sorted(runs)


def oracle_windowed_step(w, fetch, runs, threads, piece=1 << 28):
    """One oracle step of workload w timed the windowed way: the squared norm over the
    whole gradient, streamed through a host buffer `piece` elements at a time
    (fetch(lo, k, out) fills out[:k] with the gradient's bits [lo, lo + k); each piece
    is scanned on `threads` threads, partials added in thread order), one decision, then
    the update of the given runs on `threads` threads.  fetch(lo, k) returns the
    gradient's bits [lo, lo + k) as a uint16 array (k <= piece) that stays valid until the
    next call.  Only the oracle's calls are timed.  Returns (scan seconds, update seconds,
    updated params, decision, squared norm)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from oracle import oracle as O
    cfg, st = _oracle_config(w)
    inv, inv32 = O.unscale_factor(cfg, st)
    n = w.numel
    sumsq, of, scan_s = 0.0, 0, 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for lo in range(0, n, piece):
            k = min(piece, n - lo)
            buf = fetch(lo, k)
            cut = [k * p // threads for p in range(threads + 1)]
            t0 = time.perf_counter()
            parts = list(ex.map(lambda p: O.scan(cfg.dtype, buf[cut[p]:cut[p + 1]], inv, inv32),
                                range(threads)))
            scan_s += time.perf_counter() - t0
            for s_, o_ in parts:
                sumsq += s_
                of |= o_
        d = O.decide(cfg, st, of, sumsq)
        # the runs' inputs: the gradient from the shard, a fresh step-0 state of the
        # workload's recipe (master ~ N(0, sigma), half = cast(master), m = v = 0)
        rng = np.random.default_rng([w.wid, 8])
        work = []
        for a, k, decay in runs:
            g = np.array(fetch(a, k), copy=True)
            master = (rng.standard_normal(k) * w.master_sigma).astype(np.float32)
            work.append(dict(grad=g, half=O.float_to_half(cfg.dtype, master), master=master,
                             m=np.zeros(k, np.float32), v=np.zeros(k, np.float32), decay=decay))
        # longest runs first, each to the least-loaded thread
        groups, load = [[] for _ in range(threads)], [0] * threads
        for r in sorted(work, key=lambda r: -r["grad"].size):
            t = load.index(min(load))
            groups[t].append(r)
            load[t] += r["grad"].size
        lr = np.float32(w.hyper.lr)

        def update_group(group):
            for r in group:
                O.update(cfg, d, lr, r["grad"], r["half"], r["master"], r["m"], r["v"],
                         r["decay"])

        t0 = time.perf_counter()
        list(ex.map(update_group, groups))
        upd_s = time.perf_counter() - t0
    return scan_s, upd_s, sum(k for _, k, _ in runs), d, sumsq


def cpu_opt_style_windowed(dev, threads):
    """The oracle on the 6e9-param OPT-style shard, windowed (its 108 GB of host arrays
    and tens of minutes of single-core work are out of a bench run's reach): the norm over
    the whole device-drawn step-0 gradient, the update on seeded windows, and the step
    time estimated as norm time + update time scaled to the whole shard."""
    import gc

    import torch

    import workloads as W
    w = make_workload("opt_style_6b")
    dt = torch.float16 if w.hyper.dtype == W.F16 else torch.bfloat16
    grad = torch.empty(w.numel, dtype=dt, device=dev)
    W.device_grads_(w, grad, 0, w.hyper.init_scale)
    piece = min(1 << 28, w.numel)
    pinned = torch.empty(piece, dtype=dt, pin_memory=True)
    pinned_bits = pinned.view(torch.int16).numpy().view("uint16")

    def fetch(lo, k):
        pinned[:k].copy_(grad[lo:lo + k])      # synchronous device-to-host copy
        return pinned_bits[:k]

    runs = windowed_runs(w)
    try:
        scan_s, upd_s, n_upd, d, _ = oracle_windowed_step(w, fetch, runs, threads, piece)
    finally:
        del grad, pinned
        gc.collect()
        torch.cuda.empty_cache()
    n = w.numel
    est = scan_s + upd_s * n / n_upd
    return {"value": n / est, "unit": "params/s", "params": n, "segments": len(w.segments),
            "cores": threads, "windowed": True,
            "norm_pass": {"params": n, "seconds": round(scan_s, 2),
                          "params_per_s": n / scan_s},
            "update": {"params": n_upd, "runs": len(runs), "seconds": round(upd_s, 3),
                       "params_per_s": n_upd / upd_s},
            "estimated_step_s": round(est, 2), "skipped": bool(d.skip),
            "gbps": STEP_BYTES_PER_PARAM * n / est / 1e9,
            "sample": "windowed: squared norm over the whole device-drawn step-0 gradient "
                      "(copied to host in 2^28-element pieces, copies not timed), update on 64 "
                      "seeded 1M-element windows plus every segment's first and last 4K "
                      "elements; value = params / (norm time + update time scaled to the "
                      "whole shard)"}


def time_skipped_steps(Z, h, grad, one_step, steps, events):
    """Steps whose gradient holds an inf at element 0: the norm pass still reads the whole
    gradient, the finalize decides to skip, and the update's blocks read the decision and
    return.  Returns wall ms per step and, with events, the per-kernel averages.  The
    element is restored afterwards; the handle's scaler state keeps the skips."""
    import torch

    before = Z.neox_scaler_state(h).skipped_total
    saved = grad[0:1].clone()
    grad[0:1].fill_(float("inf"))
    one_step()
    one_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    kernels = None
    if events:
        Z.neox_zero1_timing_begin(h, steps)
        for _ in range(steps):
            one_step()
        sums, k = Z.neox_zero1_timing_end(h)
        kernels = {"norm": sums[0] / k, "finalize": sums[1] / k, "update": sums[2] / k}
    st = Z.neox_scaler_state(h)
    grad[0:1].copy_(saved)
    torch.cuda.synchronize()
    done = 2 + steps + (steps if events else 0)
    assert st.skipped_total - before == done and st.last_skipped == 1, "steps were not skipped"
    return ms, kernels


# Data-parallel ranks of the GPT-NeoX-20B run that the 215M shard is one of (20.6e9 / 96).
SPLIT_RANKS = 96


def time_split_steps(Z, h, lr, stream, steps, ranks=SPLIT_RANKS, rank=0, device="cuda"):
    """The step a data-parallel rank runs: step_local, the exchange of the ranks' squared
    norms, step_apply over all `ranks` values.  The exchange itself needs other GPUs and
    is left out: step_local writes the local value straight into its slot of the rank
    array, and the other ranks' slots hold fixed values near it.  Returns wall ms per
    step over `steps` steps after 3 untimed ones; asserts that none was skipped."""
    import torch

    r = torch.zeros(ranks, dtype=torch.float64, device=device)
    slot = r.data_ptr() + 8 * rank

    def one():
        Z.neox_zero1_step_local(h, slot, stream)
        Z.neox_zero1_step_apply(h, r.data_ptr(), lr, stream, nranks=ranks)

    Z.neox_zero1_step_local(h, slot, stream)
    torch.cuda.synchronize()
    local = float(r[rank])
    others = torch.linspace(0.9, 1.1, ranks, dtype=torch.float64, device=device) * local
    r.copy_(others)
    before = Z.neox_scaler_state(h).skipped_total
    for _ in range(3):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    assert Z.neox_scaler_state(h).skipped_total == before, "split steps were skipped"
    return ms


def alloc_shard(w, dev, sgd):
    """The workload's five device arrays (one buffer per array for a flat shard, else one
    allocation per array per segment), initialized, with the step-0 gradient drawn; the
    segment list for the library.  Returns (buffer dicts, segments)."""
    import torch

    import mixed_precision_zero_amd as Z
    import workloads as W
    dt = torch.float16 if w.hyper.dtype == W.F16 else torch.bfloat16
    kinds = [("grad", dt), ("half", dt), ("master", torch.float32), ("m", torch.float32)]
    if not sgd:
        kinds.append(("v", torch.float32))
    keep, segs = [], []
    if w.flat:
        n = w.numel
        bufs = {k: torch.empty(n, dtype=t, device=dev) for k, t in kinds}
        bufs.setdefault("v", None)
        W.device_init_(w, bufs["master"], bufs["half"], bufs["m"], bufs["v"])
        W.device_grads_(w, bufs["grad"], 0, w.hyper.init_scale)
        off = 0
        for numel, decay in w.segments:
            sl = slice(off, off + numel)
            v = None if sgd else bufs["v"][sl]
            segs.append(Z.segment(bufs["grad"][sl], bufs["half"][sl], bufs["master"][sl],
                                  bufs["m"][sl], v, decay))
            off += numel
        keep.append(bufs)
    else:
        off = 0
        for i, (numel, decay) in enumerate(w.segments):
            a = {k: torch.empty(numel, dtype=t, device=dev) for k, t in kinds}
            a.setdefault("v", None)
            W.device_init_(w, a["master"], a["half"], a["m"], a["v"], i + 1)
            W.device_grads_(w, a["grad"], 0, w.hyper.init_scale, off)
            segs.append(Z.segment(a["grad"], a["half"], a["master"], a["m"], a["v"], decay))
            keep.append(a)
            off += numel
    return keep, segs


def norm_plan(Z, cfg, segs):
    """How the norm pass runs and who decides, from the library's own plan."""
    plan = Z.neox_zero1_plan(cfg, segs, tables=False)[0]
    return {"norm_blocks": min(plan.norm_chunks, cfg.norm_blocks or plan.norm_chunks),
            "norm_block_threads": plan.norm_block_threads,
            "update_decides": bool(plan.update_decides)}


def lib_config(Z, w, **over):
    return Z.neox_zero1_default_config(
        beta1=w.hyper.beta1, beta2=w.hyper.beta2, eps=w.hyper.eps,
        weight_decay=w.hyper.weight_decay, clip_norm=w.hyper.clip_norm,
        predivide_factor=w.hyper.predivide_factor, dp_world_size=w.hyper.dp_world_size,
        dtype=w.hyper.dtype, scaler_mode=w.hyper.scaler_mode,
        growth_interval=w.hyper.growth_interval, init_scale=w.hyper.init_scale,
        min_scale=w.hyper.min_scale, optimizer=w.hyper.optimizer, **over)


def median(xs):
    ys = sorted(xs)
    k = len(ys)
    return ys[k // 2] if k % 2 else 0.5 * (ys[k // 2 - 1] + ys[k // 2])


def timed_steps(Z, h, one_step, steps, events):
    """K steps by wall clock between synchronizations (the update kernel's own dispatch
    events recording on the side when `events`), then, with events, K more steps with all
    three kernels timed for the per-step durations (norm start to update end) and the
    norm / finalize split.  Returns a dict of the timings in ms."""
    import torch
    if events:
        Z.neox_zero1_timing_begin(h, steps, update_only=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    out = {"wall_ms": (t1 - t0) * 1e3 / steps}
    if events:
        sums, k, upd = Z.neox_zero1_timing_end(h, per_step=steps)
        out["update_ms"] = sums[2] / k
        out["update_median_ms"], out["update_min_ms"] = median(upd), min(upd)
        Z.neox_zero1_timing_begin(h, steps)
        for _ in range(steps):
            one_step()
        sums, k, per = Z.neox_zero1_timing_end(h, per_step=steps)
        out["norm_ms"], out["finalize_ms"] = sums[0] / k, sums[1] / k
        out["step_median_ms"], out["step_min_ms"] = median(per), min(per)
        out["event_steps"] = k
    return out


def extra_workload(name, dev, steps, warmup):
    """One more workload end to end (allocate, create, warm up, time, free): its line of
    the `workloads` object."""
    import gc

    import torch

    import mixed_precision_zero_amd as Z
    import workloads as W
    w = make_workload(name)
    n = w.numel
    print(f"[bench] workload {name}: {n} params, {len(w.segments)} segments", file=sys.stderr,
          flush=True)
    keep, segs = alloc_shard(w, dev, sgd=False)
    stream = torch.cuda.current_stream()
    cfg = lib_config(Z, w)
    h = Z.neox_zero1_create(cfg, segs, stream.cuda_stream)
    try:
        flat_path = Z.neox_zero1_update_path(h) == Z.NEOX_PATH_FLAT
        plan_info = norm_plan(Z, cfg, segs)

        def one_step():
            Z.neox_zero1_step(h, w.hyper.lr, stream.cuda_stream)

        for _ in range(warmup):
            one_step()
        t = timed_steps(Z, h, one_step, steps, events=True)
        st = Z.neox_scaler_state(h)
        assert st.skipped_total == 0 and st.step == warmup + 2 * steps, "bench steps were skipped"
    finally:
        Z.neox_zero1_destroy(h)
        del keep, segs
        gc.collect()
        torch.cuda.empty_cache()
    upd_gbs = UPDATE_BYTES_PER_PARAM * n / (t["update_ms"] * 1e-3) / 1e9
    upd_name = "flat_update_kernel" if flat_path else "update_kernel"
    return {"params": n, "segments": len(w.segments),
            "layout": "flat shard" if w.flat else "separate allocations",
            "grad_dtype": "f16" if w.hyper.dtype == W.F16 else "bf16",
            "update_path": "flat" if flat_path else "chunked", **plan_info,
            "steps": steps, "warmup": warmup,
            "value": n / (t["wall_ms"] * 1e-3), "unit": "params/s",
            "ms_per_step": t["wall_ms"], "ms_per_step_median": t["step_median_ms"],
            "ms_per_step_min": t["step_min_ms"],
            "step_gbps": STEP_BYTES_PER_PARAM * n / (t["wall_ms"] * 1e-3) / 1e9,
            "roofline": {"bound": "hbm", "kernel": upd_name,
                         "achieved": upd_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": upd_gbs / HBM_PEAK_GBS, "avg_ms": t["update_ms"],
                         "traffic": read_traffic(name, n, upd_name),
                         "bytes_per_launch": UPDATE_BYTES_PER_PARAM * n},
            "kernel_avg_ms": {"norm": t["norm_ms"], "finalize": t["finalize_ms"],
                              "update": t["update_ms"]}}


# the other shards of at least 2e8 params, timed in the default run: the largest one that
# fits one GPU (OPT-style, 6e9 params, 96 GB of state) and the 5,000 separately allocated
# tensors (chunk-table update)
EXTRA_WORKLOADS = (("opt_style_6b", 6, 2), ("multi_tensor_5000_bf16", 20, 6))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first (the first ~20 steps of a fresh process run up to 30%% slower while the GPU settles)")
    ap.add_argument("--workload", default="neox20b_shard_215m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cpu-large", action="store_true",
                    help="CPU baseline without the 5,000-tensor (in full) and 6e9 (windowed) "
                         "shards")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the copy / access-pattern probes after the timed steps")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="time only --workload (not the other >= 2e8-param shards)")
    ap.add_argument("--optimizer", choices=("adamw", "sgd"), default="adamw",
                    help="sgd: momentum SGD on the same shard (no second moment)")
    ap.add_argument("--split", action="store_true",
                    help="time the split step (step_local + step_apply on the local value)")
    ap.add_argument("--segment-norms", action="store_true",
                    help="keep per-segment squared norms (telemetry) during the step")
    ap.add_argument("--chunked-update", action="store_true",
                    help="run the update from the per-chunk work table even on a flat shard")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays")
    ap.add_argument("--no-timing-events", action="store_true",
                    help="time whole steps only (no per-kernel events)")
    ap.add_argument("--skip-steps", type=int, default=20,
                    help="steps timed with an inf in the gradient after the applied ones (0: none)")
    ap.add_argument("--copy-probe-only", type=int, default=0, metavar="BYTES",
                    help="run only a plain streaming copy of BYTES (counter calibration)")
    ap.add_argument("--summarize-pmc", action="store_true",
                    help="write the update kernel's traffic summary from rocprofv3 --pmc runs")
    ap.add_argument("--summarize-trace", metavar="DIR", dest="trace",
                    help="write the kernel-time summary of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--summarize-stalls", metavar="DIR", dest="stalls",
                    help="write the memory-side counter table (update against copy) from rocprofv3 "
                         "--pmc runs under DIR")
    ap.add_argument("--trace-steps", type=int, default=20)
    ap.add_argument("--bench-log")
    ap.add_argument("--bench-flags", default="",
                    help="extra bench.py flags the profiled runs used (recorded in the summary)")
    ap.add_argument("--pmc-fetch")
    ap.add_argument("--pmc-write")
    ap.add_argument("--pmc-copy-fetch")
    ap.add_argument("--pmc-copy-write")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--out")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.trace:
        summarize_trace(args)
        return
    if args.stalls:
        summarize_stalls(args)
        return
    if args.copy_probe_only:
        copy_probe(args.copy_probe_only)
        return
    if args.gpus != 1:
        print(f"bench.py: the step is one rank's work and is measured on one GPU only "
              f"(--gpus {args.gpus} requested); multi-GPU runs are not supported", file=sys.stderr)
        sys.exit(2)

    import gc

    import torch

    import mixed_precision_zero_amd as Z
    import workloads as W

    w = make_workload(args.workload)
    sgd = args.optimizer == "sgd"
    w.hyper.optimizer = 1 if sgd else 0
    n = w.numel
    upd_bpp = update_bytes(args.optimizer)
    step_bpp = upd_bpp + 2
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] workload {w.name}: {n} params, {len(w.segments)} segments, "
          f"{'flat' if w.flat else 'separate allocations'}", file=sys.stderr, flush=True)

    keep, segs = alloc_shard(w, dev, sgd)
    stream = torch.cuda.current_stream()
    cfg = lib_config(Z, w, segment_norms=int(args.segment_norms),
                     chunked_update=int(args.chunked_update))
    h = Z.neox_zero1_create(cfg, segs, stream.cuda_stream)
    flat_path = Z.neox_zero1_update_path(h) == Z.NEOX_PATH_FLAT
    plan_info = norm_plan(Z, cfg, segs)
    loc = torch.zeros(1, dtype=torch.float64, device=dev)

    def one_step():
        if args.split:
            # one rank: the exchange of the local norm is the identity
            Z.neox_zero1_step_local(h, loc.data_ptr(), stream.cuda_stream)
            Z.neox_zero1_step_apply(h, loc.data_ptr(), w.hyper.lr, stream.cuda_stream)
        else:
            Z.neox_zero1_step(h, w.hyper.lr, stream.cuda_stream)

    for _ in range(args.warmup):
        one_step()
    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            Z.neox_zero1_step(h, w.hyper.lr, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        one_step = graph.replay
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {args.steps} steps", file=sys.stderr,
          flush=True)

    # The timed steps record only the update kernel's two events; per-step durations and
    # the norm / finalize split come from as many steps with all events right after.
    timed_events = not args.no_timing_events and not args.split and not args.graph
    t = timed_steps(Z, h, one_step, args.steps, timed_events)
    st = Z.neox_scaler_state(h)
    done = args.warmup + args.steps * (2 if timed_events else 1)
    assert st.skipped_total == 0 and st.step == done, "bench steps were skipped"
    split = None
    if not args.split and not args.graph and not args.segment_norms:
        print(f"[bench] {args.steps} split steps over {SPLIT_RANKS} ranks", file=sys.stderr,
              flush=True)
        split = time_split_steps(Z, h, w.hyper.lr, stream.cuda_stream, args.steps)
    skipped = None
    if args.skip_steps > 0:
        print(f"[bench] {args.skip_steps} skipped steps (inf in the gradient)", file=sys.stderr,
              flush=True)
        skipped = time_skipped_steps(Z, h, keep[0]["grad"], one_step, args.skip_steps,
                                     timed_events)
    Z.neox_zero1_destroy(h)
    ceiling = measure_ceiling(keep[0], n) if (w.flat and n % 8 == 0 and not sgd
                                             and not args.no_ceiling) else None
    del keep, segs
    gc.collect()
    torch.cuda.empty_cache()

    ms_per_step = t["wall_ms"]
    value = n / (ms_per_step * 1e-3)
    out = {
        "metric": "params/sec per fused ZeRO-1 Adam step; achieved HBM GB/s vs MI355X peak",
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_median": t.get("step_median_ms"),
        "ms_per_step_min": t.get("step_min_ms"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "params": n, "segments": len(w.segments),
                   "grad_dtype": "f16" if w.hyper.dtype == W.F16 else "bf16",
                   "layout": "flat shard" if w.flat else "separate allocations",
                   "optimizer": args.optimizer, "split": args.split,
                   "segment_norms": args.segment_norms, "graph": args.graph,
                   "update_path": "flat" if flat_path else "chunked", **plan_info},
        "hbm": {"step_bytes": step_bpp * n,
                "step_gbps": step_bpp * n / (ms_per_step * 1e-3) / 1e9,
                "step_frac_of_peak": step_bpp * n / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "step_timing": {"value_and_ms_per_step": "wall clock over the timed steps",
                        "median_and_min": "per-step durations from the kernels' own dispatch "
                                          "events (norm start to update end), as many steps "
                                          "right after the timed ones"},
    }
    if timed_events:
        upd_gbs = upd_bpp * n / (t["update_ms"] * 1e-3) / 1e9
        default_mode = not args.segment_norms
        upd_name = "flat_update_kernel" if flat_path else "update_kernel"
        out["roofline"] = {"bound": "hbm", "achieved": upd_gbs, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": upd_gbs / HBM_PEAK_GBS,
                           "traffic": read_traffic(w.name, n, upd_name, args.optimizer)
                           if default_mode else None,
                           "kernel": upd_name,
                           "avg_ms": t["update_ms"],
                           "median_ms": t["update_median_ms"],
                           "min_ms": t["update_min_ms"],
                           "bytes_per_launch": upd_bpp * n}
        out["kernel_avg_ms"] = {"norm": t["norm_ms"], "finalize": t["finalize_ms"],
                                "update": t["update_ms"]}
    if split:
        out["split_step"] = {"ranks": SPLIT_RANKS, "steps": args.steps, "ms_per_step": split,
                             "value": n / (split * 1e-3), "unit": "params/s",
                             "note": "step_local + step_apply over the ranks' squared norms, "
                                     "the step a data-parallel rank runs; the exchange "
                                     "between them needs other GPUs and is not timed"}
    if skipped:
        sk_ms, sk_kernels = skipped
        out["skipped_step"] = {"steps": args.skip_steps, "ms_per_step": sk_ms,
                               "bytes": 2 * n, "gbps": 2 * n / (sk_ms * 1e-3) / 1e9}
        if sk_kernels:
            out["skipped_step"]["kernel_avg_ms"] = sk_kernels
    if ceiling:
        ceiling["note"] = ("measured on this GPU right after the timed steps, on the same "
                           "arrays: a plain copy (best of plain and non-temporal stores), the "
                           "attainable rate of the simplest in-place-free stream; and a second "
                           "kernel with the update's access pattern and trivial arithmetic, "
                           "best of the launch shapes swept (threads x vectors per thread / "
                           "blocks per CU / non-temporal stores) -- a comparison, not an upper "
                           "bound")
        if timed_events:
            out["roofline"]["copy_gbps"] = ceiling["copy_gbps"]
            out["roofline"]["frac_of_copy"] = out["roofline"]["achieved"] / ceiling["copy_gbps"]
            ceiling["update_kernel_over_pattern"] = out["roofline"]["achieved"] / \
                ceiling["update_pattern_gbps"]
        ceiling["step_over_copy"] = out["hbm"]["step_gbps"] / ceiling["copy_gbps"]
        out["probes"] = ceiling
    if not args.no_extra_workloads and not args.split and not args.graph and not sgd \
            and not args.segment_norms and not args.chunked_update:
        out["workloads"] = {}
        for name, k, wu in EXTRA_WORKLOADS:
            if name != w.name:
                out["workloads"][name] = extra_workload(name, dev, k, wu)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        large = (not args.no_extra_workloads and not args.no_cpu_large and
                 "workloads" in out)
        out["cpu_baseline"] = cpu_baseline(w, dev=dev if large else None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
