#!/usr/bin/env python3
"""Throughput of the ZeRO-1 mixed-precision Adam step on one MI355X.

One step = the whole hot path on the shard: norm/overflow pass, finalize, fused
unscale + clip + AdamW + cast update.  Inputs are synthetic and already resident in
HBM.  Prints one JSON line:
  value     params/s over the timed steps (wall clock between synchronizations)
  roofline  the update kernel (the dominant one): algorithmic bytes per launch over its
            average duration from HIP events its own dispatch stamps, against 8 TB/s;
            traffic = HBM bytes per launch from the committed rocprofv3 counter summary
            of this workload and kernel (null when there is none for the current sources)
  kernel_avg_ms  norm / finalize / update durations (a short all-kernel pass after)
  skipped_step   the cost of a step with an inf in the gradient (timed last)
  ceiling   a kernel with the update's access pattern and trivial arithmetic, swept over
            launch shapes, and a plain copy, both on this GPU right after the timed steps
  cpu_baseline  the CPU oracle, single thread, on a bounded sample of the workload
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

    import workloads as W
    files = glob.glob(os.path.join(args.trace, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {args.trace}")
    with open(files[0]) as fh:
        rows = [r for r in csv.DictReader(fh) if "nz1::" in r["Name"]]
    n = W.BENCH_WORKLOADS[args.workload]().numel
    flags = f" {args.bench_flags}" if getattr(args, "bench_flags", "") else ""
    per_param = {"update_kernel": update_bytes(flags_optimizer(args)), "norm_kernel": 2}
    lines = [
        f"# rocprofv3 kernel trace of the ZeRO-1 step on {args.workload} ({n} params), MI355X (gfx950).",
        "# Commands (from the repository root, on an MI355X):",
        f"#   rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o trace -- python3 bench.py "
        f"--workload {args.workload} --steps {args.trace_steps} --warmup 3 --no-cpu-baseline --skip-steps 0"
        f"{flags} > <log>",
        f"#   python3 bench.py --summarize-trace <dir> --workload {args.workload} "
        f"--trace-steps {args.trace_steps} --bench-log <log>{bench_flags_arg(args)}",
        f"# Calls = 3 warm-up + {args.trace_steps} timed steps (update-kernel events only) + "
        f"{min(20, args.trace_steps)} steps",
        "# with events around every kernel; the torch kernels that draw the synthetic inputs and the",
        "# ceiling probes are left out.  Durations in ns.",
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
    import workloads as W
    n = W.BENCH_WORKLOADS[args.workload]().numel
    traffic = (fetch * ff + write * fw) * 1024.0
    flags = f" {args.bench_flags}" if getattr(args, "bench_flags", "") else ""
    opt = flags_optimizer(args)
    bpp = update_bytes(opt)
    lines = [
        f"# HBM traffic of the update on {args.workload} ({n} params), from rocprofv3 PMC.",
        "# Commands (from the repository root, on an MI355X):",
        f"#   rocprofv3 --pmc FETCH_SIZE -d <fetch_dir> --output-format csv -- python3 bench.py "
        f"--workload {args.workload} --steps 5 --warmup 1 --no-cpu-baseline --no-timing-events --skip-steps 0"
        f"{flags}",
        "#   rocprofv3 --pmc WRITE_SIZE -d <write_dir> ... (same program)",
        f"#   rocprofv3 --pmc FETCH_SIZE -d <copy_fetch_dir> --output-format csv -- python3 bench.py "
        f"--copy-probe-only {args.copy_bytes}",
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


def cpu_baseline(w, budget_s=12.0, sample=1 << 24):
    """The oracle as it stands, one thread, on the first `sample` params of the shard."""
    import numpy as np

    import workloads as W
    from oracle import oracle as O

    sample = min(sample, w.numel)
    segs, left = [], sample
    for n, d in w.segments:
        if left == 0:
            break
        segs.append((min(n, left), d))
        left -= segs[-1][0]
    st0 = W.host_init(w, n=sample)
    h = w.hyper
    cfg = O.Config(beta1=h.beta1, beta2=h.beta2, eps=h.eps, weight_decay=h.weight_decay,
                   clip_norm=h.clip_norm, predivide_factor=h.predivide_factor,
                   dp_world_size=h.dp_world_size, dtype=h.dtype, scaler_mode=h.scaler_mode,
                   growth_interval=h.growth_interval, growth_factor=h.growth_factor,
                   backoff_factor=h.backoff_factor, min_scale=h.min_scale,
                   optimizer=h.optimizer)
    st = O.Scaler(loss_scale=h.init_scale)
    spent, steps = 0.0, 0
    while spent < budget_s and steps < 50:
        g = W.host_grads(w, steps, st.loss_scale, n=sample)
        osegs, off = [], 0
        for n, d in segs:
            sl = slice(off, off + n)
            osegs.append(dict(grad=g[sl], half=st0["half"][sl], master=st0["master"][sl],
                              m=st0["m"][sl], v=None if h.optimizer else st0["v"][sl], decay=d))
            off += n
        t0 = time.perf_counter()
        O.step(cfg, st, np.float32(h.lr), osegs)
        spent += time.perf_counter() - t0
        steps += 1
    return {"value": sample * steps / spent, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"first {sample} params of the shard ({len(segs)} segments), {steps} steps, "
                      f"{spent:.1f} s of single-thread oracle time (fp64 scalar C, -O2)"}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="neox20b_shard_215m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the attainable-bandwidth probes after the timed steps")
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
    if args.copy_probe_only:
        copy_probe(args.copy_probe_only)
        return
    if args.gpus != 1:
        print(f"bench.py: the step is one rank's work and is measured on one GPU only "
              f"(--gpus {args.gpus} requested); multi-GPU runs are not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixed_precision_zero_amd as Z
    import workloads as W

    if args.workload not in W.BENCH_WORKLOADS:
        sys.exit(f"unknown workload {args.workload}; one of {sorted(W.BENCH_WORKLOADS)}")
    w = W.BENCH_WORKLOADS[args.workload]()
    sgd = args.optimizer == "sgd"
    w.hyper.optimizer = 1 if sgd else 0
    n = w.numel
    upd_bpp = update_bytes(args.optimizer)
    step_bpp = upd_bpp + 2
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    dt = torch.float16 if w.hyper.dtype == W.F16 else torch.bfloat16
    print(f"[bench] workload {w.name}: {n} params, {len(w.segments)} segments, "
          f"{'flat' if w.flat else 'separate allocations'}", file=sys.stderr, flush=True)

    keep = []
    segs = []
    kinds = [("grad", dt), ("half", dt), ("master", torch.float32), ("m", torch.float32)]
    if not sgd:
        kinds.append(("v", torch.float32))
    if w.flat:
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
    stream = torch.cuda.current_stream()
    h = Z.neox_zero1_create(Z.neox_zero1_default_config(
        beta1=w.hyper.beta1, beta2=w.hyper.beta2, eps=w.hyper.eps,
        weight_decay=w.hyper.weight_decay, clip_norm=w.hyper.clip_norm,
        predivide_factor=w.hyper.predivide_factor, dp_world_size=w.hyper.dp_world_size,
        dtype=w.hyper.dtype, scaler_mode=w.hyper.scaler_mode,
        growth_interval=w.hyper.growth_interval, init_scale=w.hyper.init_scale,
        min_scale=w.hyper.min_scale, optimizer=w.hyper.optimizer,
        segment_norms=int(args.segment_norms), chunked_update=int(args.chunked_update)),
        segs, stream.cuda_stream)
    flat_path = Z.neox_zero1_update_path(h) == Z.NEOX_PATH_FLAT
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

    # The timed steps record only the update kernel's two events; the norm / finalize
    # split comes from a short pass with all events after the timed region.
    timed_events = not args.no_timing_events and not args.split and not args.graph
    if timed_events:
        Z.neox_zero1_timing_begin(h, args.steps, update_only=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    st = Z.neox_scaler_state(h)
    kernel_ms = None
    if timed_events:
        sums, k = Z.neox_zero1_timing_end(h)
        update_ms = sums[2] / k
        nb = min(20, args.steps)
        Z.neox_zero1_timing_begin(h, nb)
        for _ in range(nb):
            one_step()
        sums, k2 = Z.neox_zero1_timing_end(h)
        kernel_ms = [sums[0] / k2, sums[1] / k2, update_ms]
    assert st.skipped_total == 0 and st.step == args.warmup + args.steps, "bench steps were skipped"
    skipped = None
    if args.skip_steps > 0:
        print(f"[bench] {args.skip_steps} skipped steps (inf in the gradient)", file=sys.stderr,
              flush=True)
        skipped = time_skipped_steps(Z, h, keep[0]["grad"], one_step, args.skip_steps,
                                     timed_events)
    Z.neox_zero1_destroy(h)
    ceiling = measure_ceiling(keep[0], n) if (w.flat and n % 8 == 0 and not sgd
                                             and not args.no_ceiling) else None

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = n / (ms_per_step * 1e-3)
    out = {
        "metric": "params/sec per fused ZeRO-1 Adam step; achieved HBM GB/s vs MI355X peak",
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
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
                   "update_path": "flat" if flat_path else "chunked"},
        "hbm": {"step_bytes": step_bpp * n,
                "step_gbps": step_bpp * n / (ms_per_step * 1e-3) / 1e9,
                "step_frac_of_peak": step_bpp * n / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }
    if kernel_ms:
        upd_gbs = upd_bpp * n / (kernel_ms[2] * 1e-3) / 1e9
        default_mode = not args.segment_norms
        upd_name = "flat_update_kernel" if flat_path else "update_kernel"
        out["roofline"] = {"bound": "hbm", "achieved": upd_gbs, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": upd_gbs / HBM_PEAK_GBS,
                           "traffic": read_traffic(w.name, n, upd_name, args.optimizer)
                           if default_mode else None,
                           "kernel": upd_name,
                           "avg_ms": kernel_ms[2],
                           "bytes_per_launch": upd_bpp * n}
        out["kernel_avg_ms"] = {"norm": kernel_ms[0], "finalize": kernel_ms[1],
                                "update": kernel_ms[2]}
    if skipped:
        sk_ms, sk_kernels = skipped
        out["skipped_step"] = {"steps": args.skip_steps, "ms_per_step": sk_ms,
                               "bytes": 2 * n, "gbps": 2 * n / (sk_ms * 1e-3) / 1e9}
        if sk_kernels:
            out["skipped_step"]["kernel_avg_ms"] = sk_kernels
    if ceiling:
        ceiling["note"] = ("measured on this GPU right after the timed steps: a kernel with the "
                           "update's access pattern and trivial arithmetic, best of the launch "
                           "shapes swept (threads x vectors per thread / blocks per CU / "
                           "non-temporal stores), and a plain copy (best of plain and "
                           "non-temporal stores)")
        if kernel_ms:
            ceiling["update_kernel_frac_of_pattern"] = out["roofline"]["achieved"] / \
                ceiling["update_pattern_gbps"]
        ceiling["step_frac_of_pattern"] = out["hbm"]["step_gbps"] / ceiling["update_pattern_gbps"]
        out["ceiling"] = ceiling
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle, one thread)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
