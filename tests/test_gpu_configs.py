"""GPU parity at the full sizes of the five workloads, in the default launch
configuration (the one bench.py times).

Every step's decisions (skip, loss scale, counters, step count) are compared with the
oracle's scaler; on selected steps the oracle also scans the whole gradient (global
norm) and recomputes sampled windows elementwise: every segment's first and last
elements plus seeded random windows."""
import numpy as np
import pytest
import torch

import mixed_precision_zero_amd as Z
import workloads as W
from gpu_harness import Checker, DeviceShard, lib_config, log

pytestmark = pytest.mark.gpu


def sample_windows(shard, seed, nwin=24, wlen=1 << 15, ends=2048, max_segments=64):
    """Both ends of every segment (of a seeded sample of max_segments segments when
    there are more), plus nwin seeded windows of wlen elements."""
    rng = np.random.default_rng(seed)
    out = []
    sizes = [s["grad"].numel() for s in shard.segs]
    pick = range(len(sizes))
    if len(sizes) > max_segments:
        pick = sorted(rng.choice(len(sizes), size=max_segments, replace=False).tolist())
    for i in pick:
        n = sizes[i]
        if n <= 2 * ends:
            out.append((i, 0, n))
        else:
            out += [(i, 0, ends), (i, n - ends, n)]
    big = [i for i, n in enumerate(sizes) if n > wlen]
    for _ in range(nwin if big else 0):
        i = big[int(rng.integers(0, len(big)))]
        lo = int(rng.integers(0, sizes[i] - wlen))
        out.append((i, lo, lo + wlen))
    return out


def run(w, checked_steps, threads=8, windows_seed=0, full_steps=(), **cfg_over):
    """Steps w on the GPU and the oracle; on checked_steps the oracle scans the whole
    gradient and recomputes sampled windows, on full_steps every element."""
    shard = DeviceShard(w)
    shard.init_()
    chk = Checker(shard, **cfg_over)
    try:
        wins = sample_windows(shard, windows_seed)
        for k in range(w.steps):
            shard.grads_(k, chk.scale())
            injected = bool(w.injections.get(k))
            if k in full_steps:
                log(f"  {w.name} step {k}: full scan + every element of every segment")
                chk.step(w.hyper.lr, windows=None, threads=threads, where=f" {w.name} step {k}")
            elif k in checked_steps:
                log(f"  {w.name} step {k}: full scan + {len(wins)} windows")
                chk.step(w.hyper.lr, windows=wins, threads=threads, where=f" {w.name} step {k}")
            else:
                # no draw of N(0, sigma) * scale reaches the half range's limit: the
                # overflow flag is exactly "this step has an injection"
                chk.step(w.hyper.lr, check=injected, windows=wins if injected else None,
                         overflow=injected, where=f" {w.name} step {k}")
    finally:
        chk.close()
    return chk


def test_pythia410m_rank0_and_rank1():
    """Pythia-410M-like, DP = 8: rank 0 (all embedding, one segment) and rank 1 (36
    segments, 38,912 no-decay elements), 20 steps; the segment list is the library's
    own partition."""
    t = W.pythia410m_tensors()
    for rank in (0, 1):
        segs, P = Z.neox_zero1_partition([n for n, _ in t], [d for _, d in t], 8, rank, 64)
        assert P == 44_227_584 and len(segs) == (1 if rank == 0 else 36)
        w = W.pythia410m(rank, [(s.numel, s.flags) for s in segs])
        log(f"case pythia410m rank {rank}: {len(segs)} segments")
        chk = run(w, checked_steps={0, 1, 19}, windows_seed=rank)
        assert chk.ost.step == 20


def test_pythia410m_eight_ranks_equal_unsharded():
    """ZeRO-1 sharding: with clipping off the eight ranks' shards, stepped one after
    another on this GPU, equal the unsharded step bit for bit (3 steps)."""
    t = W.pythia410m_tensors()
    numel = [n for n, _ in t]
    decay = [d for _, d in t]
    total = sum(numel)
    hy = W.Hyper(clip_norm=0.0)
    full_w = W.Workload("pythia410m_full", 2, list(t), hy, steps=3)
    full = DeviceShard(full_w)
    full.init_()
    init = {k: full.buffers[k].clone() for k in ("master", "half", "m", "v")}
    stream = torch.cuda.current_stream().cuda_stream
    grads = []
    for k in range(3):
        g = torch.empty(total, dtype=torch.float16, device="cuda")
        W.device_grads_(full_w, g, k, 65536.0)
        grads.append(g)
    h = Z.neox_zero1_create(lib_config(full_w), full.neox_segments(), stream)
    for k in range(3):
        full.buffers["grad"].copy_(grads[k])
        Z.neox_zero1_step(h, 6e-4, stream)
    Z.neox_zero1_destroy(h)
    want = {k: full.buffers[k].clone() for k in ("master", "half", "m", "v")}
    del full

    for rank in range(8):
        segs, P = Z.neox_zero1_partition(numel, decay, 8, rank, 64)
        lo = rank * P
        bufs = {k: init[k][lo:lo + P].clone() for k in init}
        gbuf = torch.empty(P, dtype=torch.float16, device="cuda")
        nsegs = []
        for s in segs:
            sl = slice(s.shard_offset, s.shard_offset + s.numel)
            nsegs.append(Z.segment(gbuf[sl], bufs["half"][sl], bufs["master"][sl], bufs["m"][sl],
                                   bufs["v"][sl], bool(s.flags)))
        h = Z.neox_zero1_create(lib_config(full_w), nsegs, stream)
        for k in range(3):
            gbuf.copy_(grads[k][lo:lo + P])
            Z.neox_zero1_step(h, 6e-4, stream)
        Z.neox_zero1_destroy(h)
        torch.cuda.synchronize()
        for k in bufs:
            assert torch.equal(bufs[k], want[k][lo:lo + P]), (rank, k)
        log(f"  rank {rank} equals the unsharded step")


def test_neox20b_shard_100_steps():
    """215,000,000-param shard, 9 segments, 100 steps, default launch shape: every one of
    the 215M elements of master, exp_avg, exp_avg_sq and the half copy against the oracle
    on the first and the last step, sampled windows on steps 1 and 50."""
    w = W.neox20b_shard()
    log("case neox20b shard")
    chk = run(w, checked_steps={1, 50}, full_steps={0, 99}, threads=16)
    assert chk.ost.step == 100 and chk.ost.skipped_total == 0


def test_multi_tensor_5000_bf16():
    """5,000 separately allocated tensors (~1e9 params), bf16, static scale 1, 20%
    no-decay, clip 1.0 (active: the norm is ~3.2)."""
    w = W.multi_tensor()
    assert len(w.segments) == 5000 and abs(w.numel - 1e9) < 1e6
    log(f"case multi-tensor: {w.numel} params")
    chk = run(w, checked_steps={0, 1, 19})
    assert chk.ost.last_coef < 1.0 and chk.ost.loss_scale == 1.0


def test_opt_style_6b_collapse_and_recovery():
    """6e9 params (> 2^32 elements), f = 8, D = 128, clip 0.3: 3 clean steps, 20 forced
    overflows (scale 2^16 -> floor 1.0 after 16, then 4 more at the floor), 16 clean
    steps in which the scale doubles every 4 steps to 16."""
    w = W.opt_large()
    assert w.numel == 6_000_000_000 and len(w.segments) == 41
    log("case opt-style 6e9")
    chk = run(w, checked_steps={0, 38}, threads=16)
    st = chk.ost
    assert (st.skipped_total, st.step, st.loss_scale) == (20, 19, 16.0)


def test_multi_tensor_literal_draws_138gb():
    """The multi-tensor workload with its sizes drawn literally (5,000 tensors of
    log-uniform 1K..16M elements, ~8.6e9 params, ~138 GB of resident state): decisions
    every step, the oracle's full norm and sampled windows on the first and last steps."""
    w = W.multi_tensor(steps=4, literal=True)
    assert w.numel > 8e9
    log(f"case multi-tensor literal: {w.numel} params")
    chk = run(w, checked_steps={0, 3}, threads=16)
    assert chk.ost.step == 4 and chk.ost.last_coef < 1.0
