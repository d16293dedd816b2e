"""GPU parity of the rows after the core step: the split step for data-parallel ranks,
the scaler set / reset, per-segment norm telemetry, and the momentum-SGD variant."""
import numpy as np
import pytest
import torch

import mixed_precision_zero_amd as Z
import workloads as W
from gpu_harness import (Checker, DeviceShard, assert_close, assert_half_close, lib_config, log,
                         oracle_config)
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _custom(name, sizes, decays, dtype=W.F16, steps=4, **hy):
    return W.Workload(name, 910, list(zip(sizes, decays)), W.Hyper(dtype=dtype, **hy), steps=steps)


def _outputs(shard):
    torch.cuda.synchronize()
    return {k: torch.cat([s[k].reshape(-1) for s in shard.segs]).clone()
            for k in ("half", "master", "m", "v") if shard.segs[0][k] is not None}


# ----------------------------------------------------------------------------------
# split step
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("sizes", [[70_001, 4096, 33], [3000] * 150, [1000] * 256],
                         ids=["38_parts", "150_parts", "256_parts"])
def test_split_step_equals_step_on_one_rank(sizes):
    """step == step_local followed by step_apply on the local value, bit for bit.  With
    per-segment norms the norm chunks follow the segments, so these shards' norm passes
    have from 38 up to 256 blocks, whose partials fill one wave of the fixed-order sum or
    all four; the step's update adds the partials itself, the split step reduces them to
    one value first, and the two must agree bit for bit."""
    w = _custom("split1", sizes, [k % 3 != 1 for k in range(len(sizes))], clip_norm=0.05)
    w.injections = {2: [(10, "nan")]}
    stream = torch.cuda.current_stream().cuda_stream
    outs, states = [], []
    for mode in ("step", "split"):
        sh = DeviceShard(w)
        sh.init_()
        cfg = lib_config(w, segment_norms=1)
        h = Z.neox_zero1_create(cfg, sh.neox_segments(), stream)
        plan, _, _, _ = Z.neox_zero1_plan(cfg, sh.neox_segments(), tables=False)
        assert plan.norm_chunks <= 256 and plan.update_decides == 1, plan.norm_chunks
        assert plan.norm_chunks >= min(38, len(sizes)), plan.norm_chunks
        loc = torch.zeros(1, dtype=torch.float64, device="cuda")
        st_seq = []
        for k in range(5):
            sh.grads_(k, Z.neox_scaler_state(h).loss_scale)
            if mode == "step":
                Z.neox_zero1_step(h, 1e-3, stream)
            else:
                Z.neox_zero1_step_local(h, loc.data_ptr(), stream)
                Z.neox_zero1_step_apply(h, loc.data_ptr(), 1e-3, stream)
            st = Z.neox_scaler_state(h)
            st_seq.append((st.loss_scale, st.step, st.skipped_total, st.last_grad_norm,
                           st.last_sumsq, st.last_clip_coef))
        Z.neox_zero1_destroy(h)
        outs.append(_outputs(sh))
        states.append(st_seq)
    assert states[0] == states[1]
    for k in outs[0]:
        assert torch.equal(outs[0][k], outs[1][k]), k


@pytest.mark.parametrize("optimizer", [Z.NEOX_OPT_ADAMW, Z.NEOX_OPT_SGD], ids=["adamw", "sgd"])
def test_split_step_with_telemetry_and_sgd(optimizer):
    """The split step combined with per-segment telemetry, for both optimizers: outputs,
    scaler state and every segment's squared norm equal the fused step's bit for bit,
    over clean steps and one with a NaN (whose segment alone reports a non-finite norm)."""
    w = _custom("split_combo", [30_000, 2048, 17, 9000], [True, False, True, False],
                clip_norm=0.05, optimizer=optimizer)
    w.injections = {1: [(30_000 + 2048 + 5, "nan")]}       # element 5 of segment 2
    stream = torch.cuda.current_stream().cuda_stream
    results = []
    for mode in ("step", "split"):
        sh = DeviceShard(w)
        sh.init_()
        h = Z.neox_zero1_create(lib_config(w, segment_norms=1), sh.neox_segments(), stream)
        loc = torch.zeros(1, dtype=torch.float64, device="cuda")
        seq = []
        try:
            for k in range(4):
                sh.grads_(k, Z.neox_scaler_state(h).loss_scale)
                if mode == "step":
                    Z.neox_zero1_step(h, 1e-3, stream)
                else:
                    Z.neox_zero1_step_local(h, loc.data_ptr(), stream)
                    Z.neox_zero1_step_apply(h, loc.data_ptr(), 1e-3, stream)
                st = Z.neox_scaler_state(h)
                seg = Z.neox_zero1_segment_sumsq(h, len(w.segments))
                seq.append(((st.loss_scale, st.step, st.skipped_total, st.last_sumsq),
                            [float(x) for x in seg]))
        finally:
            Z.neox_zero1_destroy(h)
        results.append((_outputs(sh), seq))
        log(f"case split+telemetry optimizer={optimizer} mode={mode}")
    (out_a, seq_a), (out_b, seq_b) = results
    assert [s for s, _ in seq_a] == [s for s, _ in seq_b]
    for (_, ga), (_, gb) in zip(seq_a, seq_b):
        assert np.array_equal(np.array(ga), np.array(gb), equal_nan=True)
    skipped = seq_a[1][1]
    assert [bool(np.isfinite(x)) for x in skipped] == [True, True, False, True]
    assert seq_a[1][0][2] == 1                                # that step was skipped
    for k in out_a:
        assert torch.equal(out_a[k], out_b[k]), k


def test_split_step_keeps_the_finalize_on_a_large_chunk_table():
    """A separately allocated shard of ~9M elements: its norm pass has more than 256
    blocks, so neither its step's update nor its split step's update decides; both run
    the finalize, and step == step_local + step_apply (one rank) bit for bit, with
    clipping active and a skipped step."""
    w = _custom("split_table", [4_000_000, 3_000_001, 2_000_000, 77], [True, False, True, False],
                clip_norm=0.05)
    w.flat = False
    w.injections = {1: [(3_999_999, "-inf")]}
    stream = torch.cuda.current_stream().cuda_stream
    outs, states = [], []
    for mode in ("step", "split"):
        sh = DeviceShard(w)
        sh.init_()
        cfg = lib_config(w)
        plan = Z.neox_zero1_plan(cfg, sh.neox_segments(), tables=False)[0]
        assert plan.update_path == Z.NEOX_PATH_CHUNKED and plan.update_decides == 0
        assert plan.norm_chunks > 256, plan.norm_chunks
        h = Z.neox_zero1_create(cfg, sh.neox_segments(), stream)
        loc = torch.zeros(1, dtype=torch.float64, device="cuda")
        seq = []
        try:
            for k in range(3):
                sh.grads_(k, Z.neox_scaler_state(h).loss_scale)
                if mode == "step":
                    Z.neox_zero1_step(h, 1e-3, stream)
                else:
                    Z.neox_zero1_step_local(h, loc.data_ptr(), stream)
                    Z.neox_zero1_step_apply(h, loc.data_ptr(), 1e-3, stream)
                st = Z.neox_scaler_state(h)
                seq.append((st.loss_scale, st.step, st.skipped_total, st.last_sumsq,
                            st.last_clip_coef))
        finally:
            Z.neox_zero1_destroy(h)
        log(f"case split on a large chunk table mode={mode}")
        outs.append(_outputs(sh))
        states.append(seq)
    assert states[0] == states[1]
    assert states[0][1][2] == 1 and states[0][2][4] < 1.0
    for k in outs[0]:
        assert torch.equal(outs[0][k], outs[1][k]), k


@pytest.mark.parametrize("optimizer", [Z.NEOX_OPT_ADAMW, Z.NEOX_OPT_SGD], ids=["adamw", "sgd"])
def test_split_apply_update_decides_like_the_finalize(optimizer):
    """step_apply over at most 256 rank values lets the update add them and decide; over
    more it launches the finalize.  The sum of 256 values and of the same values followed
    by one +0.0 have the same bits in the fixed order, so the two paths, on identical
    shards, must give identical outputs and scaler state every step: clipping active, a
    NaN on one rank skipping a step, the local value at rank 5 of 256."""
    w = _custom("split_paths", [300_000, 4099, 65_536], [True, False, True], clip_norm=0.05,
                optimizer=optimizer)
    w.injections = {2: [(123, "nan")]}
    stream = torch.cuda.current_stream().cuda_stream
    shards = [DeviceShard(w), DeviceShard(w)]
    hs = []
    for sh in shards:
        sh.init_()
        hs.append(Z.neox_zero1_create(lib_config(w), sh.neox_segments(), stream))
    rng = np.random.default_rng(77)
    others = torch.tensor(rng.uniform(0.5, 2.0, 256), dtype=torch.float64, device="cuda")
    loc = torch.zeros(1, dtype=torch.float64, device="cuda")
    try:
        for k in range(4):
            ranks = []
            for sh, h, n in zip(shards, hs, (256, 257)):
                sh.grads_(k, Z.neox_scaler_state(h).loss_scale)
                Z.neox_zero1_step_local(h, loc.data_ptr(), stream)
                r = torch.zeros(n, dtype=torch.float64, device="cuda")
                r[:256] = others * loc        # the other ranks: multiples of this one
                r[5] = loc[0]
                Z.neox_zero1_step_apply(h, r.data_ptr(), 1e-3, stream, nranks=n)
                ranks.append(r)
            a, b = (Z.neox_scaler_state(h) for h in hs)
            assert (a.loss_scale, a.step, a.skipped_total, a.last_sumsq, a.last_clip_coef) == \
                (b.loss_scale, b.step, b.skipped_total, b.last_sumsq, b.last_clip_coef), k
            if k != 2:
                assert a.last_clip_coef < 1.0 and not a.last_skipped
            oa, ob = _outputs(shards[0]), _outputs(shards[1])
            for name in oa:
                assert torch.equal(oa[name], ob[name]), (k, name)
        assert Z.neox_scaler_state(hs[0]).skipped_total == 1
    finally:
        for h in hs:
            Z.neox_zero1_destroy(h)


@pytest.mark.parametrize("D", [4, 8])
def test_split_step_ranks_match_the_global_oracle(D):
    """D ZeRO-1 ranks of one model on this GPU, one after another: each runs step_local,
    the D local squared norms are gathered in rank order and every rank's step_apply adds
    them (the same bits on every rank).  Decisions equal the oracle's on the whole model every step,
    clipping is active, an inf in one rank's shard skips every rank, and every rank's
    elements match the oracle's global step."""
    tensors = [(50_000, True), (1_000, False), (120_011, True), (7, False), (30_000, True),
               (2_048, False), (64_000, True)]
    A = 64
    numel = [n for n, _ in tensors]
    decay = [d for _, d in tensors]
    hy = W.Hyper(clip_norm=0.02)
    full = W.Workload(f"split{D}", 911, tensors, hy, grad_sigma=1e-4)
    total = full.numel
    stream = torch.cuda.current_stream().cuda_stream

    ranks = []
    for r in range(D):
        segs, P = Z.neox_zero1_partition(numel, decay, D, r, A)
        wr = W.Workload(f"rank{r}", 911, [(s.numel, bool(s.flags)) for s in segs], hy)
        sh = DeviceShard(wr)
        sh.init_(seed_extra=r)
        chk = Checker(sh)
        ranks.append(dict(P=P, lo=r * P, shard=sh, chk=chk,
                          loc=torch.zeros(1, dtype=torch.float64, device="cuda"),
                          glob=torch.zeros(1, dtype=torch.float64, device="cuda")))
    padded = ranks[0]["P"] * D
    ocfg = oracle_config(full)
    ost = O.Scaler(loss_scale=hy.init_scale)
    gfull = torch.zeros(padded, dtype=torch.float16, device="cuda")
    lr = np.float32(1e-3)
    try:
        for k in range(5):
            W.device_grads_(full, gfull[:total], k, ost.loss_scale)
            if k == 3:   # overflow inside rank 2's shard only
                gfull.view(torch.int16)[ranks[2]["lo"] + 5] = 0x7C00
            for rk in ranks:
                rk["shard"].buffers["grad"].copy_(gfull[rk["lo"]:rk["lo"] + rk["P"]])
            torch.cuda.synchronize()
            # oracle on the whole model
            g_host = gfull.view(torch.int16).cpu().numpy().view(np.uint16)
            inv, inv32 = O.unscale_factor(ocfg, ost)
            sumsq, of = O.scan(W.F16, g_host, inv, inv32)
            pre = [rk["shard"].host_window(i, 0, s["grad"].numel())
                   for rk in ranks for i, s in enumerate(rk["shard"].segs)]
            d = O.decide(ocfg, ost, of, sumsq)
            # the ranks: local norms, gathered in rank order (an all-gather's result) into
            # every rank's copy of the array, then apply (the library adds them)
            for rk in ranks:
                Z.neox_zero1_step_local(rk["chk"].handle, rk["loc"].data_ptr(), stream)
            gathered = torch.cat([rk["loc"] for rk in ranks])
            for rk in ranks:
                rk["glob"] = gathered.clone()
                Z.neox_zero1_step_apply(rk["chk"].handle, rk["glob"].data_ptr(), float(lr), stream,
                                        nranks=D)
            sums = {Z.neox_scaler_state(rk["chk"].handle).last_sumsq for rk in ranks}
            assert len(sums) == 1, sums                  # the same bits on every rank
            j = 0
            for r, rk in enumerate(ranks):
                st = Z.neox_scaler_state(rk["chk"].handle)
                assert (st.loss_scale, st.step, st.skipped_total, st.last_skipped) == \
                    (ost.loss_scale, ost.step, ost.skipped_total, ost.last_skipped), (k, r)
                if not d.skip:
                    assert abs(st.last_grad_norm - ost.last_norm) <= 1e-5 * ost.last_norm
                    assert st.last_clip_coef < 1.0
                for i, s in enumerate(rk["shard"].segs):
                    p = pre[j]
                    j += 1
                    post = rk["shard"].host_window(i, 0, s["grad"].numel())
                    if d.skip:
                        for a in ("half", "master", "m", "v"):
                            assert np.array_equal(post[a], p[a]), (k, r, i, a)
                        continue
                    o = {a: p[a].copy() for a in ("grad", "half", "master", "m", "v")}
                    sm, sv, sw = O.update(ocfg, d, lr, o["grad"], o["half"], o["master"], o["m"],
                                          o["v"], rk["shard"].decay(i), scales=True)
                    tag = f" step {k} rank {r} seg {i}"
                    assert_close("exp_avg", post["m"], o["m"], sm, tag)
                    assert_close("exp_avg_sq", post["v"], o["v"], sv, tag)
                    assert_close("master", post["master"], o["master"], sw, tag)
                    assert_half_close(post["half"], o["half"], tag, rk["shard"].w.hyper.dtype,
                                      o["master"], sw)
            log(f"  step {k}: skip={d.skip} norm={ost.last_norm:.4g} ranks agree with the oracle")
        assert ost.skipped_total == 1
    finally:
        for rk in ranks:
            rk["chk"].close()


# ----------------------------------------------------------------------------------
# scaler set / reset
# ----------------------------------------------------------------------------------

def test_scaler_reset_after_collapse():
    """Drive the scale to its floor with overflows, reset it to 2^16 with
    neox_scaler_set (the OPT card's remedy), and keep matching the oracle."""
    w = _custom("reset", [40_000, 999], [True, False], min_scale=1.0)
    w.injections = {k: [(123 + k, "+inf")] for k in range(1, 19)}
    sh = DeviceShard(w)
    sh.init_()
    chk = Checker(sh)
    try:
        for k in range(20):
            if k == 19:
                st = Z.neox_scaler_state(chk.handle)
                assert st.loss_scale == 1.0 and st.consecutive_overflows == 18
                Z.neox_scaler_set(chk.handle, 65536.0, good_steps=0, step=st.step,
                                  skipped_total=st.skipped_total, consecutive_overflows=0,
                                  stream_ptr=torch.cuda.current_stream().cuda_stream)
                chk.ost.loss_scale, chk.ost.good_steps, chk.ost.consecutive_overflows = 65536.0, 0, 0
                st = Z.neox_scaler_state(chk.handle)
                assert (st.loss_scale, st.consecutive_overflows) == (65536.0, 0)
            sh.grads_(k, chk.scale())
            chk.step(6e-4, where=f" reset step {k}")
        assert chk.ost.step == 2 and chk.ost.skipped_total == 18
    finally:
        chk.close()


def test_scaler_set_rejects_bad_state():
    w = _custom("reset_bad", [1024], [True])
    sh = DeviceShard(w)
    sh.init_()
    h = Z.neox_zero1_create(lib_config(w), sh.neox_segments(), 0)
    try:
        for bad in (dict(loss_scale=0.0), dict(loss_scale=float("inf")),
                    dict(loss_scale=1.0, step=-1)):
            with pytest.raises(Z.NeoxError):
                Z.neox_scaler_set(h, **bad)
    finally:
        Z.neox_zero1_destroy(h)


# ----------------------------------------------------------------------------------
# per-segment telemetry
# ----------------------------------------------------------------------------------

def test_segment_norms_match_oracle():
    """Each segment's squared norm of the unscaled gradient matches the oracle's scan of
    that segment; they add up to the step's squared norm; an overflow shows in the
    segment that holds it."""
    sizes = [100_000, 3, 65_536, 17, 4096 * 5 + 1, 250_000]
    w = _custom("telemetry", sizes, [True, False, True, False, True, True])
    w.injections = {1: [(100_000 + 3 + 500, "nan")]}     # inside segment 2
    sh = DeviceShard(w)
    sh.init_()
    chk = Checker(sh, segment_norms=1)
    try:
        for k in range(3):
            sh.grads_(k, chk.scale())
            inv, inv32 = O.unscale_factor(chk.ocfg, chk.ost)
            want = [O.scan(W.F16, sh.host_window(i, 0, n)["grad"], inv, inv32) for i, (n, _) in
                    enumerate(w.segments)]
            chk.step(6e-4, where=f" telemetry step {k}")
            got = Z.neox_zero1_segment_sumsq(chk.handle, len(sizes))
            st = Z.neox_scaler_state(chk.handle)
            for i, ((ws, wof), g) in enumerate(zip(want, got)):
                if wof:
                    assert not np.isfinite(g), (k, i)
                else:
                    assert np.isfinite(g) and abs(g - ws) <= 1e-5 * ws, (k, i, g, ws)
            if not st.last_skipped:
                assert abs(sum(got) - st.last_sumsq) <= 1e-12 * st.last_sumsq
            else:
                assert k == 1 and [np.isfinite(g) for g in got] == [True, True, False, True, True, True]
    finally:
        chk.close()


@pytest.mark.parametrize("flat", [True, False], ids=["flat", "separate"])
def test_segment_norms_many_segments(flat):
    """2,000 segments of 1 .. 3,000 elements (many norm blocks, tiny segments): every
    segment's squared norm matches the oracle's scan of that segment, and they add up to
    the step's squared norm."""
    rng = np.random.default_rng(2000 + flat)
    sizes = [int(x) for x in rng.integers(1, 3001, 2000)]
    decays = [bool(x) for x in rng.integers(0, 2, 2000)]
    w = _custom("telemetry_many", sizes, decays)
    sh = DeviceShard(w, flat=flat)
    sh.init_()
    chk = Checker(sh, segment_norms=1)
    log(f"case telemetry 2000 segments flat={flat} n={sum(sizes)}")
    try:
        sh.grads_(0, chk.scale())
        inv, inv32 = O.unscale_factor(chk.ocfg, chk.ost)
        want = [O.scan(W.F16, sh.host_window(i, 0, n)["grad"], inv, inv32)[0]
                for i, n in enumerate(sizes)]
        chk.step(6e-4, check=False, where=" telemetry many")
        got = Z.neox_zero1_segment_sumsq(chk.handle, len(sizes))
        st = Z.neox_scaler_state(chk.handle)
        for i, (g, ws) in enumerate(zip(got, want)):
            assert abs(g - ws) <= 1e-5 * ws + 1e-300, (i, g, ws)
        assert abs(sum(got) - st.last_sumsq) <= 1e-12 * st.last_sumsq
    finally:
        chk.close()


# ----------------------------------------------------------------------------------
# momentum SGD
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [W.F16, W.BF16], ids=["f16", "bf16"])
@pytest.mark.parametrize("misalign", [(0, 0, 0, 0, 0), (1, 2, 3, 1, 0)], ids=["aligned", "mixed"])
def test_sgd_parity(dtype, misalign):
    """Momentum SGD (exp_avg = momentum, no second moment) on ragged segments, both
    formats, aligned and unaligned arrays, with one skipped step."""
    sizes = [1, 9, 255, 4097, 33_333, 8, 70_000]
    extra = dict(scaler_mode=W.STATIC, init_scale=1.0) if dtype == W.BF16 else {}
    w = _custom("sgd", sizes, [i % 2 == 0 for i in range(len(sizes))], dtype, optimizer=1,
                weight_decay=0.05, clip_norm=0.5, **extra)
    w.grad_sigma = 1e-3
    w.injections = {2: [(4000, "-inf")]}
    sh = DeviceShard(w, misalign=misalign)
    sh.init_()
    chk = Checker(sh, chunk_elems=1024)
    try:
        for k in range(5):
            sh.grads_(k, chk.scale())
            chk.step(1e-2, where=f" sgd step {k}")
        assert chk.ost.skipped_total == 1
    finally:
        chk.close()


# ----------------------------------------------------------------------------------
# graph capture
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["adamw", "sgd", "split"])
def test_step_replayed_from_a_hip_graph_matches_eager(mode):
    """The step enqueues only kernels (no allocation, no memset, no host sync), so a
    caller can capture it in a HIP graph: the whole step, the momentum-SGD step, or the
    split step's two halves around a device double.  Replays, with eager gradient
    generation and synchronisations between them and an overflow on one step, match the
    eager step bit for bit every time."""
    w = _custom("graph", [200_000, 777, 65_536], [True, False, True], clip_norm=0.01,
                optimizer=1 if mode == "sgd" else 0)
    w.injections = {3: [(1234, "+inf")]}
    log(f"case graph {mode}")
    eager, graphed = DeviceShard(w), DeviceShard(w)
    eager.init_()
    graphed.init_()
    stream = torch.cuda.current_stream().cuda_stream
    he = Z.neox_zero1_create(lib_config(w), eager.neox_segments(), stream)
    side = torch.cuda.Stream()
    hg = Z.neox_zero1_create(lib_config(w), graphed.neox_segments(), side.cuda_stream)
    g = torch.cuda.CUDAGraph()
    loc = torch.zeros(1, dtype=torch.float64, device="cuda")      # allocated before capture
    try:
        with torch.cuda.graph(g, stream=side):
            cap = torch.cuda.current_stream().cuda_stream
            if mode == "split":
                Z.neox_zero1_step_local(hg, loc.data_ptr(), cap)
                Z.neox_zero1_step_apply(hg, loc.data_ptr(), 1e-3, cap)
            else:
                Z.neox_zero1_step(hg, 1e-3, cap)
        torch.cuda.synchronize()
        for k in range(6):
            eager.grads_(k, Z.neox_scaler_state(he).loss_scale)
            graphed.buffers["grad"].copy_(eager.buffers["grad"])
            Z.neox_zero1_step(he, 1e-3, stream)
            g.replay()
            torch.cuda.synchronize()
            se, sg = Z.neox_scaler_state(he), Z.neox_scaler_state(hg)
            assert (se.loss_scale, se.step, se.skipped_total, se.last_sumsq) == \
                (sg.loss_scale, sg.step, sg.skipped_total, sg.last_sumsq), k
            oe, og = _outputs(eager), _outputs(graphed)
            for a in oe:
                assert torch.equal(oe[a], og[a]), (k, a)
        assert se.skipped_total == 1 and se.step == 5
    finally:
        del g
        Z.neox_zero1_destroy(he)
        Z.neox_zero1_destroy(hg)


# ----------------------------------------------------------------------------------
# per-kernel timing (what the benchmark's roofline reads)
# ----------------------------------------------------------------------------------

def test_timing_events_record_and_change_nothing():
    """Timed steps give the untimed steps' bits; all-kernel and update-only recordings
    count the steps they cover (up to max_steps), report positive durations that fit in
    the wall-clock time of those steps, and a new begin discards an unfinished one."""
    import time
    # separate allocations: the norm pass keeps 32K-element chunks (over 256 of them), so
    # the finalize is its own launch
    sizes = [9_000_000, 7, 1_000_001] + [33] * 130
    w = _custom("timing", sizes, [i % 2 == 0 for i in range(len(sizes))])
    stream = torch.cuda.current_stream().cuda_stream
    a, b = DeviceShard(w, flat=False), DeviceShard(w, flat=False)
    a.init_()
    b.init_()
    assert Z.neox_zero1_plan(lib_config(w), a.neox_segments(), tables=False)[0].update_decides == 0
    ha = Z.neox_zero1_create(lib_config(w), a.neox_segments(), stream)
    hb = Z.neox_zero1_create(lib_config(w), b.neox_segments(), stream)
    log("case timing events")
    try:
        def both(k):
            a.grads_(k, Z.neox_scaler_state(ha).loss_scale)
            b.grads_(k, Z.neox_scaler_state(hb).loss_scale)
            torch.cuda.synchronize()
            Z.neox_zero1_step(ha, 1e-3, stream)
            Z.neox_zero1_step(hb, 1e-3, stream)

        Z.neox_zero1_timing_begin(ha, 3)                 # all three kernels
        t0 = time.perf_counter()
        for k in range(4):                               # the 4th step is not recorded
            both(k)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3
        sums, n, per = Z.neox_zero1_timing_end(ha, per_step=3)
        assert n == 3 and all(s > 0.0 for s in sums), (n, sums)
        assert sum(sums) < wall_ms, (sums, wall_ms)
        # each step spans its three kernels and the gaps between them
        assert len(per) == 3 and sum(sums) <= sum(per) * 1.0001 and sum(per) < wall_ms, (per, sums)
        assert sums[2] > sums[1]                         # the update outlasts the finalize
        Z.neox_zero1_timing_begin(ha, 5)                 # discarded by the next begin
        both(4)
        Z.neox_zero1_timing_begin(ha, 5, update_only=True)
        for k in range(5, 7):
            both(k)
        sums, n, per = Z.neox_zero1_timing_end(ha, per_step=8)
        assert n == 2 and sums[0] == 0.0 and sums[1] == 0.0 and sums[2] > 0.0, (n, sums)
        assert len(per) == 2 and abs(sum(per) - sums[2]) <= 1e-6 * sums[2] + 1e-9, (per, sums)
        sa, sb = Z.neox_scaler_state(ha), Z.neox_scaler_state(hb)
        assert sa.step == sb.step == 7 and sa.last_sumsq == sb.last_sumsq
        # a shard whose norm pass has at most 256 blocks: the update takes the decisions
        # itself, no finalize is launched and its time reads 0
        small = DeviceShard(_custom("timing_small", [40_000, 3], [True, False]))
        small.init_()
        small.grads_(0, 65536.0)
        hs = Z.neox_zero1_create(lib_config(small.w), small.neox_segments(), stream)
        try:
            Z.neox_zero1_timing_begin(hs, 2)
            Z.neox_zero1_step(hs, 1e-3, stream)
            Z.neox_zero1_step(hs, 1e-3, stream)
            sums, n, per = Z.neox_zero1_timing_end(hs, per_step=2)
            assert n == 2 and sums[0] > 0.0 and sums[1] == 0.0 and sums[2] > 0.0, sums
            assert len(per) == 2 and sum(per) >= sums[0] + sums[2] - 1e-6, (per, sums)
            assert Z.neox_scaler_state(hs).step == 2
        finally:
            Z.neox_zero1_destroy(hs)
        oa, ob = _outputs(a), _outputs(b)
        for k in oa:
            assert torch.equal(oa[k], ob[k]), k
    finally:
        Z.neox_zero1_destroy(ha)
        Z.neox_zero1_destroy(hb)
