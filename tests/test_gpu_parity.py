"""GPU parity of the step against the oracle on small and mid-size shards.

Every case runs the library through its C ABI on the same bytes the oracle reads and
compares every element (see gpu_harness for the tolerances)."""
import numpy as np
import pytest
import torch

import mixed_precision_zero_amd as Z
import workloads as W
from gpu_harness import Checker, DeviceShard, lib_config, log

pytestmark = pytest.mark.gpu


def run_sequence(w, steps, lr=None, shard=None, where="", **cfg_over):
    shard = shard or DeviceShard(w)
    shard.init_()
    chk = Checker(shard, **cfg_over)
    lr = w.hyper.lr if lr is None else lr
    try:
        for k in range(steps):
            shard.grads_(k, chk.scale())
            chk.step(lr, where=f"{where} step {k}")
    finally:
        chk.close()
    return chk


def test_tiny_1m_sequence():
    """1,048,576 params, 10 steps, +inf at element 777,777 on step 5: the skip leaves
    every array untouched and halves the scale; all other steps match elementwise."""
    w = W.tiny()
    log("case tiny_1m")
    chk = run_sequence(w, w.steps, where="tiny_1m")
    assert chk.ost.skipped_total == 1 and chk.ost.step == 9
    assert chk.ost.loss_scale == 32768.0


def _custom(name, sizes, decays, dtype=W.F16, **hy):
    hyper = W.Hyper(dtype=dtype, **hy)
    if dtype == W.BF16:
        hyper.scaler_mode = hy.get("scaler_mode", W.STATIC)
        hyper.init_scale = hy.get("init_scale", 1.0)
    return W.Workload(name, 900, list(zip(sizes, decays)), hyper, steps=4)


@pytest.mark.parametrize("dtype", [W.F16, W.BF16], ids=["f16", "bf16"])
@pytest.mark.parametrize("misalign", [(0, 0, 0, 0, 0), (3, 3, 3, 3, 3), (1, 2, 0, 3, 1)],
                         ids=["aligned", "same_offset", "mixed_offsets"])
def test_tiny_shards_bruteforce(dtype, misalign):
    """Random segment splits of 1..64 elements, random decay flags, both half formats,
    aligned / consistently offset / inconsistently offset arrays, and an inf or NaN
    injected at a random element on one step."""
    rng = np.random.default_rng(100 + dtype * 10 + sum(misalign))
    for case in range(12):
        n = int(rng.integers(1, 65))
        cuts = sorted(set(int(c) for c in rng.integers(1, n, size=int(rng.integers(0, 4))))) if n > 1 else []
        sizes = np.diff([0] + cuts + [n]).tolist()
        decays = [bool(x) for x in rng.integers(0, 2, len(sizes))]
        w = _custom(f"tiny{case}", sizes, decays, dtype, clip_norm=float(rng.choice([0.0, 1e-3, 1.0])))
        w.grad_sigma = float(rng.choice([1e-4, 1e-2]))
        kind = ["+inf", "-inf", "nan"][case % 3]
        w.injections = {2: [(int(rng.integers(0, n)), kind)]}
        log(f"case tiny dtype={dtype} misalign={misalign} n={n} sizes={sizes}")
        chk = run_sequence(w, 4, shard=DeviceShard(w, flat=True, misalign=misalign),
                           where=f" n={n}")
        assert chk.ost.skipped_total == 1


@pytest.mark.parametrize("dtype", [W.F16, W.BF16], ids=["f16", "bf16"])
def test_ragged_many_chunks(dtype):
    """~70k elements in segments of awkward lengths, 256-element chunks (hundreds of
    blocks, ragged tails) and a 3-block norm pass looping over them."""
    sizes = [1, 7, 8, 9, 255, 256, 257, 4095, 4097, 12_345, 33_333, 8, 1000, 15_000]
    decays = [i % 3 != 0 for i in range(len(sizes))]
    w = _custom("ragged", sizes, decays, dtype)
    log(f"case ragged dtype={dtype}")
    run_sequence(w, 3, chunk_elems=256, norm_blocks=3, where=" ragged")
    run_sequence(w, 2, shard=DeviceShard(w, flat=False, misalign=(1, 1, 1, 1, 1)),
                 chunk_elems=512, where=" ragged separate")


def _outputs(shard):
    torch.cuda.synchronize()
    return {k: torch.cat([s[k].reshape(-1) for s in shard.segs]).clone()
            for k in ("half", "master", "m", "v")}


def test_chunking_and_grid_independence_and_determinism():
    """Elementwise outputs are bitwise independent of the chunk size and of the norm
    pass's grid; the same configuration run twice is bitwise identical, norm included."""
    sizes = [100_000, 3, 77_777, 8192, 1]
    w = _custom("chunking", sizes, [True, False, True, False, True], clip_norm=0.01)
    results = []
    for chunk, blocks in ((0, 0), (0, 0), (256, 1), (1024, 7), (65536, 2)):
        log(f"case chunking chunk={chunk} blocks={blocks}")
        shard = DeviceShard(w)
        shard.init_()
        h = Z.neox_zero1_create(lib_config(w, chunk_elems=chunk, norm_blocks=blocks),
                                shard.neox_segments(), torch.cuda.current_stream().cuda_stream)
        norms = []
        for k in range(3):
            shard.grads_(k, Z.neox_scaler_state(h).loss_scale)
            Z.neox_zero1_step(h, 1e-3, torch.cuda.current_stream().cuda_stream)
            st = Z.neox_scaler_state(h)
            norms.append((st.last_grad_norm, st.last_sumsq))
        Z.neox_zero1_destroy(h)
        results.append((_outputs(shard), norms))
    base, base_norms = results[0]
    again, again_norms = results[1]
    for k in base:
        assert torch.equal(base[k], again[k]), k
    assert base_norms == again_norms
    for out, norms in results[2:]:
        for k in base:
            assert torch.equal(out[k], base[k]), k
        for (a, _), (b, _) in zip(norms, base_norms):
            assert abs(a - b) <= 1e-5 * b


def test_subnormals_kept():
    """Tiny gradients drive v into the FP32 subnormal range and tiny weights give fp16
    subnormal half copies; both must match the oracle (no flush to zero)."""
    w = _custom("subnormal", [4096], [True])
    w.grad_sigma = 1e-21
    w.master_sigma = 1e-6
    w.hyper.init_scale = 2.0 ** 60
    log("case subnormals")
    run_sequence(w, 3, clip_norm=0.0, where=" subnormal")


def test_overflow_from_unscale_factor():
    """bf16 gradients with a scale below one: finite gradients whose FP32 unscaled
    value overflows must skip, exactly as the oracle decides in FP32."""
    w = _custom("bf16_big", [1000], [True], W.BF16, scaler_mode=W.DYNAMIC,
                init_scale=2.0 ** -10, min_scale=2.0 ** -20)
    shard = DeviceShard(w)
    shard.init_()
    chk = Checker(shard)
    try:
        big = torch.full((1000,), 2.0 ** 120, dtype=torch.bfloat16, device="cuda")
        shard.segs[0]["grad"].copy_(big)
        gst, d = chk.step(1e-3, where=" overflow")
        assert d.skip == 1 and gst.loss_scale == 2.0 ** -11
        W.device_grads_(w, shard.segs[0]["grad"], 1, 1.0)
        gst, d = chk.step(1e-3, where=" clean")
        assert d.skip == 0
    finally:
        chk.close()


def test_overflow_decided_on_the_fp32_product():
    """x = (1 + 2^-7) 2^126 in bf16 times a pre-divide factor whose FP32 rounding pushes
    the product past the FP32 range (the exact product stays below it): the step skips,
    as the oracle decides in FP32; without that element the step is clean."""
    x, inv = (1 + 2.0 ** -7) * 2.0 ** 126, 3.9689921219219535
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(x) * np.float32(inv)) and np.isfinite(np.float32(x * inv))
    w = _custom("fp32_window", [1000], [True], W.BF16, predivide_factor=inv)
    shard = DeviceShard(w)
    shard.init_()
    chk = Checker(shard)
    try:
        W.device_grads_(w, shard.segs[0]["grad"], 0, 1.0)
        shard.segs[0]["grad"][517] = x
        assert float(shard.segs[0]["grad"][517]) == x
        gst, d = chk.step(1e-3, where=" fp32 window")
        assert d.skip == 1 and gst.skipped_total == 1
        W.device_grads_(w, shard.segs[0]["grad"], 1, 1.0)
        gst, d = chk.step(1e-3, where=" clean")
        assert d.skip == 0
    finally:
        chk.close()


def test_resume_equals_continuous():
    """N steps, destroy, re-create with the state read back, M steps == N+M steps."""
    w = _custom("resume", [30_000, 2048], [True, False], growth_interval=2)
    w.injections = {1: [(5, "nan")]}
    a = DeviceShard(w)
    a.init_()
    ha = Z.neox_zero1_create(lib_config(w), a.neox_segments(), 0)
    stream = torch.cuda.current_stream().cuda_stream
    for k in range(6):
        a.grads_(k, Z.neox_scaler_state(ha).loss_scale)
        Z.neox_zero1_step(ha, 1e-3, stream)
    ref = Z.neox_scaler_state(ha)
    Z.neox_zero1_destroy(ha)

    b = DeviceShard(w)
    b.init_()
    hb = Z.neox_zero1_create(lib_config(w), b.neox_segments(), 0)
    for k in range(3):
        b.grads_(k, Z.neox_scaler_state(hb).loss_scale)
        Z.neox_zero1_step(hb, 1e-3, stream)
    st = Z.neox_scaler_state(hb)
    Z.neox_zero1_destroy(hb)
    hb = Z.neox_zero1_create(
        lib_config(w, init_scale=st.loss_scale, init_step=st.step, init_skipped=st.skipped_total,
                   init_good_steps=st.good_steps,
                   init_consecutive_overflows=st.consecutive_overflows),
        b.neox_segments(), 0)
    for k in range(3, 6):
        b.grads_(k, Z.neox_scaler_state(hb).loss_scale)
        Z.neox_zero1_step(hb, 1e-3, stream)
    st2 = Z.neox_scaler_state(hb)
    Z.neox_zero1_destroy(hb)
    assert (st2.loss_scale, st2.step, st2.skipped_total, st2.good_steps) == \
        (ref.loss_scale, ref.step, ref.skipped_total, ref.good_steps)
    oa, ob = _outputs(a), _outputs(b)
    for k in oa:
        assert torch.equal(oa[k], ob[k]), k


@pytest.mark.parametrize("t0", [996, 4093, 123_457, 2 ** 40 + 3])
def test_parity_after_restored_step_count(t0):
    """A handle created at a large step count (a restored run): the bias corrections
    1 - beta^t of the next steps match the oracle's.  With both betas at 0.999, beta^t is
    about 0.37 and 0.017 in the first two cases (long exponent chains that still matter),
    negligible in the third and zero (underflow) in the last."""
    w = _custom(f"restored{t0}", [40_000, 3, 9000], [True, False, True])
    log(f"case restored step {t0}")
    for beta1, beta2 in ((0.9, 0.95), (0.999, 0.999)):
        w.hyper.beta1, w.hyper.beta2 = beta1, beta2
        chk = run_sequence(w, 3, init_step=t0, where=f" t0={t0} betas={beta1},{beta2}")
        assert chk.ost.step == t0 + 3


_DEGENERATE = {
    "zero_grad": {},                                # gradient all zero: norm 0, only decay moves w
    "betas_zero": dict(beta1=0.0, beta2=0.0),       # Adam reduces to g / (|g| + eps)
    "eps_tiny": dict(eps=1e-45),                    # smallest positive FP32 (eps 0 is refused)
    "lr_zero": {},                                  # w and half unchanged, m and v move
    "no_decay": dict(weight_decay=0.0),
}


@pytest.mark.parametrize("case", sorted(_DEGENERATE))
def test_degenerate_hyperparameters(case):
    """Settings at the edge of what the method admits, against the oracle, on a flat
    shard and on separately allocated, misaligned arrays: clipping must not divide by a
    zero norm, and the arithmetic must not special-case any of them."""
    w = _custom(f"degenerate_{case}", [5000, 3, 2048, 777], [True, False, True, False],
                **_DEGENERATE[case])
    if case == "zero_grad":
        w.grad_sigma = 0.0
    lr = 0.0 if case == "lr_zero" else None
    log(f"case degenerate {case}")
    for shard in (DeviceShard(w, flat=True), DeviceShard(w, flat=False, misalign=(1, 2, 1, 3, 1))):
        chk = run_sequence(w, 3, lr=lr, shard=shard, where=f" {case}")
        assert chk.ost.skipped_total == 0 and chk.ost.step == 3
        if case == "zero_grad":
            assert chk.ost.last_sumsq == 0.0 and chk.ost.last_coef == 1.0


@pytest.mark.parametrize("seed", range(8))
def test_random_hyperparameters(seed):
    """Seeded random draws of every hyper-parameter at once (betas, eps, weight decay,
    clip threshold, lr, pre-divide factor and rank count, half format, scaler mode,
    optimizer) on a random segment layout, flat or separately allocated, three steps
    against the oracle."""
    rng = np.random.default_rng(4000 + seed)
    dtype = [W.F16, W.BF16][seed % 2]
    nseg = int(rng.integers(1, 6))
    sizes = [int(x) for x in rng.integers(1, 20_000, nseg)]
    decays = [bool(x) for x in rng.integers(0, 2, nseg)]
    f = float(2.0 ** rng.integers(0, 4))
    D = int(2 ** rng.integers(0, 4))
    hy = dict(beta1=float(rng.choice([0.0, 0.5, 0.9, 0.99])),
              beta2=float(rng.choice([0.0, 0.9, 0.95, 0.999])),
              eps=float(rng.choice([1e-8, 1e-6, 1e-3])),
              weight_decay=float(rng.choice([0.0, 0.01, 0.1])),
              clip_norm=float(rng.choice([0.0, 0.3, 1.0, 10.0])),
              predivide_factor=f, dp_world_size=D)
    sigma = float(rng.choice([1e-5, 1e-3, 1e-1]))
    if dtype == W.F16:
        # the largest scale at which 6 sigma of the stored gradient stays finite in fp16
        # after up to three growths (no step may skip)
        top = int(np.floor(np.log2(65504.0 / (6 * 8 * sigma * D / f))))
        hy.update(scaler_mode=W.DYNAMIC, init_scale=float(2.0 ** max(0, min(16, top))),
                  growth_interval=int(rng.integers(1, 4)))
    w = _custom(f"random_hyper{seed}", sizes, decays, dtype, **hy)
    w.grad_sigma = sigma
    w.grad_mult = D / f              # the stored gradient is summed over D ranks, each / f
    lr = float(rng.choice([1e-5, 6e-4, 1e-2]))
    flat = bool(seed % 3)
    mis = (0, 0, 0, 0, 0) if flat else tuple(int(x) for x in rng.integers(0, 4, 5))
    w.hyper.optimizer = int(rng.integers(0, 2))      # AdamW or momentum SGD
    log(f"case random hyper seed={seed} dtype={dtype} sizes={sizes} hyper={hy} lr={lr} "
        f"flat={flat} optimizer={w.hyper.optimizer}")
    chk = run_sequence(w, 3, lr=lr, shard=DeviceShard(w, flat=flat, misalign=mis),
                       where=f" seed={seed}")
    assert chk.ost.skipped_total == 0 and chk.ost.step == 3


def test_zero1_wrapper_equals_raw_calls():
    """The Python convenience class (create on the current stream, step, state, close)
    produces bitwise the raw C-ABI calls' results; a closed handle refuses to step."""
    w = _custom("wrapper", [12_345, 7, 4096], [True, False, True])
    a, b = DeviceShard(w), DeviceShard(w)
    a.init_()
    b.init_()
    log("case Zero1 wrapper")
    opt = Z.Zero1(lib_config(w), a.neox_segments())
    stream = torch.cuda.current_stream().cuda_stream
    h = Z.neox_zero1_create(lib_config(w), b.neox_segments(), stream)
    try:
        for k in range(3):
            a.grads_(k, opt.state().loss_scale)
            b.grads_(k, Z.neox_scaler_state(h).loss_scale)
            opt.step(lr=6e-4)
            Z.neox_zero1_step(h, 6e-4, stream)
        sa, sb = opt.state(), Z.neox_scaler_state(h)
        assert (sa.step, sa.loss_scale, sa.last_sumsq) == (sb.step, sb.loss_scale, sb.last_sumsq)
        oa, ob = _outputs(a), _outputs(b)
        for k in oa:
            assert torch.equal(oa[k], ob[k]), k
    finally:
        opt.close()
        Z.neox_zero1_destroy(h)
    with pytest.raises(Z.NeoxError):
        opt.step(lr=6e-4)


def _path(w, shard, **over):
    h = Z.neox_zero1_create(lib_config(w, **over), shard.neox_segments(),
                            torch.cuda.current_stream().cuda_stream)
    try:
        return Z.neox_zero1_update_path(h)
    finally:
        Z.neox_zero1_destroy(h)


def test_update_path_selection():
    """The flat update runs exactly for a flat, 16-byte-aligned partition with the default
    chunk size and chunked_update 0; every other layout takes the chunk table."""
    w = _custom("paths", [5000, 3, 9000], [True, False, True])
    flat = DeviceShard(w, flat=True)
    assert _path(w, flat) == Z.NEOX_PATH_FLAT
    assert _path(w, flat, chunked_update=1) == Z.NEOX_PATH_CHUNKED
    assert _path(w, flat, chunk_elems=4096) == Z.NEOX_PATH_CHUNKED
    assert _path(w, DeviceShard(w, flat=True, misalign=(0, 0, 1, 0, 0))) == Z.NEOX_PATH_CHUNKED
    assert _path(w, DeviceShard(w, flat=False)) == Z.NEOX_PATH_CHUNKED
    ws = _custom("paths_sgd", [5000, 3, 9000], [True, False, True], optimizer=1)
    assert _path(ws, DeviceShard(ws, flat=True), optimizer=1) == Z.NEOX_PATH_FLAT


# Segment lengths that put flag changes at 2,048- and 4,096-element boundaries, mid-tile,
# inside one 8-element vector and several to a tile, over tens of full tiles and a
# ragged last one with a scalar tail (55,499 elements).
_MIXED_SIZES = [1, 4095, 4096, 7, 1, 9, 3000, 1096, 100, 100, 100, 8184, 5, 3, 17, 4096,
                12_288, 2, 2, 2, 2, 2, 2, 2, 2, 8190, 6000, 2, 4093]
_MIXED_DECAY = [i % 2 == 0 for i in range(len(_MIXED_SIZES))]


@pytest.mark.parametrize("dtype", [W.F16, W.BF16], ids=["f16", "bf16"])
def test_flat_mixed_decay_tiles(dtype):
    """Flat update on tiles holding several segments with alternating decay flags, with an
    overflow (skipped step) in a full tile: every element against the oracle."""
    w = _custom("mixed_tiles", _MIXED_SIZES, _MIXED_DECAY, dtype, weight_decay=0.5)
    w.injections = {2: [(20_000, "nan")]}
    shard = DeviceShard(w, flat=True)
    assert _path(w, shard) == Z.NEOX_PATH_FLAT
    log(f"case flat mixed tiles dtype={dtype} n={w.numel}")
    chk = run_sequence(w, 5, shard=shard, where=" flat mixed")
    assert chk.ost.skipped_total == 1 and w.numel % 8 != 0 and w.numel > 13 * 4096


@pytest.mark.parametrize("optimizer", [0, 1], ids=["adamw", "sgd"])
def test_flat_equals_chunked_bitwise(optimizer):
    """Both update kernels run the same arithmetic, so on the same inputs they agree bit
    for bit: master, m, v, half and the scaler state, over clean and skipped steps.  (With
    per-segment norms, so that both norm passes cut the same chunks: a flat partition's
    norm chunks otherwise run across segment bounds, which changes the squared norm's
    summation order.)"""
    w = _custom("flat_vs_chunked", _MIXED_SIZES * 3, _MIXED_DECAY * 3, optimizer=optimizer,
                weight_decay=0.5)
    w.injections = {1: [(70_000, "+inf")], 3: [(w.numel - 1, "-inf")]}
    stream = torch.cuda.current_stream().cuda_stream
    outs, states = [], []
    for chunked in (0, 1):
        shard = DeviceShard(w, flat=True)
        shard.init_()
        h = Z.neox_zero1_create(lib_config(w, chunked_update=chunked, optimizer=optimizer,
                                           segment_norms=1),
                                shard.neox_segments(), stream)
        assert Z.neox_zero1_update_path(h) == (Z.NEOX_PATH_CHUNKED if chunked else Z.NEOX_PATH_FLAT)
        log(f"case flat vs chunked optimizer={optimizer} chunked={chunked}")
        for k in range(6):
            shard.grads_(k, Z.neox_scaler_state(h).loss_scale)
            Z.neox_zero1_step(h, 1e-3, stream)
        st = Z.neox_scaler_state(h)
        states.append((st.loss_scale, st.step, st.skipped_total, st.good_steps, st.last_sumsq))
        Z.neox_zero1_destroy(h)
        torch.cuda.synchronize()
        outs.append({k: torch.cat([s[k].reshape(-1) for s in shard.segs]).clone()
                     for k in (("half", "master", "m") if optimizer else ("half", "master", "m", "v"))})
    assert states[0] == states[1] and states[0][2] == 2
    for k in outs[0]:
        assert torch.equal(outs[0][k], outs[1][k]), k


def test_argument_errors_enqueue_nothing():
    """Calls rejected by validation (non-finite lr, misaligned or null device doubles,
    wrong telemetry length, bad timing requests) return NEOX_EINVAL and leave the state
    and every array untouched."""
    import ctypes as C
    w = _custom("errors", [5000, 3], [True, False])
    shard = DeviceShard(w)
    shard.init_()
    shard.grads_(0, w.hyper.init_scale)
    stream = torch.cuda.current_stream().cuda_stream
    h = Z.neox_zero1_create(lib_config(w), shard.neox_segments(), stream)
    L = Z.lib()
    try:
        before = _outputs(shard)
        st0 = Z.neox_scaler_state(h)
        d = torch.zeros(2, dtype=torch.float64, device="cuda")
        for lr in (float("nan"), float("inf"), float("-inf")):
            assert L.neox_zero1_step(C.c_void_p(h), C.c_float(lr), C.c_void_p(stream)) == Z.NEOX_EINVAL
            assert L.neox_zero1_step_apply(C.c_void_p(h), C.c_void_p(d.data_ptr()), 1, C.c_float(lr),
                                           C.c_void_p(stream)) == Z.NEOX_EINVAL
        odd = d.data_ptr() + 4
        assert L.neox_zero1_step_local(C.c_void_p(h), C.c_void_p(odd), C.c_void_p(stream)) == Z.NEOX_EINVAL
        assert L.neox_zero1_step_apply(C.c_void_p(h), C.c_void_p(odd), 1, C.c_float(1e-3),
                                       C.c_void_p(stream)) == Z.NEOX_EINVAL
        assert L.neox_zero1_step_apply(C.c_void_p(h), C.c_void_p(d.data_ptr()), 0, C.c_float(1e-3),
                                       C.c_void_p(stream)) == Z.NEOX_EINVAL
        assert L.neox_zero1_step_local(C.c_void_p(h), None, C.c_void_p(stream)) == Z.NEOX_EINVAL
        out = (C.c_double * 2)()
        assert L.neox_zero1_segment_sumsq(C.c_void_p(h), out, 2) == Z.NEOX_EINVAL   # telemetry off
        for steps, upd in ((0, 0), (-1, 0), (4, 2)):
            assert L.neox_zero1_timing_begin(C.c_void_p(h), steps, upd) == Z.NEOX_EINVAL
        assert Z.neox_zero1_update_path(h) in (Z.NEOX_PATH_FLAT, Z.NEOX_PATH_CHUNKED)
        st1 = Z.neox_scaler_state(h)
        assert (st1.step, st1.skipped_total, st1.loss_scale, st1.good_steps) == \
            (st0.step, st0.skipped_total, st0.loss_scale, st0.good_steps)
        after = _outputs(shard)
        for k in before:
            assert torch.equal(before[k], after[k]), k
    finally:
        Z.neox_zero1_destroy(h)


@pytest.mark.parametrize("sizes", [[2048], [1000, 1048], [4096, 7, 2041, 2048], [8, 8192 - 8]],
                         ids=["one_tile", "two_segments", "three_tiles", "four_tiles"])
def test_flat_shard_of_whole_tiles(sizes):
    """Flat shards that end exactly on a tile boundary (no short last tile), with a flag
    change inside a tile, against the oracle, one step skipped."""
    decays = [i % 2 == 0 for i in range(len(sizes))]
    w = _custom("whole_tiles", sizes, decays, weight_decay=0.5)
    w.injections = {1: [(sum(sizes) - 1, "nan")]}
    shard = DeviceShard(w, flat=True)
    plan = Z.neox_zero1_plan(lib_config(w), shard.neox_segments(), tables=False)[0]
    assert plan.update_path == Z.NEOX_PATH_FLAT and w.numel % plan.tile_elems == 0
    log(f"case whole tiles {sizes}")
    chk = run_sequence(w, 3, shard=shard, where=f" whole tiles {sizes}")
    assert chk.ost.skipped_total == 1


def test_norm_chunks_across_many_segments():
    """A flat partition of 600 segments (~2.7M elements, bf16, clipping active): its norm
    pass cuts the gradient into at most 256 large chunks across segment bounds and the
    update decides.  Every element against the oracle over three steps, the second with
    a NaN; then the same shard with per-segment norms, whose 600+ chunks follow the
    segments and keep the finalize launch."""
    rng = np.random.default_rng(61)
    sizes = [int(x) for x in rng.integers(1, 9000, 600)]
    decays = [bool(x) for x in rng.integers(0, 2, 600)]
    w = _custom("many_segments", sizes, decays, W.BF16, clip_norm=0.05)
    w.injections = {1: [(int(rng.integers(0, w.numel)), "nan")]}
    for seg_norms, decides in ((0, 1), (1, 0)):
        shard = DeviceShard(w, flat=True)
        plan = Z.neox_zero1_plan(lib_config(w, segment_norms=seg_norms), shard.neox_segments(),
                                 tables=False)[0]
        assert plan.update_path == Z.NEOX_PATH_FLAT and plan.update_decides == decides
        assert (plan.norm_chunks <= 256) == bool(decides) and (plan.norm_block_threads == 512) == bool(decides)
        log(f"case many segments segment_norms={seg_norms}: {w.numel} elements, "
            f"{plan.norm_chunks} norm chunks")
        chk = run_sequence(w, 3, shard=shard, where=f" many segments {seg_norms}",
                           segment_norms=seg_norms)
        assert chk.ost.skipped_total == 1 and chk.ost.last_coef < 1.0


# Shard sizes on either side of the library's size-dependent launch choices: the AdamW
# update runs 4 blocks per CU up to 48 grid blocks per CU, else 2 (on 256 CUs: 12,288
# tiles of 2,048 elements), and the norm pass keeps the gradient cached up to 2^24
# elements.  Results must not depend on them.
_BOUNDARY_SIZES = {
    "grid_48_per_cu": (12288 * 2048, W.F16),
    "grid_48_per_cu_plus_one_tile": (12288 * 2048 + 2048, W.F16),
    "cached_norm_2e24": (1 << 24, W.F16),
    "uncached_norm_2e24_plus_ragged": ((1 << 24) + 2048 + 5, W.F16),
    "grid_48_per_cu_plus_ragged_bf16": (12288 * 2048 + 3, W.BF16),
    "large_norm_blocks_bf16": (3_000_007, W.BF16),
    "short_norm_chunks_2e6": (64 * 32767, W.F16),
}


@pytest.mark.parametrize("case", sorted(_BOUNDARY_SIZES))
def test_launch_choice_boundaries(case):
    """Every element against the oracle for two steps (the second with clipping active)
    at each size-dependent launch boundary, on a flat two-segment shard; the norm pass
    runs as large blocks above 64 chunks of 32K elements and the update decides."""
    n, dtype = _BOUNDARY_SIZES[case]
    w = _custom(f"boundary_{case}", [n - 4099, 4099], [True, False], dtype=dtype, clip_norm=0.05)
    shard = DeviceShard(w, flat=True)
    plan = Z.neox_zero1_plan(lib_config(w), shard.neox_segments(), tables=False)[0]
    assert plan.update_decides == 1
    assert plan.norm_block_threads == (512 if -(-n // 64) >= 32768 else 256), plan.norm_block_threads
    log(f"case launch boundary {case}: {n} elements")
    shard.init_()
    chk = Checker(shard)
    try:
        for k in range(2):
            shard.grads_(k, chk.scale())
            chk.step(w.hyper.lr, threads=16, where=f" {case} step {k}")
    finally:
        chk.close()
    assert chk.ost.step == 2 and chk.ost.last_coef < 1.0


# The chunk table of a two-segment shard (the second segment 4,099 elements) has 12,288
# entries (48 per CU on 256 CUs) at the first size and 12,290 at the second.
_TABLE_BOUNDARY_SIZES = {"table_48_per_cu": 12288 * 2048 - 2048,
                         "table_49_per_cu": 12288 * 2048 + 2048}


@pytest.mark.parametrize("case", sorted(_TABLE_BOUNDARY_SIZES))
def test_launch_choice_boundaries_chunk_table(case):
    """The same AdamW cut in the chunk-table update: every element against the oracle
    for two steps (the second with clipping active) on either side of it."""
    n, dtype = _TABLE_BOUNDARY_SIZES[case], W.F16
    w = _custom(f"boundary_table_{case}", [n - 4099, 4099], [True, False], dtype=dtype,
                clip_norm=0.05)
    shard = DeviceShard(w, flat=True)
    plan = Z.neox_zero1_plan(lib_config(w, chunked_update=1), shard.neox_segments(),
                             tables=False)[0]
    assert plan.update_path == Z.NEOX_PATH_CHUNKED
    assert (plan.update_chunks <= 48 * 256) == (case == "table_48_per_cu"), plan.update_chunks
    log(f"case launch boundary {case} on the chunk table: {n} elements, "
        f"{plan.update_chunks} chunks")
    shard.init_()
    chk = Checker(shard, chunked_update=1)
    try:
        for k in range(2):
            shard.grads_(k, chk.scale())
            chk.step(w.hyper.lr, threads=16, where=f" {case} chunk table step {k}")
    finally:
        chk.close()
    assert chk.ost.step == 2 and chk.ost.last_coef < 1.0


# Momentum SGD runs 4 blocks per CU up to 64 grid blocks per CU and 2 beyond (on 256 CUs:
# 16,384 tiles or chunks of 2,048 elements), in both update kernels.  Sizes per kernel
# (the chunk table also counts the second segment's head and tail chunks): the first of
# each pair has a grid of 16,384 blocks, the second one of more.
_SGD_BOUNDARY_SIZES = {
    ("grid_64_per_cu", 0): 16384 * 2048,
    ("grid_64_per_cu_plus_ragged", 0): 16384 * 2048 + 2048 + 3,
    ("grid_64_per_cu", 1): 16384 * 2048 - 2048,
    ("grid_64_per_cu_plus_ragged", 1): 16384 * 2048 + 2048 + 3,
}


@pytest.mark.parametrize("chunked", [0, 1], ids=["flat", "chunk_table"])
@pytest.mark.parametrize("case", ["grid_64_per_cu", "grid_64_per_cu_plus_ragged"])
def test_sgd_launch_choice_boundaries(case, chunked):
    """Momentum SGD, every element against the oracle for two steps (the second with
    clipping active) on either side of its blocks-per-CU boundary, in the flat and the
    chunk-table update."""
    n = _SGD_BOUNDARY_SIZES[(case, chunked)]
    w = _custom(f"sgd_boundary_{case}", [n - 4099, 4099], [True, False], optimizer=1,
                weight_decay=0.05, clip_norm=0.05)
    shard = DeviceShard(w, flat=True)
    plan = Z.neox_zero1_plan(lib_config(w, chunked_update=chunked), shard.neox_segments(),
                             tables=False)[0]
    grid = plan.update_chunks if chunked else plan.flat_tiles
    assert (grid <= 64 * 256) == (case == "grid_64_per_cu"), grid
    assert plan.update_path == (Z.NEOX_PATH_CHUNKED if chunked else Z.NEOX_PATH_FLAT)
    log(f"case sgd launch boundary {case} chunked={chunked}: {n} elements")
    shard.init_()
    chk = Checker(shard, chunked_update=chunked)
    try:
        for k in range(2):
            shard.grads_(k, chk.scale())
            chk.step(1e-2, threads=16, where=f" sgd {case} chunked={chunked} step {k}")
    finally:
        chk.close()
    assert chk.ost.step == 2 and chk.ost.last_coef < 1.0
