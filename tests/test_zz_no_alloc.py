"""neox_zero1_step_noalloc (the entry point for callers that cannot allocate device
memory) against neox_zero1_step on identical inputs, through the C ABI.  (Named to be
collected last: the GPU suite runs with -x.)

Both run the same kernels, so every array and every scaler field must agree bit for bit.
Two calls in a row, the second on a smaller input with another layout: a flat fp16
partition of four segments (three steps, the second with an inf in the gradient, so the
scaler state carried between calls goes through a skip), then separately allocated,
misaligned bf16 arrays that take the chunk-table update.  The first call's applied
steps are also held to the oracle's tolerances (the second call's are covered by the
same comparison with neox_zero1_step, which the parity tests hold to the oracle)."""
import numpy as np
import pytest
import torch

import mixed_precision_zero_amd as Z
import workloads as W
from gpu_harness import ARRAYS, Checker, DeviceShard, lib_config, log

pytestmark = pytest.mark.gpu


def _clone_shard(src: DeviceShard, misalign=(0, 0, 0, 0, 0)) -> DeviceShard:
    dst = DeviceShard(src.w, flat=src.flat, misalign=misalign)
    for a, b in zip(src.segs, dst.segs):
        for k in ARRAYS:
            if a[k] is not None:
                b[k].copy_(a[k])
    return dst


def _state_from_config(cfg) -> Z.neox_scaler_state_t:
    st = Z.neox_scaler_state_t()
    st.loss_scale = float(np.float32(cfg.init_scale))
    st.good_steps = cfg.init_good_steps
    st.step = cfg.init_step
    st.skipped_total = cfg.init_skipped
    st.consecutive_overflows = cfg.init_consecutive_overflows
    return st


def _assert_same_arrays(a: DeviceShard, b: DeviceShard, where):
    torch.cuda.synchronize()
    for i, (sa, sb) in enumerate(zip(a.segs, b.segs)):
        for k in ("half", "master", "m", "v"):
            if sa[k] is not None:
                assert torch.equal(sa[k].view(torch.int16 if sa[k].element_size() == 2 else torch.int32),
                                   sb[k].view(torch.int16 if sb[k].element_size() == 2 else torch.int32)), \
                    f"{k} of segment {i} differs{where}"


def _assert_same_state(got: Z.neox_scaler_state_t, want: Z.neox_scaler_state_t, where):
    fields = ("loss_scale", "good_steps", "step", "skipped_total", "consecutive_overflows",
              "last_skipped", "last_grad_norm", "last_clip_coef", "last_sumsq")
    for f in fields:
        g, w = getattr(got, f), getattr(want, f)
        assert (g == w) or (np.isnan(g) and np.isnan(w)), f"{f}: noalloc {g!r} step {w!r}{where}"


def _run_pair(w: W.Workload, steps, flat, misalign, oracle_check):
    """Steps a handle (with the oracle beside it when oracle_check) and the no-alloc entry
    point on copies of the same arrays; compares them after every step."""
    ref = DeviceShard(w, flat=flat, misalign=misalign)
    ref.init_()
    mine = _clone_shard(ref, misalign)
    stream = torch.cuda.current_stream()
    chk = Checker(ref, stream=stream)
    cfg = lib_config(w)
    st = _state_from_config(cfg)
    try:
        for k in range(steps):
            scale = chk.scale()
            assert scale == st.loss_scale
            ref.grads_(k, scale)
            for sa, sb in zip(ref.segs, mine.segs):
                sb["grad"].copy_(sa["grad"])
            injected = bool(w.injections.get(k))
            if oracle_check:
                chk.step(w.hyper.lr, overflow=True if injected else None, check=True,
                         where=f" {w.name} step {k}")
            else:
                Z.neox_zero1_step(chk.handle, w.hyper.lr, stream.cuda_stream)
            Z.neox_zero1_step_noalloc(cfg, mine.neox_segments(), st, w.hyper.lr, stream.cuda_stream)
            where = f" ({w.name} step {k})"
            _assert_same_state(st, Z.neox_scaler_state(chk.handle), where)
            _assert_same_arrays(mine, ref, where)
            assert st.last_skipped == int(injected), where
            log(f"  {w.name} step {k}: noalloc == step (skipped={st.last_skipped})")
    finally:
        chk.close()
    return st


def test_noalloc_equals_step_two_calls_second_smaller():
    big = W.Workload("noalloc_flat_f16", 71, [(40_000, True), (3, False), (9_000, True),
                                              (2048 * 10 + 5, False)], W.Hyper(), steps=3,
                     injections={1: [(12_345, "+inf")]})
    log(f"case noalloc flat f16: {big.numel} elements")
    st = _run_pair(big, 3, flat=True, misalign=(0, 0, 0, 0, 0), oracle_check=True)
    assert (st.step, st.skipped_total) == (2, 1)

    small = W.Workload("noalloc_sep_bf16", 72, [(5_000, True), (777, False), (2_051, True)],
                       W.Hyper(dtype=W.BF16, scaler_mode=W.STATIC, init_scale=1.0), steps=2)
    assert small.numel < big.numel
    log(f"case noalloc separate bf16: {small.numel} elements")
    st = _run_pair(small, 2, flat=False, misalign=(1, 2, 1, 3, 1), oracle_check=False)
    assert (st.step, st.skipped_total) == (2, 0)



def _fake_flat(sizes, decays):
    """Segments of a flat layout at fake addresses: the plan only compares them."""
    base, off, fake = 1 << 36, 0, []
    for n, d in zip(sizes, decays):
        fake.append(Z.neox_segment(base + 2 * off, base + (1 << 34) + 2 * off,
                                   base + 2 * (1 << 34) + 4 * off, base + 3 * (1 << 34) + 4 * off,
                                   base + 4 * (1 << 34) + 4 * off, n,
                                   Z.NEOX_SEG_DECAY if d else 0, 0, 0))
        off += n
    return fake


def _fake_separate(sizes, decays):
    """Segments in separate fake allocations (16-byte aligned): the plan only compares them."""
    fake = []
    for i, (n, d) in enumerate(zip(sizes, decays)):
        base = (1 << 40) + i * (1 << 38)
        fake.append(Z.neox_segment(base, base + (1 << 34), base + 2 * (1 << 34),
                                   base + 3 * (1 << 34), base + 4 * (1 << 34), n,
                                   Z.NEOX_SEG_DECAY if d else 0, i, 0))
    return fake


def test_noalloc_equals_step_on_large_norm_blocks_a_separate_finalize_and_sgd():
    """A 9M-element flat shard of 133 segments, whose norm pass runs as at most 256 large
    blocks across the segments and whose update takes the decisions itself; the same
    segments in separate allocations, which keep the norm pass's short chunks (over 256)
    and the separate finalize launch; both checked against the oracle too.  Then a smaller
    momentum-SGD shard in separate allocations."""
    sizes = [6_000_000, 7, 3_000_001] + [41] * 130
    decays = [k % 2 == 0 for k in range(len(sizes))]
    for name, wid, flat, decides in (("noalloc_flat_9m_large_blocks", 73, True, 1),
                                     ("noalloc_separate_9m_finalize", 75, False, 0)):
        big = W.Workload(name, wid, list(zip(sizes, decays)), W.Hyper(), steps=2)
        fake = _fake_flat(sizes, decays) if flat else _fake_separate(sizes, decays)
        plan, _, _, _ = Z.neox_zero1_plan(lib_config(big), fake, tables=False)
        assert plan.update_decides == decides, (name, plan.norm_chunks)
        assert plan.update_path == (Z.NEOX_PATH_FLAT if flat else Z.NEOX_PATH_CHUNKED)
        log(f"case {name}: {big.numel} elements, {plan.norm_chunks} norm chunks of "
            f"{plan.norm_block_threads} threads")
        st = _run_pair(big, 2, flat=flat, misalign=(0, 0, 0, 0, 0), oracle_check=True)
        assert (st.step, st.skipped_total) == (2, 0)

    sgd = W.Workload("noalloc_sep_sgd", 74, [(30_000, True), (1_001, False)],
                     W.Hyper(optimizer=1), steps=3, injections={1: [(7, "nan")]})
    log(f"case noalloc separate sgd: {sgd.numel} elements")
    st = _run_pair(sgd, 3, flat=False, misalign=(1, 0, 1, 2, 0), oracle_check=True)
    assert (st.step, st.skipped_total) == (2, 1)
