"""C-ABI checks that need no GPU: the library loads, exports every declared symbol,
its shard partition matches the oracle's element-by-element one bit for bit, and
argument validation rejects bad input before touching the device."""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest

import mixed_precision_zero_amd as Z
import workloads as W
from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "neox_zero1.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(neox_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert len(syms) >= 9
    L = C.CDLL(Z.LIB_PATH)
    for s in syms:
        assert hasattr(L, s), s
    assert sorted(Z.EXPORTS) == syms


def test_probe_library_exports_every_declared_symbol():
    from mixed_precision_zero_amd import probe as P
    text = open(os.path.join(ROOT, "include", "neox_stream_probe.h")).read()
    syms = sorted(set(re.findall(r"^(?:int|const char\*)\s+(neox_\w+)\s*\(", text, re.M)))
    assert sorted(P.EXPORTS) == syms
    L = C.CDLL(P.LIB_PATH)
    for s in syms:
        assert hasattr(L, s), s


def test_probe_rejects_bad_arguments():
    from mixed_precision_zero_amd import probe as P
    with pytest.raises(RuntimeError):
        P.neox_probe_copy(0, 0, 16)
    with pytest.raises(RuntimeError):
        P.neox_probe_update_pattern(16, 16, 16, 16, 16, 7)
    for shape in ((100, 2, 0), (256, 3, 0), (256, 2, -1), (256, 2, 17)):
        with pytest.raises(RuntimeError):
            P.neox_probe_update_pattern(16, 16, 16, 16, 16, 8, *shape)


def test_default_config():
    cfg = Z.neox_zero1_default_config()
    assert (cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.clip_norm) == (0.9, 0.95, 1e-8, 0.01, 1.0)
    assert (cfg.init_scale, cfg.growth_factor, cfg.backoff_factor, cfg.min_scale) == (65536.0, 2.0, 0.5, 1.0)
    assert cfg.growth_interval == 1000 and cfg.dtype == Z.NEOX_F16


def _lib_partition(numel, decay, D, r, align):
    segs, P = Z.neox_zero1_partition(numel, decay, D, r, align)
    out = []
    for s in segs:
        tid = len(numel) if s.tensor_id == Z.NEOX_PAD_TENSOR else s.tensor_id
        out.append((s.shard_offset, s.numel, s.tensor_offset, tid, s.flags))
    return out, P


def _orc_partition(numel, decay, D, r, align):
    segs, P = O.partition(numel, decay, D, r, align)
    return [(s["shard_offset"], s["numel"], s["tensor_offset"], s["tensor_id"], s["flags"])
            for s in segs], P


def test_partition_matches_oracle_random():
    rng = np.random.default_rng(40)
    for _ in range(200):
        k = int(rng.integers(1, 15))
        numel = [int(x) for x in rng.integers(0, 70, k)]
        if sum(numel) == 0:
            numel[-1] = 3
        decay = [int(x) for x in rng.integers(0, 2, k)]
        D, A = int(rng.integers(1, 10)), int(rng.integers(1, 17))
        for r in range(D):
            assert _lib_partition(numel, decay, D, r, A) == _orc_partition(numel, decay, D, r, A)


def test_partition_matches_oracle_pythia410m_all_ranks():
    t = W.pythia410m_tensors()
    numel = [n for n, _ in t]
    decay = [int(d) for _, d in t]
    for r in (0, 1, 5, 7):
        assert _lib_partition(numel, decay, 8, r, 64) == _orc_partition(numel, decay, 8, r, 64)


def test_partition_large_counts_64bit():
    """Totals beyond 2^32 (the 6e9-param OPT-style shard is one rank of such a concat)."""
    numel = [3_000_000_000, 5_000_000_000, 7]
    segs, P = _lib_partition(numel, [1, 0, 1], 2, 1, 64)
    total = sum(numel)
    assert P == math.ceil(total / 128) * 128 // 2
    assert segs[0] == (0, 3_000_000_000 + 5_000_000_000 - P, P - 3_000_000_000, 1, 0)
    assert sum(s[1] for s in segs) == P


def test_partition_errors():
    with pytest.raises(Z.NeoxError):
        Z.neox_zero1_partition([1, 2], [0, 0], 0, 0, 64)
    with pytest.raises(Z.NeoxError):
        Z.neox_zero1_partition([1, 2], [0, 0], 2, 2, 64)
    with pytest.raises(Z.NeoxError):
        Z.neox_zero1_partition([1, 2], [0, 0], 2, 0, 0)
    with pytest.raises(Z.NeoxError):
        Z.neox_zero1_partition([2 ** 63, 2 ** 63], [0, 0], 1, 0, 1)


def _fake_seg(n=16, base=0x10000, flags=0):
    return Z.neox_segment(base, base + 0x1000, base + 0x2000, base + 0x3000, base + 0x4000,
                          n, flags, 0, 0)


@pytest.mark.parametrize("field,value", [
    ("beta1", 1.0), ("beta1", -0.1), ("beta2", 1.5), ("eps", -1.0), ("eps", float("nan")),
    ("eps", 0.0), ("eps", 1e-50), ("weight_decay", -0.01), ("clip_norm", float("inf")), ("predivide_factor", 0.0),
    ("dp_world_size", 0), ("dtype", 3), ("scaler_mode", 2), ("growth_interval", 0),
    ("init_scale", 0.0), ("init_scale", 1e39), ("growth_factor", 0.5), ("backoff_factor", 0.0),
    ("backoff_factor", 1.5), ("min_scale", 0.0), ("init_step", -1), ("chunk_elems", 100),
    ("chunk_elems", 257), ("chunk_elems", 1 << 25), ("optimizer", 2), ("segment_norms", 2), ("chunked_update", 2)])
def test_create_rejects_bad_config(field, value):
    cfg = Z.neox_zero1_default_config()
    setattr(cfg, field, value)
    with pytest.raises(Z.NeoxError) as e:
        Z.neox_zero1_create(cfg, [_fake_seg()])
    assert e.value.code == Z.NEOX_EINVAL


@pytest.mark.parametrize("seg", [
    Z.neox_segment(0, 0x2000, 0x3000, 0x4000, 0x5000, 16, 0, 0, 0),        # null grad
    Z.neox_segment(0x1001, 0x2000, 0x3000, 0x4000, 0x5000, 16, 0, 0, 0),   # odd grad
    Z.neox_segment(0x1000, 0x2000, 0x3002, 0x4000, 0x5000, 16, 0, 0, 0),   # fp32 misaligned
    Z.neox_segment(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0, 0, 0, 0),    # empty
    Z.neox_segment(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 16, 4, 0, 0),   # unknown flag
    Z.neox_segment(0x1000, 0x2000, 0x3000, 0x3020, 0x5000, 16, 0, 0, 0),   # m overlaps master
], ids=["null", "odd_grad", "f32_misaligned", "empty", "bad_flag", "overlap"])
def test_create_rejects_bad_segments(seg):
    with pytest.raises(Z.NeoxError) as e:
        Z.neox_zero1_create(Z.neox_zero1_default_config(), [seg])
    assert e.value.code == Z.NEOX_EINVAL


def test_create_rejects_segment_norms_with_striding_norm_grid():
    cfg = Z.neox_zero1_default_config(segment_norms=1, norm_blocks=4)
    with pytest.raises(Z.NeoxError) as e:
        Z.neox_zero1_create(cfg, [_fake_seg()])
    assert e.value.code == Z.NEOX_EINVAL


def test_create_exp_avg_sq_required_for_adamw_only():
    seg = Z.neox_segment(0x1000, 0x2000, 0x3000, 0x4000, 0, 16, 0, 0, 0)
    with pytest.raises(Z.NeoxError) as e:
        Z.neox_zero1_create(Z.neox_zero1_default_config(), [seg])
    assert "null array" in str(e.value)
    # with SGD the missing second moment passes validation (creation then needs a GPU)
    try:
        Z.neox_zero1_create(Z.neox_zero1_default_config(optimizer=Z.NEOX_OPT_SGD), [seg])
    except Z.NeoxError as e2:
        assert e2.code != Z.NEOX_EINVAL or "null array" not in str(e2)


def test_create_rejects_empty_and_null():
    L = Z.lib()
    h = C.c_void_p()
    cfg = Z.neox_zero1_default_config()
    assert L.neox_zero1_create(C.byref(cfg), None, 1, None, C.byref(h)) == Z.NEOX_EINVAL
    assert L.neox_zero1_create(None, None, 0, None, C.byref(h)) == Z.NEOX_EINVAL
    assert L.neox_zero1_create(C.byref(cfg), None, 0, None, None) == Z.NEOX_EINVAL
    with pytest.raises(Z.NeoxError):
        Z.neox_zero1_create(cfg, [])
    # overlapping segments across the list
    with pytest.raises(Z.NeoxError):
        Z.neox_zero1_create(cfg, [_fake_seg(16, 0x10000), _fake_seg(16, 0x10020)])


def test_null_handle_calls():
    L = Z.lib()
    assert L.neox_zero1_step(None, C.c_float(1e-3), None) == Z.NEOX_EINVAL
    st = Z.neox_scaler_state_t()
    assert L.neox_scaler_state(None, C.byref(st)) == Z.NEOX_EINVAL
    assert L.neox_zero1_destroy(None) == Z.NEOX_OK
    assert "null" in Z.neox_zero1_last_error().lower()
    assert L.neox_zero1_timing_begin(None, 4, 0) == Z.NEOX_EINVAL
    assert L.neox_zero1_step_local(None, None, None) == Z.NEOX_EINVAL
    assert L.neox_zero1_step_apply(None, None, 1, C.c_float(1e-3), None) == Z.NEOX_EINVAL
    assert L.neox_scaler_set(None, None, None) == Z.NEOX_EINVAL
    assert L.neox_zero1_segment_sumsq(None, None, 0) == Z.NEOX_EINVAL
    assert L.neox_zero1_update_path(None) == Z.NEOX_EINVAL


def test_plan_rejects_gradients_aliasing_written_arrays():
    """A gradient that overlaps a written array (its own half copy, or another segment's
    master) would be read while other blocks overwrite it: rejected at validation."""
    a = _fake_seg(16, 0x10000)
    b = _fake_seg(16, 0x80000)
    cfg = Z.neox_zero1_default_config()
    Z.neox_zero1_plan(cfg, [a, b], tables=False)       # disjoint: accepted
    own_half = Z.neox_segment(a.half, a.half, a.master, a.exp_avg, a.exp_avg_sq, 16, 0, 0, 0)
    into_master = Z.neox_segment(b.master + 8, b.half, b.master, b.exp_avg, b.exp_avg_sq,
                                 16, 0, 0, 0)
    for segs in ([own_half], [a, Z.neox_segment(a.master + 8, b.half, b.master, b.exp_avg,
                                                b.exp_avg_sq, 16, 0, 0, 0)], [into_master]):
        with pytest.raises(Z.NeoxError) as e:
            Z.neox_zero1_plan(cfg, segs, tables=False)
        assert e.value.code == Z.NEOX_EINVAL and "grad overlaps" in str(e.value)
    # two segments may read the same gradient (nothing writes it)
    shared = Z.neox_segment(a.grad, b.half, b.master, b.exp_avg, b.exp_avg_sq, 16, 0, 0, 0)
    Z.neox_zero1_plan(cfg, [a, shared], tables=False)


def test_noalloc_validates_before_any_device_work():
    """neox_zero1_step_noalloc refuses bad arguments, and a shard whose work tables do not
    fit its fixed scratch, before it touches a device (so this runs without a GPU)."""
    L = Z.lib()
    cfg = Z.neox_zero1_default_config()
    st = Z.neox_scaler_state_t()
    st.loss_scale = 65536.0
    seg = (Z.neox_segment * 1)(_fake_seg())
    assert L.neox_zero1_step_noalloc(None, seg, 1, C.byref(st), C.c_float(1e-3), None) == Z.NEOX_EINVAL
    assert L.neox_zero1_step_noalloc(C.byref(cfg), seg, 1, None, C.c_float(1e-3), None) == Z.NEOX_EINVAL
    assert L.neox_zero1_step_noalloc(C.byref(cfg), seg, 1, C.byref(st), C.c_float(float("nan")),
                                     None) == Z.NEOX_EINVAL
    bad = Z.neox_scaler_state_t()
    bad.loss_scale = 0.0
    assert L.neox_zero1_step_noalloc(C.byref(cfg), seg, 1, C.byref(bad), C.c_float(1e-3), None) == Z.NEOX_EINVAL
    tel = Z.neox_zero1_default_config(segment_norms=1)
    assert L.neox_zero1_step_noalloc(C.byref(tel), seg, 1, C.byref(st), C.c_float(1e-3), None) == Z.NEOX_EINVAL
    # 600M elements in separate allocations need ~19 MB of chunk table: beyond 16 MiB
    n = 600_000_000
    big = Z.neox_segment(1 << 40, 1 << 41, 1 << 42, (1 << 42) + (1 << 40), 1 << 43, n,
                         Z.NEOX_SEG_DECAY, 0, 0)
    with pytest.raises(Z.NeoxError) as e:
        Z.neox_zero1_step_noalloc(Z.neox_zero1_default_config(chunked_update=1), [big], st, 1e-3)
    assert e.value.code == Z.NEOX_EINVAL and "scratch" in str(e.value)
    # a flat partition needs ~2 bytes per 1,000 elements (its tile table): 9e9 is beyond
    n = 9_000_000_000
    flat = Z.neox_segment(1 << 44, 1 << 45, 1 << 46, (1 << 46) + (1 << 45), 1 << 47, n,
                          Z.NEOX_SEG_DECAY, 0, 0)
    plan = Z.neox_zero1_plan(Z.neox_zero1_default_config(), [flat], tables=False)[0]
    assert plan.update_path == Z.NEOX_PATH_FLAT and plan.update_decides == 1
    with pytest.raises(Z.NeoxError) as e:
        Z.neox_zero1_step_noalloc(Z.neox_zero1_default_config(), [flat], st, 1e-3)
    assert e.value.code == Z.NEOX_EINVAL and "scratch" in str(e.value)
    assert Z.NEOX_NOALLOC_SCRATCH_BYTES == 16 * 1024 * 1024
