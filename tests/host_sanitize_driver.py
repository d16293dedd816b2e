"""Exercises the step library's host code (no GPU needed) for tests/test_sanitize_cpu.py:
random shard partitions, random plans with their tables for flat and separately
allocated layouts, create's validation and error paths, and null-handle calls.
Usage: python host_sanitize_driver.py <path of the library build to load>."""
import ctypes as C
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import numpy as np  # noqa: E402

import mixed_precision_zero_amd as Z  # noqa: E402

Z.LIB_PATH = sys.argv[1]
Z._lib = None
import test_plan_cpu as TP  # noqa: E402

L = Z.lib()
rng = np.random.default_rng(5)
for case in range(200):
    nt = int(rng.integers(0, 40))
    numel = [int(x) for x in rng.integers(1, 100_000, nt)]
    decay = [bool(x) for x in rng.integers(0, 2, nt)]
    D = int(rng.integers(1, 9))
    A = int(rng.choice([1, 8, 64]))
    for r in range(D):
        Z.neox_zero1_partition(numel, decay, D, r, A)
for case in range(300):
    nseg = int(rng.integers(1, 40))
    sizes = [int(x) for x in rng.choice([1, 2, 7, 8, 9, 255, 256, 2047, 2048, 2049, 40_000, 70_001], nseg)]
    decays = [bool(x) for x in rng.integers(0, 2, nseg)]
    segs = TP.separate_segments(rng, sizes, decays) if case % 2 else TP.flat_segments(sizes, decays)
    cfg = Z.neox_zero1_default_config(chunk_elems=int(rng.choice([0, 256, 1000, 4096])),
                                      optimizer=int(rng.integers(0, 2)),
                                      segment_norms=int(rng.integers(0, 2)))
    try:
        Z.neox_zero1_plan(cfg, segs)
    except Z.NeoxError:
        pass
segs = TP.flat_segments([5000, 3], [True, False])
for bad in (dict(beta1=1.0), dict(eps=-1.0), dict(chunk_elems=100), dict(dtype=7), dict(init_scale=0.0)):
    try:
        Z.neox_zero1_create(Z.neox_zero1_default_config(**bad), segs)
        raise SystemExit(f"create accepted {bad}")
    except Z.NeoxError:
        pass
try:
    Z.neox_zero1_create(Z.neox_zero1_default_config(), segs)   # fails at the first HIP call
except Z.NeoxError:
    pass
# gradients aliasing written arrays, and the allocation-free step's validation
a = TP.flat_segments([64], [True])[0]
for alias in (Z.neox_segment(a.half, a.half, a.master, a.exp_avg, a.exp_avg_sq, 64, 0, 0, 0),
              Z.neox_segment(a.master + 4, a.half, a.master, a.exp_avg, a.exp_avg_sq, 64, 0, 0, 0)):
    try:
        Z.neox_zero1_plan(Z.neox_zero1_default_config(), [alias])
        raise SystemExit("plan accepted an aliased gradient")
    except Z.NeoxError:
        pass
st = Z.neox_scaler_state_t()
st.loss_scale = 65536.0
for cfg, sg in ((Z.neox_zero1_default_config(chunked_update=1),
                 [Z.neox_segment(1 << 40, 1 << 41, 1 << 42, (1 << 42) + (1 << 40), 1 << 43,
                                 600_000_000, 1, 0, 0)]),       # beyond the scratch
                (Z.neox_zero1_default_config(), segs)):          # fails at the first HIP call
    try:
        Z.neox_zero1_step_noalloc(cfg, sg, st, 1e-3)
    except Z.NeoxError:
        pass
L.neox_zero1_step(None, C.c_float(1e-3), None)
L.neox_zero1_update_path(None)
L.neox_zero1_timing_begin(None, 10, 0)
L.neox_zero1_destroy(None)
print("host code exercised", flush=True)
