"""ctypes front end of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the benchmark's
CPU-baseline leg; the library never imports it.  Arrays are numpy arrays on the host;
half-precision values travel as their uint16 bit patterns.
"""
import ctypes as C
import dataclasses
import os

import numpy as np

from . import build as _build

F16, BF16 = 1, 2
DYNAMIC, STATIC = 0, 1
DECAY = 1
ADAMW, SGD = 0, 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        so = _build.build_oracle(force=False)
        _lib = C.CDLL(so)
        _declare(_lib)
    return _lib


class _Config(C.Structure):
    _fields_ = [("beta1", C.c_double), ("beta2", C.c_double), ("eps", C.c_double),
                ("weight_decay", C.c_double), ("clip_norm", C.c_double),
                ("predivide_factor", C.c_double), ("dp_world_size", C.c_int32),
                ("dtype", C.c_int32), ("scaler_mode", C.c_int32),
                ("growth_interval", C.c_int32), ("growth_factor", C.c_double),
                ("backoff_factor", C.c_double), ("min_scale", C.c_double),
                ("optimizer", C.c_int32), ("pad_", C.c_int32)]


class _Scaler(C.Structure):
    _fields_ = [("loss_scale", C.c_float), ("last_skipped", C.c_int32),
                ("good_steps", C.c_int64), ("step", C.c_int64),
                ("skipped_total", C.c_int64), ("consecutive_overflows", C.c_int64),
                ("last_sumsq", C.c_double), ("last_norm", C.c_double),
                ("last_coef", C.c_double)]


class _Decision(C.Structure):
    _fields_ = [("skip", C.c_int32), ("inv", C.c_double), ("inv32", C.c_float),
                ("coef", C.c_double), ("bc1", C.c_double), ("bc2", C.c_double),
                ("t", C.c_int64)]


class _Segment(C.Structure):
    _fields_ = [("grad", C.c_void_p), ("half", C.c_void_p), ("master", C.c_void_p),
                ("exp_avg", C.c_void_p), ("exp_avg_sq", C.c_void_p),
                ("numel", C.c_int64), ("flags", C.c_int32), ("pad_", C.c_int32)]


class _ShardSegment(C.Structure):
    _fields_ = [("shard_offset", C.c_uint64), ("numel", C.c_uint64),
                ("tensor_offset", C.c_uint64), ("tensor_id", C.c_uint32),
                ("flags", C.c_uint32)]


def _declare(L):
    P = C.POINTER
    L.orc_half_to_double.argtypes = [C.c_int32, C.c_uint16]
    L.orc_half_to_double.restype = C.c_double
    L.orc_float_to_half.argtypes = [C.c_int32, C.c_float]
    L.orc_float_to_half.restype = C.c_uint16
    L.orc_float_to_half_array.argtypes = [C.c_int32, C.c_void_p, C.c_void_p, C.c_int64]
    L.orc_half_to_double_array.argtypes = [C.c_int32, C.c_void_p, C.c_void_p, C.c_int64]
    L.orc_scan.argtypes = [C.c_int32, C.c_void_p, C.c_int64, C.c_double, C.c_float,
                           P(C.c_double), P(C.c_int32)]
    L.orc_unscale_factor.argtypes = [P(_Config), P(_Scaler), P(C.c_double), P(C.c_float)]
    L.orc_decide.argtypes = [P(_Config), P(_Scaler), C.c_int32, C.c_double, P(_Decision)]
    L.orc_update.argtypes = [P(_Config), P(_Decision), C.c_float] + [C.c_void_p] * 5 + \
        [C.c_int64, C.c_int32] + [C.c_void_p] * 3
    L.orc_update_sgd.argtypes = [P(_Config), P(_Decision), C.c_float] + [C.c_void_p] * 4 + \
        [C.c_int64, C.c_int32] + [C.c_void_p] * 2
    L.orc_step.argtypes = [P(_Config), P(_Scaler), C.c_float, P(_Segment), C.c_int64]
    L.orc_partition.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_int64,
                                C.c_int64, P(_ShardSegment), C.c_int64, P(C.c_uint64)]
    L.orc_partition.restype = C.c_int64


@dataclasses.dataclass
class Config:
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.01
    clip_norm: float = 1.0
    predivide_factor: float = 1.0
    dp_world_size: int = 1
    dtype: int = F16
    scaler_mode: int = DYNAMIC
    growth_interval: int = 1000
    growth_factor: float = 2.0
    backoff_factor: float = 0.5
    min_scale: float = 1.0
    optimizer: int = ADAMW

    def c(self):
        return _Config(**dataclasses.asdict(self), pad_=0)


@dataclasses.dataclass
class Scaler:
    loss_scale: float = 65536.0
    last_skipped: int = 0
    good_steps: int = 0
    step: int = 0
    skipped_total: int = 0
    consecutive_overflows: int = 0
    last_sumsq: float = 0.0
    last_norm: float = 0.0
    last_coef: float = 1.0

    def c(self):
        return _Scaler(**dataclasses.asdict(self))

    def load(self, cs):
        for f in dataclasses.fields(self):
            setattr(self, f.name, getattr(cs, f.name))
        return self


@dataclasses.dataclass
class Decision:
    skip: int
    inv: float
    inv32: float
    coef: float
    bc1: float
    bc2: float
    t: int


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p)


def _check(a, dtype, n=None):
    assert isinstance(a, np.ndarray) and a.dtype == dtype and a.flags.c_contiguous, (a.dtype, dtype)
    if n is not None:
        assert a.size == n, (a.size, n)


def half_to_double(dtype, bits):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib().orc_half_to_double_array(dtype, _ptr(bits), _ptr(out), bits.size)
    return out


def float_to_half(dtype, x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_float_to_half_array(dtype, _ptr(x), _ptr(out), x.size)
    return out


def unscale_factor(cfg: Config, st: Scaler):
    inv, inv32 = C.c_double(), C.c_float()
    lib().orc_unscale_factor(C.byref(cfg.c()), C.byref(st.c()), C.byref(inv), C.byref(inv32))
    return inv.value, inv32.value


def scan(dtype, grad, inv, inv32, sumsq=0.0, overflow=0):
    _check(grad, np.uint16)
    s, o = C.c_double(sumsq), C.c_int32(overflow)
    lib().orc_scan(dtype, _ptr(grad), grad.size, inv, inv32, C.byref(s), C.byref(o))
    return s.value, o.value


def decide(cfg: Config, st: Scaler, overflow, sumsq) -> Decision:
    cs = st.c()
    d = _Decision()
    lib().orc_decide(C.byref(cfg.c()), C.byref(cs), int(overflow), float(sumsq), C.byref(d))
    st.load(cs)
    return Decision(d.skip, d.inv, d.inv32, d.coef, d.bc1, d.bc2, d.t)


def update(cfg: Config, d: Decision, lr, grad, half, master, m, v, decay, scales=False):
    """In-place AdamW on host arrays; returns (s_m, s_v, s_w) when scales=True."""
    n = grad.size
    _check(grad, np.uint16, n)
    _check(half, np.uint16, n)
    for a in (master, m, v):
        _check(a, np.float32, n)
    cd = _Decision(d.skip, d.inv, d.inv32, d.coef, d.bc1, d.bc2, d.t)
    sm = sv = sw = None
    if scales:
        sm, sv, sw = (np.zeros(n, np.float64) for _ in range(3))
    nul = C.c_void_p(0)
    lib().orc_update(C.byref(cfg.c()), C.byref(cd), lr, _ptr(grad), _ptr(half), _ptr(master),
                     _ptr(m), _ptr(v), n, int(bool(decay)),
                     _ptr(sm) if scales else nul, _ptr(sv) if scales else nul,
                     _ptr(sw) if scales else nul)
    return (sm, sv, sw) if scales else None


def update_sgd(cfg: Config, d: Decision, lr, grad, half, master, m, decay, scales=False):
    """In-place momentum SGD on host arrays; returns (s_m, s_w) when scales=True."""
    n = grad.size
    _check(grad, np.uint16, n)
    _check(half, np.uint16, n)
    for a in (master, m):
        _check(a, np.float32, n)
    cd = _Decision(d.skip, d.inv, d.inv32, d.coef, d.bc1, d.bc2, d.t)
    sm = sw = None
    if scales:
        sm, sw = (np.zeros(n, np.float64) for _ in range(2))
    nul = C.c_void_p(0)
    lib().orc_update_sgd(C.byref(cfg.c()), C.byref(cd), lr, _ptr(grad), _ptr(half), _ptr(master),
                         _ptr(m), n, int(bool(decay)), _ptr(sm) if scales else nul,
                         _ptr(sw) if scales else nul)
    return (sm, sw) if scales else None


def step(cfg: Config, st: Scaler, lr, segments):
    """One whole step; segments = list of dicts with keys grad, half, master, m, v, decay."""
    arr = (_Segment * max(1, len(segments)))()
    for i, s in enumerate(segments):
        n = s["grad"].size
        _check(s["grad"], np.uint16, n)
        _check(s["half"], np.uint16, n)
        for k in ("master", "m") + (() if cfg.optimizer == SGD else ("v",)):
            _check(s[k], np.float32, n)
        v = _ptr(s["v"]).value if s.get("v") is not None else None
        arr[i] = _Segment(_ptr(s["grad"]).value, _ptr(s["half"]).value, _ptr(s["master"]).value,
                          _ptr(s["m"]).value, v, n, DECAY if s.get("decay", False) else 0, 0)
    cs = st.c()
    lib().orc_step(C.byref(cfg.c()), C.byref(cs), lr, arr, len(segments))
    st.load(cs)
    return st


def pieces(sizes, parts):
    """Cut the concatenation of segments of the given sizes into `parts` contiguous pieces
    of nearly equal length: per piece, the list of (segment, lo, hi) runs it covers."""
    total = int(sum(sizes))
    bounds = [total * p // parts for p in range(parts + 1)]
    out, starts, off = [], [], 0
    for n in sizes:
        starts.append(off)
        off += int(n)
    for p in range(parts):
        a, b, runs = bounds[p], bounds[p + 1], []
        for k, n in enumerate(sizes):
            lo, hi = max(a, starts[k]), min(b, starts[k] + int(n))
            if lo < hi:
                runs.append((k, lo - starts[k], hi - starts[k]))
        out.append(runs)
    return out


def step_parallel(cfg: Config, st: Scaler, lr, segments, threads):
    """One whole step with the elementwise work on `threads` host threads: the segments'
    elements, concatenated, are cut into `threads` contiguous pieces; each thread scans
    its piece into its own double partial sum (orc_scan), the partials are added in
    thread order, one orc_decide takes the step's decisions, and each thread updates its
    piece (orc_update / orc_update_sgd).  ctypes releases the interpreter lock during each
    call, so the threads run in parallel.  Equals step() except for the summation order
    of the squared norm (its last bits).  segments as for step()."""
    from concurrent.futures import ThreadPoolExecutor

    sizes = [s["grad"].size for s in segments]
    work = pieces(sizes, max(1, int(threads)))
    inv, inv32 = unscale_factor(cfg, st)

    def scan_piece(runs):
        acc, of = 0.0, 0
        for k, lo, hi in runs:
            acc, of = scan(cfg.dtype, segments[k]["grad"][lo:hi], inv, inv32, acc, of)
        return acc, of

    def update_piece(d, runs):
        for k, lo, hi in runs:
            s = segments[k]
            sl = slice(lo, hi)
            if cfg.optimizer == SGD:
                update_sgd(cfg, d, lr, s["grad"][sl], s["half"][sl], s["master"][sl],
                           s["m"][sl], s.get("decay", False))
            else:
                update(cfg, d, lr, s["grad"][sl], s["half"][sl], s["master"][sl], s["m"][sl],
                       s["v"][sl], s.get("decay", False))

    with ThreadPoolExecutor(max_workers=len(work)) as ex:
        parts = list(ex.map(scan_piece, work))
        sumsq, of = 0.0, 0
        for acc, o in parts:                  # thread order
            sumsq += acc
            of |= o
        d = decide(cfg, st, of, sumsq)
        list(ex.map(lambda runs: update_piece(d, runs), work))
    return st


def partition(tensor_numel, tensor_decay, dp_world_size, rank, align=64):
    """Segments of `rank` as a list of dicts, plus the shard length P."""
    numel = np.ascontiguousarray(tensor_numel, dtype=np.uint64)
    decay = np.ascontiguousarray(tensor_decay, dtype=np.uint8)
    assert numel.size == decay.size and dp_world_size >= 1 and align >= 1
    assert 0 <= rank < dp_world_size
    P = C.c_uint64()
    n = lib().orc_partition(_ptr(numel), _ptr(decay), numel.size, dp_world_size, rank, align,
                            None, 0, C.byref(P))
    out = (_ShardSegment * max(1, n))()
    lib().orc_partition(_ptr(numel), _ptr(decay), numel.size, dp_world_size, rank, align,
                        out, n, C.byref(P))
    segs = [dict(shard_offset=s.shard_offset, numel=s.numel, tensor_offset=s.tensor_offset,
                 tensor_id=s.tensor_id, flags=s.flags) for s in out[:n]]
    return segs, P.value
