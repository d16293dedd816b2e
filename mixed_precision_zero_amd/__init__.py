"""Python binding of libneox_zero1.so: the ZeRO-1 mixed-precision Adam step on one
data-parallel shard, hand-written HIP for gfx950 (MI355X).

Argument marshalling only: every step of the path runs in the library's kernels.
PyTorch supplies device memory and streams.  The functions keep the C names
(neox_zero1_create, neox_zero1_step, neox_scaler_state, neox_zero1_destroy,
neox_zero1_partition, ...); `Zero1` is a small owner of one handle.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libneox_zero1.so")

NEOX_OK, NEOX_EINVAL, NEOX_EHIP, NEOX_ENOMEM = 0, -1, -2, -3
NEOX_F16, NEOX_BF16 = 1, 2
NEOX_SCALER_DYNAMIC, NEOX_SCALER_STATIC = 0, 1
NEOX_OPT_ADAMW, NEOX_OPT_SGD = 0, 1
NEOX_PATH_CHUNKED, NEOX_PATH_FLAT = 0, 1
NEOX_CHUNK_DECAY, NEOX_CHUNK_VEC = 1, 2
NEOX_SEG_DECAY = 1
NEOX_PAD_TENSOR = 0xFFFFFFFF


class NeoxError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"neox_zero1 error {code}: {msg}")
        self.code = code


class neox_zero1_config(C.Structure):
    _fields_ = [("beta1", C.c_double), ("beta2", C.c_double), ("eps", C.c_double),
                ("weight_decay", C.c_double), ("clip_norm", C.c_double),
                ("predivide_factor", C.c_double), ("dp_world_size", C.c_int32),
                ("dtype", C.c_int32), ("scaler_mode", C.c_int32),
                ("growth_interval", C.c_int32), ("init_scale", C.c_double),
                ("growth_factor", C.c_double), ("backoff_factor", C.c_double),
                ("min_scale", C.c_double), ("init_step", C.c_int64),
                ("init_skipped", C.c_int64), ("init_good_steps", C.c_int32),
                ("init_consecutive_overflows", C.c_int32), ("chunk_elems", C.c_uint32),
                ("norm_blocks", C.c_uint32), ("optimizer", C.c_int32),
                ("segment_norms", C.c_uint32), ("chunked_update", C.c_uint32)]


class neox_segment(C.Structure):
    _fields_ = [("grad", C.c_void_p), ("half", C.c_void_p), ("master", C.c_void_p),
                ("exp_avg", C.c_void_p), ("exp_avg_sq", C.c_void_p), ("numel", C.c_uint64),
                ("flags", C.c_uint32), ("tensor_id", C.c_uint32), ("tensor_offset", C.c_uint64)]


class neox_scaler_state_t(C.Structure):
    _fields_ = [("loss_scale", C.c_float), ("good_steps", C.c_int32), ("step", C.c_int64),
                ("skipped_total", C.c_int64), ("consecutive_overflows", C.c_int32),
                ("last_skipped", C.c_int32), ("last_grad_norm", C.c_float),
                ("last_clip_coef", C.c_float), ("last_sumsq", C.c_double),
                ("device_loss_scale", C.c_void_p)]


class neox_chunk_info(C.Structure):
    _fields_ = [("offset", C.c_uint64), ("seg", C.c_uint32), ("len", C.c_uint32),
                ("flags", C.c_uint32), ("reserved", C.c_uint32)]


class neox_zero1_plan_t(C.Structure):
    _fields_ = [("numel", C.c_uint64), ("update_chunks", C.c_uint64), ("norm_chunks", C.c_uint64),
                ("flat_tiles", C.c_uint64), ("flat_changes", C.c_uint64),
                ("chunk_elems", C.c_uint32), ("norm_chunk_elems", C.c_uint32),
                ("tile_elems", C.c_uint32), ("update_path", C.c_int32),
                ("norm_block_threads", C.c_uint32), ("update_decides", C.c_uint32)]


class neox_shard_segment(C.Structure):
    _fields_ = [("shard_offset", C.c_uint64), ("numel", C.c_uint64),
                ("tensor_offset", C.c_uint64), ("tensor_id", C.c_uint32), ("flags", C.c_uint32)]


# Every symbol include/neox_zero1.h declares.
EXPORTS = ("neox_zero1_default_config", "neox_zero1_partition", "neox_zero1_create",
           "neox_zero1_step", "neox_scaler_state", "neox_zero1_destroy",
           "neox_zero1_step_local", "neox_zero1_step_apply", "neox_scaler_set",
           "neox_zero1_segment_sumsq",
           "neox_zero1_timing_begin", "neox_zero1_timing_end", "neox_zero1_update_path",
           "neox_zero1_plan", "neox_zero1_step_noalloc", "neox_zero1_last_error")
NEOX_NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024

_lib = None


def lib():
    """The loaded library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m mixed_precision_zero_amd.build`")
        L = C.CDLL(LIB_PATH)
        P = C.POINTER
        L.neox_zero1_default_config.argtypes = [P(neox_zero1_config)]
        L.neox_zero1_partition.argtypes = [C.c_void_p, C.c_void_p, C.c_uint64, C.c_uint32,
                                           C.c_uint32, C.c_uint32, P(neox_shard_segment),
                                           C.c_uint64, P(C.c_uint64), P(C.c_uint64)]
        L.neox_zero1_create.argtypes = [P(neox_zero1_config), P(neox_segment), C.c_uint64,
                                        C.c_void_p, P(C.c_void_p)]
        L.neox_zero1_step.argtypes = [C.c_void_p, C.c_float, C.c_void_p]
        L.neox_scaler_state.argtypes = [C.c_void_p, P(neox_scaler_state_t)]
        L.neox_zero1_destroy.argtypes = [C.c_void_p]
        L.neox_zero1_step_local.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p]
        L.neox_zero1_step_apply.argtypes = [C.c_void_p, C.c_void_p, C.c_uint32, C.c_float,
                                            C.c_void_p]
        L.neox_scaler_set.argtypes = [C.c_void_p, P(neox_scaler_state_t), C.c_void_p]
        L.neox_zero1_segment_sumsq.argtypes = [C.c_void_p, C.c_void_p, C.c_uint64]
        L.neox_zero1_timing_begin.argtypes = [C.c_void_p, C.c_int32, C.c_int32]
        L.neox_zero1_timing_end.argtypes = [C.c_void_p, P(C.c_double), P(C.c_int64),
                                            P(C.c_double), C.c_int64]
        L.neox_zero1_update_path.argtypes = [C.c_void_p]
        L.neox_zero1_plan.argtypes = [P(neox_zero1_config), P(neox_segment), C.c_uint64,
                                      P(neox_zero1_plan_t), P(neox_chunk_info), C.c_uint64,
                                      P(C.c_uint32), C.c_uint64, P(C.c_uint32), C.c_uint64]
        L.neox_zero1_step_noalloc.argtypes = [P(neox_zero1_config), P(neox_segment), C.c_uint64,
                                              P(neox_scaler_state_t), C.c_float, C.c_void_p]
        L.neox_zero1_last_error.argtypes = []
        L.neox_zero1_last_error.restype = C.c_char_p
        for name in EXPORTS:
            if name != "neox_zero1_last_error":
                getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def _check(rc):
    if rc != NEOX_OK:
        raise NeoxError(rc, lib().neox_zero1_last_error().decode())
    return rc


# --------------------------------------------------------------------------------------
# C names
# --------------------------------------------------------------------------------------

def neox_zero1_last_error() -> str:
    return lib().neox_zero1_last_error().decode()


def neox_zero1_default_config(**overrides) -> neox_zero1_config:
    cfg = neox_zero1_config()
    _check(lib().neox_zero1_default_config(C.byref(cfg)))
    for k, v in overrides.items():
        if not hasattr(cfg, k):
            raise AttributeError(k)
        setattr(cfg, k, v)
    return cfg


def neox_zero1_partition(tensor_numel, tensor_decay, dp_world_size, rank, align=64):
    """-> (list of neox_shard_segment, shard length P)."""
    n = len(tensor_numel)
    numel = (C.c_uint64 * max(1, n))(*tensor_numel)
    decay = (C.c_uint8 * max(1, n))(*[1 if d else 0 for d in tensor_decay])
    nseg, P = C.c_uint64(), C.c_uint64()
    _check(lib().neox_zero1_partition(numel, decay, n, dp_world_size, rank, align, None, 0,
                                      C.byref(nseg), C.byref(P)))
    out = (neox_shard_segment * max(1, nseg.value))()
    _check(lib().neox_zero1_partition(numel, decay, n, dp_world_size, rank, align, out,
                                      nseg.value, C.byref(nseg), C.byref(P)))
    return list(out[:nseg.value]), P.value


def neox_zero1_create(cfg: neox_zero1_config, segs, stream_ptr: int = 0) -> int:
    """segs: sequence of neox_segment (device pointers).  Returns the handle (int)."""
    arr = (neox_segment * max(1, len(segs)))(*segs)
    h = C.c_void_p()
    _check(lib().neox_zero1_create(C.byref(cfg), arr, len(segs), C.c_void_p(stream_ptr),
                                   C.byref(h)))
    return h.value


def neox_zero1_step(h: int, lr: float, stream_ptr: int = 0):
    _check(lib().neox_zero1_step(C.c_void_p(h), C.c_float(lr), C.c_void_p(stream_ptr)))


def neox_scaler_state(h: int) -> neox_scaler_state_t:
    st = neox_scaler_state_t()
    _check(lib().neox_scaler_state(C.c_void_p(h), C.byref(st)))
    return st


def neox_zero1_destroy(h: int):
    _check(lib().neox_zero1_destroy(C.c_void_p(h)))


def neox_zero1_step_local(h: int, local_sumsq_ptr: int, stream_ptr: int = 0):
    """Norm pass; this rank's squared norm goes to the device double at local_sumsq_ptr."""
    _check(lib().neox_zero1_step_local(C.c_void_p(h), C.c_void_p(local_sumsq_ptr),
                                       C.c_void_p(stream_ptr)))


def neox_zero1_step_apply(h: int, rank_sumsq_ptr: int, lr: float, stream_ptr: int = 0,
                          nranks: int = 1):
    """Finalize on the fixed-order sum of the nranks device doubles at rank_sumsq_ptr (the
    ranks' squared norms, in rank order), then the update."""
    _check(lib().neox_zero1_step_apply(C.c_void_p(h), C.c_void_p(rank_sumsq_ptr), nranks,
                                       C.c_float(lr), C.c_void_p(stream_ptr)))


def neox_scaler_set(h: int, loss_scale: float, good_steps=0, step=0, skipped_total=0,
                    consecutive_overflows=0, stream_ptr: int = 0):
    st = neox_scaler_state_t()
    st.loss_scale = loss_scale
    st.good_steps = good_steps
    st.step = step
    st.skipped_total = skipped_total
    st.consecutive_overflows = consecutive_overflows
    _check(lib().neox_scaler_set(C.c_void_p(h), C.byref(st), C.c_void_p(stream_ptr)))


def neox_zero1_segment_sumsq(h: int, nseg: int):
    out = (C.c_double * max(1, nseg))()
    _check(lib().neox_zero1_segment_sumsq(C.c_void_p(h), out, nseg))
    return list(out[:nseg])


def neox_zero1_timing_begin(h: int, max_steps: int, update_only: bool = False):
    _check(lib().neox_zero1_timing_begin(C.c_void_p(h), max_steps, int(update_only)))


def neox_zero1_update_path(h: int) -> int:
    """NEOX_PATH_FLAT or NEOX_PATH_CHUNKED: which update kernel the handle runs."""
    rc = lib().neox_zero1_update_path(C.c_void_p(h))
    if rc < 0:
        _check(rc)
    return rc


def neox_zero1_plan(cfg: neox_zero1_config, segs, tables: bool = True):
    """-> (neox_zero1_plan_t, chunk list, tile words, changes): the decomposition create()
    would build, computed on the host (no device call; pointers are only compared)."""
    arr = (neox_segment * max(1, len(segs)))(*segs)
    plan = neox_zero1_plan_t()
    _check(lib().neox_zero1_plan(C.byref(cfg), arr, len(segs), C.byref(plan), None, 0, None, 0,
                                 None, 0))
    if not tables:
        return plan, [], [], []
    chunks = (neox_chunk_info * max(1, plan.update_chunks))()
    nw = plan.flat_tiles + 1 if plan.update_path == NEOX_PATH_FLAT else 0
    words = (C.c_uint32 * max(1, nw))()
    changes = (C.c_uint32 * max(1, plan.flat_changes))()
    _check(lib().neox_zero1_plan(C.byref(cfg), arr, len(segs), C.byref(plan), chunks,
                                 plan.update_chunks, words, nw, changes, plan.flat_changes))
    return plan, list(chunks[:plan.update_chunks]), list(words[:nw]), list(changes[:plan.flat_changes])


def neox_zero1_step_noalloc(cfg: neox_zero1_config, segs, state: neox_scaler_state_t, lr: float,
                            stream_ptr: int = 0) -> neox_scaler_state_t:
    """One step with no handle and no device allocation; `state` (the scaler state before
    the step) is overwritten with the state after it and returned.  Waits for the stream."""
    arr = (neox_segment * max(1, len(segs)))(*segs)
    _check(lib().neox_zero1_step_noalloc(C.byref(cfg), arr, len(segs), C.byref(state),
                                         C.c_float(lr), C.c_void_p(stream_ptr)))
    return state


def neox_zero1_timing_end(h: int, per_step: int = 0):
    """-> ([norm_ms, finalize_ms, update_ms] summed, steps); with per_step = K > 0 also
    the durations (ms) of the first K recorded steps."""
    ms = (C.c_double * 3)()
    n = C.c_int64()
    steps = (C.c_double * per_step)() if per_step > 0 else None
    _check(lib().neox_zero1_timing_end(C.c_void_p(h), ms, C.byref(n), steps, max(0, per_step)))
    if per_step > 0:
        return list(ms), n.value, list(steps[:min(n.value, per_step)])
    return list(ms), n.value


# --------------------------------------------------------------------------------------
# torch-facing conveniences (pointer extraction only)
# --------------------------------------------------------------------------------------

def segment(grad, half, master, exp_avg, exp_avg_sq, decay: bool, tensor_id=0, tensor_offset=0):
    """neox_segment over five 1-D CUDA tensors of equal length (no copies); exp_avg_sq
    may be None for the SGD optimizer."""
    import torch
    n = grad.numel()
    for t, dt in ((grad, None), (half, None), (master, torch.float32), (exp_avg, torch.float32),
                  (exp_avg_sq, torch.float32)):
        if t is None:
            continue
        if not t.is_cuda or t.numel() != n or not t.is_contiguous():
            raise ValueError("segment arrays must be contiguous CUDA tensors of equal length")
        if dt is not None and t.dtype != dt:
            raise ValueError("master / exp_avg / exp_avg_sq must be float32")
    if grad.dtype not in (torch.float16, torch.bfloat16) or half.dtype != grad.dtype:
        raise ValueError("grad and half must share float16 or bfloat16")
    return neox_segment(grad.data_ptr(), half.data_ptr(), master.data_ptr(), exp_avg.data_ptr(),
                        None if exp_avg_sq is None else exp_avg_sq.data_ptr(), n,
                        NEOX_SEG_DECAY if decay else 0, tensor_id, tensor_offset)


def current_stream_ptr() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


class Zero1:
    """Owner of one step handle.  The tensors behind the segments must outlive it."""

    def __init__(self, cfg: neox_zero1_config, segs, stream_ptr: int | None = None):
        self._segs = list(segs)
        self.handle = neox_zero1_create(cfg, self._segs,
                                        current_stream_ptr() if stream_ptr is None else stream_ptr)

    def step(self, lr: float, stream_ptr: int | None = None):
        neox_zero1_step(self.handle, lr, current_stream_ptr() if stream_ptr is None else stream_ptr)

    def state(self) -> neox_scaler_state_t:
        return neox_scaler_state(self.handle)

    def close(self):
        if self.handle:
            h, self.handle = self.handle, 0
            neox_zero1_destroy(h)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
