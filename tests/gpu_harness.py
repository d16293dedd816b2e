"""Helpers for the GPU parity tests (not collected by pytest).

DeviceShard holds a workload's five arrays in HBM (torch tensors as plain device
memory), builds the segment list for the C ABI, and copies windows back to the host.
`Checker` steps the library and the oracle side by side on the same bytes and
compares them at the tolerances the step is held to:
  - skip / scale / counter decisions: bit-exact;
  - global gradient norm: 1e-5 relative;
  - master, exp_avg, exp_avg_sq: |gpu - oracle| <= 2e-6 * max(|oracle|, s), s the
    magnitude of the largest term that entered the element's last operation (as the
    oracle reports it);
  - half copy: within 1 unit in the last place of the oracle's value.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import mixed_precision_zero_amd as Z
import workloads as W
from oracle import oracle as O

TOL_REL = 2e-6
# Below the FP32 normal range a relative bound is finer than the format's own grid;
# there the bound is a few subnormal quanta (2^-149 each).
TOL_ABS_SUBNORMAL = 4 * 2.0 ** -149
TOL_NORM = 1e-5
HALF_ULPS = 1


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype):
    return torch.float16 if dtype == W.F16 else torch.bfloat16


def lib_config(w: W.Workload, **over):
    h = w.hyper
    cfg = Z.neox_zero1_default_config(
        beta1=h.beta1, beta2=h.beta2, eps=h.eps, weight_decay=h.weight_decay,
        clip_norm=h.clip_norm, predivide_factor=h.predivide_factor,
        dp_world_size=h.dp_world_size, dtype=h.dtype, scaler_mode=h.scaler_mode,
        growth_interval=h.growth_interval, init_scale=h.init_scale,
        growth_factor=h.growth_factor, backoff_factor=h.backoff_factor,
        min_scale=h.min_scale, optimizer=h.optimizer)
    for k, v in over.items():
        setattr(cfg, k, v)
    return cfg


def oracle_config(w: W.Workload):
    h = w.hyper
    return O.Config(beta1=h.beta1, beta2=h.beta2, eps=h.eps, weight_decay=h.weight_decay,
                    clip_norm=h.clip_norm, predivide_factor=h.predivide_factor,
                    dp_world_size=h.dp_world_size, dtype=h.dtype, scaler_mode=h.scaler_mode,
                    growth_interval=h.growth_interval, growth_factor=h.growth_factor,
                    backoff_factor=h.backoff_factor, min_scale=h.min_scale,
                    optimizer=h.optimizer)


def u16(t):
    """bit view of a CUDA half tensor as host uint16"""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f32(t):
    return t.cpu().numpy()


ARRAYS = ("grad", "half", "master", "m", "v")


class DeviceShard:
    """Five device arrays per segment.  flat=True: one buffer per array and segments are
    views into it at `misalign` + running offset; flat=False: one allocation per array
    per segment."""

    def __init__(self, w: W.Workload, flat: bool | None = None, misalign=(0, 0, 0, 0, 0),
                 device="cuda"):
        self.w = w
        self.flat = w.flat if flat is None else flat
        dt = torch_dtype(w.hyper.dtype)
        kinds = (dt, dt, torch.float32, torch.float32, torch.float32)
        self.sgd = w.hyper.optimizer == 1
        names = ARRAYS[:4] if self.sgd else ARRAYS     # SGD keeps no second moment
        self.segs = []                    # per segment: dict name -> 1-D tensor view
        if self.flat:
            n = w.numel
            self.buffers = {"v": None}
            for name, k, mis in zip(names, kinds, misalign):
                self.buffers[name] = torch.empty(n + mis, dtype=k, device=device)[mis:]
            off = 0
            for numel, _ in w.segments:
                seg = {a: self.buffers[a][off:off + numel] for a in names}
                seg.setdefault("v", None)
                self.segs.append(seg)
                off += numel
        else:
            self.buffers = None
            for numel, _ in w.segments:
                seg = {a: torch.empty(numel + mis, dtype=k, device=device)[mis:]
                       for a, k, mis in zip(names, kinds, misalign)}
                seg.setdefault("v", None)
                self.segs.append(seg)

    def init_(self, seed_extra=0):
        if self.flat:
            b = self.buffers
            W.device_init_(self.w, b["master"], b["half"], b["m"], b["v"], seed_extra)
        else:
            for i, s in enumerate(self.segs):
                W.device_init_(self.w, s["master"], s["half"], s["m"], s["v"],
                               seed_extra * 100_003 + i + 1)

    def grads_(self, step, scale, seed_extra=0):
        if self.flat:
            W.device_grads_(self.w, self.buffers["grad"], step, scale, 0, seed_extra)
        else:
            off = 0
            for s in self.segs:
                W.device_grads_(self.w, s["grad"], step, scale, off, seed_extra)
                off += s["grad"].numel()

    def neox_segments(self):
        out = []
        for (numel, decay), s in zip(self.w.segments, self.segs):
            out.append(Z.segment(s["grad"], s["half"], s["master"], s["m"], s["v"], decay))
        return out

    def decay(self, i):
        return bool(self.w.segments[i][1])

    def host_window(self, i, lo, hi):
        s = self.segs[i]
        return dict(grad=u16(s["grad"][lo:hi]), half=u16(s["half"][lo:hi]),
                    master=f32(s["master"][lo:hi]), m=f32(s["m"][lo:hi]),
                    v=None if s["v"] is None else f32(s["v"][lo:hi]))

    def host_grad_pieces(self, piece=1 << 28):
        for s in self.segs:
            g = s["grad"]
            for lo in range(0, g.numel(), piece):
                yield u16(g[lo:lo + piece])

    def full_windows(self):
        return [(i, 0, s["grad"].numel()) for i, s in enumerate(self.segs)]


def ordinal16(bits):
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def assert_close(name, got, want, scale, where=""):
    g = got.astype(np.float64)
    o = want.astype(np.float64)
    err = np.abs(g - o)
    tol = TOL_REL * np.maximum(np.abs(o), scale) + TOL_ABS_SUBNORMAL
    bad = ~(err <= tol)
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{name}{where}: {int(bad.sum())} of {g.size} out of tolerance; "
                             f"first at {i}: gpu {g[i]!r} oracle {o[i]!r} scale {scale[i]!r}")


def half_bounds(dtype, master, scale):
    """Ordinals of the half values a master within the master bound of the oracle's
    `master` (TOL_REL * max(|master|, scale) + TOL_ABS_SUBNORMAL) rounds to: the lowest
    and the highest.  The bound is widened outward by one FP32 ulp at each end."""
    m = master.astype(np.float64)
    tol = TOL_REL * np.maximum(np.abs(m), scale) + TOL_ABS_SUBNORMAL
    lo = np.nextafter((m - tol).astype(np.float32), np.float32(-np.inf))
    hi = np.nextafter((m + tol).astype(np.float32), np.float32(np.inf))
    return ordinal16(O.float_to_half(dtype, lo)), ordinal16(O.float_to_half(dtype, hi))


def assert_half_close(got, want, where="", dtype=None, master=None, scale=None):
    """Half copy within HALF_ULPS of the oracle's; where the master's own bound is wider
    than that (an update that nearly cancels the weight leaves a result far smaller than
    the terms the bound is relative to), any rounding of a master inside that bound."""
    og, ow = ordinal16(got), ordinal16(want)
    bad = np.abs(og - ow) > HALF_ULPS
    if bad.any() and master is not None:
        lo, hi = half_bounds(dtype, master[bad], scale[bad])
        inside = (og[bad] >= np.minimum(lo, ow[bad] - HALF_ULPS)) & \
                 (og[bad] <= np.maximum(hi, ow[bad] + HALF_ULPS))
        bad[np.flatnonzero(bad)[inside]] = False
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"half{where}: {int(bad.sum())} elements outside the bound; "
                             f"first at {i}: gpu {got[i]:#06x} oracle {want[i]:#06x}")


def assert_state_equal(gst, ost: O.Scaler, where="", norm=True):
    got = (float(np.float32(gst.loss_scale)), gst.good_steps, gst.step, gst.skipped_total,
           gst.consecutive_overflows, gst.last_skipped)
    want = (float(np.float32(ost.loss_scale)), ost.good_steps, ost.step, ost.skipped_total,
            ost.consecutive_overflows, ost.last_skipped)
    assert got == want, f"state{where}: gpu {got} oracle {want}"
    if ost.last_skipped:
        assert np.isinf(gst.last_grad_norm) and gst.last_clip_coef == 1.0
    elif norm:
        assert abs(gst.last_grad_norm - ost.last_norm) <= TOL_NORM * ost.last_norm, \
            f"norm{where}: gpu {gst.last_grad_norm!r} oracle {ost.last_norm!r}"
        assert abs(gst.last_sumsq - ost.last_sumsq) <= 2 * TOL_NORM * ost.last_sumsq
        assert abs(gst.last_clip_coef - ost.last_coef) <= TOL_NORM * ost.last_coef + 1e-7


class Checker:
    """Steps a library handle and the oracle side by side."""

    def __init__(self, shard: DeviceShard, cfg=None, stream=None, **cfg_over):
        self.shard = shard
        self.w = shard.w
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self.cfg = cfg if cfg is not None else lib_config(self.w, **cfg_over)
        self.ocfg = oracle_config(self.w)
        self.ost = O.Scaler(loss_scale=float(np.float32(self.cfg.init_scale)),
                            good_steps=self.cfg.init_good_steps, step=self.cfg.init_step,
                            skipped_total=self.cfg.init_skipped,
                            consecutive_overflows=self.cfg.init_consecutive_overflows)
        self.handle = Z.neox_zero1_create(self.cfg, shard.neox_segments(), self.stream.cuda_stream)

    def close(self):
        if self.handle:
            Z.neox_zero1_destroy(self.handle)
            self.handle = 0

    def scale(self):
        return Z.neox_scaler_state(self.handle).loss_scale

    def oracle_scan(self, threads=1):
        """Overflow flag and squared norm of the whole gradient, by the oracle.  With
        threads > 1 the pieces are scanned concurrently and their partial sums added in
        piece order (a blocked index-order sum; it differs from the sequential one only
        in the last bits, far inside the norm tolerance)."""
        inv, inv32 = O.unscale_factor(self.ocfg, self.ost)
        dt = self.w.hyper.dtype
        if threads <= 1:
            sumsq, of = 0.0, 0
            for g in self.shard.host_grad_pieces():
                sumsq, of = O.scan(dt, g, inv, inv32, sumsq, of)
            return sumsq, of
        from concurrent.futures import ThreadPoolExecutor
        futs = []
        with ThreadPoolExecutor(max_workers=threads) as ex:
            for g in self.shard.host_grad_pieces(piece=1 << 26):
                futs.append(ex.submit(O.scan, dt, g, inv, inv32))
            parts = [f.result() for f in futs]
        sumsq = 0.0
        for s, _ in parts:
            sumsq += s
        return sumsq, int(any(o for _, o in parts))

    def step(self, lr, windows=None, check=True, overflow=None, threads=1, where=""):
        """One step on both sides.  windows: [(segment, lo, hi)] compared elementwise
        (None = every element); check=False compares decisions only.  overflow: the
        step's overflow flag when it is known by construction (the scan is skipped and
        the norm is not compared); otherwise the oracle scans the whole gradient."""
        sh = self.shard
        if windows is None:
            windows = sh.full_windows()
        torch.cuda.synchronize()
        pre = [(i, lo, hi, sh.host_window(i, lo, hi)) for i, lo, hi in windows] if check else []
        if overflow is None:
            sumsq, of = self.oracle_scan(threads)
        else:
            sumsq, of = float("nan"), int(overflow)
        Z.neox_zero1_step(self.handle, lr, self.stream.cuda_stream)
        gst = Z.neox_scaler_state(self.handle)
        d = O.decide(self.ocfg, self.ost, of, 0.0 if overflow is not None else sumsq)
        assert_state_equal(gst, self.ost, where, norm=overflow is None)
        if check and overflow is not None and not d.skip:
            raise ValueError("an elementwise check of an applied step needs the oracle's "
                             "own norm (pass overflow=None)")
        if not check:
            return gst, d
        posts = [sh.host_window(i, lo, hi) for i, lo, hi, _ in pre]

        def compare(i, lo, hi, p, post):
            tag = f"{where} seg {i} [{lo}:{hi})"
            if d.skip:
                for k in ("half", "master", "m", "v"):
                    if p[k] is not None:
                        assert np.array_equal(post[k], p[k]), f"{k}{tag} changed on a skipped step"
                return
            o = {k: (None if p[k] is None else p[k].copy()) for k in ARRAYS}
            if sh.sgd:
                sm, sw = O.update_sgd(self.ocfg, d, np.float32(lr), o["grad"], o["half"],
                                      o["master"], o["m"], sh.decay(i), scales=True)
            else:
                sm, sv, sw = O.update(self.ocfg, d, np.float32(lr), o["grad"], o["half"],
                                      o["master"], o["m"], o["v"], sh.decay(i), scales=True)
                assert_close("exp_avg_sq", post["v"], o["v"], sv, tag)
            assert_close("exp_avg", post["m"], o["m"], sm, tag)
            assert_close("master", post["master"], o["master"], sw, tag)
            assert_half_close(post["half"], o["half"], tag, self.w.hyper.dtype, o["master"], sw)
            # the half copy is exactly the stored FP32 master rounded to the half format
            own = O.float_to_half(self.w.hyper.dtype, post["master"])
            bad = post["half"] != own
            assert not bad.any(), (f"half{tag}: {int(bad.sum())} elements differ from the "
                                   f"cast of the GPU's own master")

        # each window in pieces of at most PIECE elements (the oracle's update of one piece
        # does not depend on any other element), on `threads` host threads
        PIECE = 1 << 23
        jobs = []
        for (i, lo, hi, p), post in zip(pre, posts):
            for a in range(0, hi - lo, PIECE):
                b = min(hi - lo, a + PIECE)
                cut = {k: (None if v is None else v[a:b]) for k, v in p.items()}
                pcut = {k: (None if v is None else v[a:b]) for k, v in post.items()}
                jobs.append((i, lo + a, lo + b, cut, pcut))
        if threads <= 1 or len(jobs) == 1:
            for j in jobs:
                compare(*j)
        else:
            from concurrent.futures import ThreadPoolExecutor
            with ThreadPoolExecutor(max_workers=threads) as ex:
                for f in [ex.submit(compare, *j) for j in jobs]:
                    f.result()
        return gst, d
