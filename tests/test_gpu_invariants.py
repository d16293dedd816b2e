"""Invariants checked on the GPU alone, bit for bit, with no oracle in the loop.

- The 8 data-parallel shards of the Pythia-410M layout, stepped one after another on
  this GPU, equal the unsharded step when nothing couples the ranks (no clipping, no
  overflow): ZeRO-1 shards only elementwise work.
- Loss-scale and pre-divide changes that scale the gradient buffer by exact powers of
  two (the buffer holds S·D/f times the mean gradient) leave every output unchanged,
  the squared norm included, with clipping active."""
import numpy as np
import pytest
import torch

import mixed_precision_zero_amd as Z
import workloads as W
from gpu_harness import log

pytestmark = pytest.mark.gpu

ARR = ("grad", "half", "master", "m", "v")


def _alloc(n, dt):
    out = {k: torch.empty(n, dtype=dt, device="cuda") for k in ("grad", "half")}
    out.update({k: torch.empty(n, dtype=torch.float32, device="cuda") for k in ("master", "m", "v")})
    return out


def _segs(buf, pieces):
    """pieces: (offset, numel, decay) into the five arrays of buf."""
    return [Z.segment(*(buf[k][o:o + n] for k in ARR), d) for o, n, d in pieces]


def test_eight_rank_shards_equal_the_unsharded_step():
    tensors = W.pythia410m_tensors()
    numel = [n for n, _ in tensors]
    decay = [d for _, d in tensors]
    N, D, A = sum(numel), 8, 64
    dt = torch.float16
    gen = torch.Generator(device="cuda").manual_seed(410)
    full = _alloc(N, dt)
    full["master"].normal_(0.0, 0.02, generator=gen)
    full["half"].copy_(full["master"].to(dt))
    full["m"].zero_()
    full["v"].zero_()
    offs = np.cumsum([0] + numel[:-1])
    pieces = [(int(o), n, d) for o, (n, d) in zip(offs, tensors)]

    ranks = []
    for r in range(D):
        parts, P = Z.neox_zero1_partition(numel, decay, D, r, A)
        lo, hi = r * P, min(N, (r + 1) * P)
        buf = _alloc(P, dt)
        for k in ARR:
            buf[k].zero_()
        for k in ("half", "master", "m", "v"):
            buf[k][:hi - lo].copy_(full[k][lo:hi])
        rp = [(p.shard_offset, p.numel, bool(p.flags & Z.NEOX_SEG_DECAY)) for p in parts]
        ranks.append(dict(lo=lo, hi=hi, P=P, buf=buf, pieces=rp))
    log(f"case 8 shards of {N} params, {ranks[0]['P']} per rank")

    cfg = Z.neox_zero1_default_config(clip_norm=0.0, dp_world_size=D, predivide_factor=2.0)
    stream = torch.cuda.current_stream().cuda_stream
    hf = Z.neox_zero1_create(cfg, _segs(full, pieces), stream)
    hr = [Z.neox_zero1_create(cfg, _segs(rk["buf"], rk["pieces"]), stream) for rk in ranks]
    try:
        grad = torch.empty(N, dtype=dt, device="cuda")
        for k in range(3):
            S = Z.neox_scaler_state(hf).loss_scale
            grad.normal_(0.0, 1e-4 * S, generator=gen)
            full["grad"].copy_(grad)
            for rk in ranks:
                rk["buf"]["grad"][:rk["hi"] - rk["lo"]].copy_(grad[rk["lo"]:rk["hi"]])
            Z.neox_zero1_step(hf, 1e-3, stream)
            for h in hr:
                Z.neox_zero1_step(h, 1e-3, stream)
        torch.cuda.synchronize()
        sf = Z.neox_scaler_state(hf)
        assert sf.step == 3 and sf.skipped_total == 0
        for h in hr:
            s = Z.neox_scaler_state(h)
            assert (s.step, s.skipped_total, s.loss_scale) == (sf.step, sf.skipped_total, sf.loss_scale)
        for k in ("half", "master", "m", "v"):
            cat = torch.cat([rk["buf"][k][:rk["hi"] - rk["lo"]] for rk in ranks])
            assert torch.equal(cat, full[k]), k
        last = ranks[-1]
        for k in ("half", "master", "m", "v"):   # the padding stays zero
            assert not last["buf"][k][last["hi"] - last["lo"]:].any(), k
    finally:
        Z.neox_zero1_destroy(hf)
        for h in hr:
            Z.neox_zero1_destroy(h)


def _exact_grads(rng, n, dtype, steps):
    """Unscaled gradients as half-format bit patterns with magnitudes in [2^-10, 2^-1):
    every power-of-two rescaling used below stays normal and finite in the format."""
    out = []
    for _ in range(steps):
        sign = rng.integers(0, 2, n).astype(np.uint16) << 15
        if dtype == W.F16:
            bits = sign | (rng.integers(5, 15, n).astype(np.uint16) << 10) | rng.integers(0, 1 << 10, n).astype(np.uint16)
        else:
            bits = sign | (rng.integers(117, 127, n).astype(np.uint16) << 7) | rng.integers(0, 1 << 7, n).astype(np.uint16)
        out.append(bits)
    return out


@pytest.mark.parametrize("dtype", [W.F16, W.BF16], ids=["f16", "bf16"])
def test_loss_scale_and_predivide_invariance(dtype):
    sizes = [100_000, 3, 77_777, 4096, 1]
    decays = [True, False, True, False, True]
    n = sum(sizes)
    rng = np.random.default_rng(77)
    gbar = _exact_grads(rng, n, dtype, 3)
    dt = torch.float16 if dtype == W.F16 else torch.bfloat16
    offs = np.cumsum([0] + sizes[:-1])
    pieces = [(int(o), s, d) for o, s, d in zip(offs, sizes, decays)]
    # (loss scale S, pre-divide f, ranks D): the buffer holds S*D/f times the gradient
    combos = [(1.0, 1.0, 1), (256.0, 1.0, 1), (1024.0, 2.0, 8), (1.0, 1.0, 8), (1.0, 4.0, 1)]
    stream = torch.cuda.current_stream().cuda_stream
    init = torch.Generator(device="cuda").manual_seed(3)
    w0 = torch.empty(n, dtype=torch.float32, device="cuda").normal_(0.0, 0.02, generator=init)
    results = []
    for S, f, D in combos:
        buf = _alloc(n, dt)
        buf["master"].copy_(w0)
        buf["half"].copy_(w0.to(dt))
        buf["m"].zero_()
        buf["v"].zero_()
        cfg = Z.neox_zero1_default_config(dtype=dtype, scaler_mode=Z.NEOX_SCALER_STATIC,
                                          init_scale=S, predivide_factor=f, dp_world_size=D,
                                          clip_norm=0.5)
        h = Z.neox_zero1_create(cfg, _segs(buf, pieces), stream)
        try:
            sumsq = []
            for bits in gbar:
                g = torch.from_numpy(bits.view(np.int16)).to("cuda").view(dt)
                buf["grad"].copy_(g.float().mul_(S * D / f).to(dt))
                Z.neox_zero1_step(h, 1e-3, stream)
                st = Z.neox_scaler_state(h)
                assert st.last_skipped == 0 and st.last_clip_coef < 1.0
                sumsq.append(st.last_sumsq)
        finally:
            Z.neox_zero1_destroy(h)
        torch.cuda.synchronize()
        results.append(({k: buf[k].clone() for k in ("half", "master", "m", "v")}, sumsq))
        log(f"case S={S} f={f} D={D}: sumsq {sumsq}")
    base, base_sumsq = results[0]
    for (out, sumsq), combo in zip(results[1:], combos[1:]):
        assert sumsq == base_sumsq, combo
        for k in base:
            assert torch.equal(out[k], base[k]), (combo, k)
