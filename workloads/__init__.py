"""Seeded synthetic workloads for the ZeRO-1 mixed-precision Adam step.

Shared by the tests, the benchmark and the smoke check.  This module only describes
shapes and draws random inputs (shard layouts, hyper-parameters, initial weights,
per-step gradients, overflow injections); it holds none of the step's arithmetic.

The shapes follow the pages' models: a Pythia-410M-like tensor list, a GPT-NeoX-20B
per-rank shard (hidden 6,144) and an OPT-175B-style shard (hidden 12,288, as in the
OPT paper card's compute-setup section).  No dataset is read: the gradients are
Gaussian stand-ins for the real ones.

Seeds: stream 0 = initial master weights, stream 1 = gradients of step k,
stream 2 = overflow injections, each mixed with the workload id.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F16, BF16 = 1, 2
DYNAMIC, STATIC = 0, 1

# Bit patterns of the non-finite values injected into gradients.
NONFINITE_BITS = {
    F16: {"+inf": 0x7C00, "-inf": 0xFC00, "nan": 0x7E00},
    BF16: {"+inf": 0x7F80, "-inf": 0xFF80, "nan": 0x7FC0},
}


@dataclasses.dataclass
class Hyper:
    lr: float = 6e-4
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.01
    clip_norm: float = 1.0
    predivide_factor: float = 1.0
    dp_world_size: int = 1
    dtype: int = F16
    scaler_mode: int = DYNAMIC
    init_scale: float = 65536.0
    growth_interval: int = 1000
    growth_factor: float = 2.0
    backoff_factor: float = 0.5
    min_scale: float = 1.0
    optimizer: int = 0             # 0 AdamW, 1 momentum SGD (no second moment)


@dataclasses.dataclass
class Workload:
    name: str
    wid: int                       # seed id
    segments: list                 # [(numel, decay)] in shard order
    hyper: Hyper
    flat: bool = True              # one contiguous buffer per array, else one per segment
    grad_sigma: float = 1e-4       # std of the unscaled gradient
    grad_mult: float = 1.0         # stored gradient = N(0, sigma) * S * grad_mult
    master_sigma: float = 0.02
    steps: int = 10
    injections: dict = dataclasses.field(default_factory=dict)  # step -> [(index, kind)]

    @property
    def numel(self) -> int:
        return int(sum(n for n, _ in self.segments))

    def offsets(self):
        off, out = 0, []
        for n, _ in self.segments:
            out.append(off)
            off += n
        return out


# --------------------------------------------------------------------------------------
# Shapes
# --------------------------------------------------------------------------------------

def pythia410m_tensors():
    """Pythia-410M-like tensor list in model order: [(numel, decay)].

    Embedding 50,304 x 1,024, then 24 layers of LN1 gain/bias, QKV weight 1,024 x 3,072
    and bias, output weight 1,024^2 and bias, LN2 gain/bias, FC weight 1,024 x 4,096 and
    bias, projection weight 4,096 x 1,024 and bias.  Weights and the embedding decay;
    biases and LayerNorm parameters do not.
    """
    h = 1024
    out = [(50304 * h, True)]
    for _ in range(24):
        out += [(h, False), (h, False), (h * 3 * h, True), (3 * h, False),
                (h * h, True), (h, False), (h, False), (h, False),
                (h * 4 * h, True), (4 * h, False), (4 * h * h, True), (h, False)]
    return out


def _layer_tensors(h):
    """One decoder layer of hidden size h in model order (LN1, QKV, out, LN2, FC, proj)."""
    return [(h, False), (h, False), (h * 3 * h, True), (3 * h, False), (h * h, True),
            (h, False), (h, False), (h, False), (h * 4 * h, True), (4 * h, False),
            (4 * h * h, True), (h, False)]


def _truncate(tensors, total):
    out, left = [], total
    for n, d in tensors:
        if left == 0:
            break
        take = min(n, left)
        out.append((take, d))
        left -= take
    assert left == 0
    return out


# --------------------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------------------

def tiny() -> Workload:
    """1,048,576 params, one decaying segment, 10 steps, +inf at element 777,777 on step 5."""
    return Workload("tiny_1m", 1, [(1 << 20, True)], Hyper(), steps=10,
                    injections={5: [(777_777, "+inf")]})


def pythia410m(rank: int, segments, dp: int = 8, steps: int = 20) -> Workload:
    """Rank `rank` of a DP=`dp` ZeRO-1 partition of the Pythia-410M-like tensor list.

    segments: the rank's [(numel, decay)] in shard order, as a partition of
    pythia410m_tensors() gives them (the library's for the GPU side, the oracle's for the
    oracle side): this module only sizes and seeds the buffers, it does not partition."""
    return Workload(f"pythia410m_dp{dp}_rank{rank}", 2, [(int(n), bool(d)) for n, d in segments],
                    Hyper(), steps=steps)


def neox20b_shard(steps: int = 100) -> Workload:
    """215,000,000-param GPT-NeoX-20B per-rank shard (20.6e9 / 96 ranks, rounded).

    Nine segments following a hidden-6,144 layer from its start: LN1 gain/bias, QKV
    weight and bias, output weight and bias, LN2 gain/bias, and the FC weight cut at
    the shard end."""
    segs = _truncate(_layer_tensors(6144), 215_000_000)
    assert len(segs) == 9
    return Workload("neox20b_shard_215m", 3, segs, Hyper(), grad_sigma=1e-5, steps=steps)


def multi_tensor(steps: int = 20, literal: bool = False, count: int = 5000,
                 total: int = 1_000_000_000) -> Workload:
    """5,000 separately allocated tensors, bf16, no loss scaling, 20% no-decay.

    Sizes are log-uniform over [2^10, 2^24].  Drawn literally their mean is ~1.7M, so
    5,000 of them hold ~8.6e9 params rather than the ~1e9 the workload names; the
    default rescales them to a ~1e9 total, keeping count and spread (`literal=True`
    keeps the raw draws)."""
    rng = np.random.default_rng([4, 0, 0])
    s = np.exp(rng.uniform(math.log(2.0 ** 10), math.log(2.0 ** 24), size=count))
    if literal:
        n = np.maximum(1, np.round(s)).astype(np.int64)
    else:
        n = np.maximum(1, np.round(s * total / s.sum())).astype(np.int64)
    nodecay = np.zeros(count, bool)
    nodecay[rng.permutation(count)[: count // 5]] = True
    segs = [(int(k), not bool(nd)) for k, nd in zip(n, nodecay)]
    hy = Hyper(dtype=BF16, scaler_mode=STATIC, init_scale=1.0)
    name = "multi_tensor_5000_bf16_literal" if literal else "multi_tensor_5000_bf16"
    return Workload(name, 4, segs, hy, flat=False, steps=steps)


def opt_large(numel: int = 6_000_000_000) -> Workload:
    """OPT-175B-style 6e9-param shard (96 GB of resident state), fp16, pre-divide 8.

    Layers of hidden 12,288 from a layer start, cut inside the fourth layer's output
    weight (41 segments).  D = 128 ranks, f = 8, clip 0.3, growth every 4 clean steps.
    Sequence of 39 steps: 3 clean, 20 forced overflows (+inf and NaN alternating at
    seeded positions; the scale falls from 2^16 to the 1.0 floor in 16 and stays there
    for 4 more), then 16 clean steps in which the scale doubles every 4."""
    segs = _truncate(_layer_tensors(12288) * 4, numel)
    hy = Hyper(clip_norm=0.3, predivide_factor=8.0, dp_world_size=128, growth_interval=4)
    rng = np.random.default_rng([5, 2, 0])
    inj = {}
    for k, step in enumerate(range(3, 23)):
        inj[step] = [(int(rng.integers(0, numel)), "+inf" if k % 2 == 0 else "nan")]
    return Workload("opt_style_6b", 5, segs, hy, grad_sigma=1e-5,
                    grad_mult=hy.dp_world_size / hy.predivide_factor, steps=39,
                    injections=inj)


# Workloads that need no partition; the Pythia-410M ranks are built from a partition by
# the caller (pythia410m).
BENCH_WORKLOADS = {
    "neox20b_shard_215m": neox20b_shard,
    "tiny_1m": tiny,
    "multi_tensor_5000_bf16": multi_tensor,
    "multi_tensor_5000_bf16_literal": lambda: multi_tensor(literal=True),
    "opt_style_6b": opt_large,
}


# --------------------------------------------------------------------------------------
# Host (numpy) draws: small cases
# --------------------------------------------------------------------------------------

def _to_half_bits_host(x32: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F16:
        with np.errstate(over="ignore"):
            return x32.astype(np.float16).view(np.uint16)
    import torch
    return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16).copy()


def host_init(w: Workload, n: int | None = None, seed_extra: int = 0):
    """Initial state on the host: master ~ N(0, master_sigma) fp32, half = cast(master),
    m = v = 0."""
    n = w.numel if n is None else n
    rng = np.random.default_rng([w.wid, 0, seed_extra])
    master = (rng.standard_normal(n) * w.master_sigma).astype(np.float32)
    half = _to_half_bits_host(master, w.hyper.dtype)
    return dict(master=master, half=half, m=np.zeros(n, np.float32), v=np.zeros(n, np.float32))


def host_grads(w: Workload, step: int, scale: float, n: int | None = None, seed_extra: int = 0):
    """Stored gradient of step `step`: cast(N(0, sigma) * scale * grad_mult), with the
    step's injections written in."""
    n = w.numel if n is None else n
    rng = np.random.default_rng([w.wid, 1, step, seed_extra])
    x = (rng.standard_normal(n) * (w.grad_sigma * scale * w.grad_mult)).astype(np.float32)
    bits = _to_half_bits_host(x, w.hyper.dtype)
    for idx, kind in w.injections.get(step, []):
        if idx < n:
            bits[idx] = NONFINITE_BITS[w.hyper.dtype][kind]
    return bits


# --------------------------------------------------------------------------------------
# Device (torch) draws: large cases, generated in place in HBM
# --------------------------------------------------------------------------------------

def _torch_seed(*parts) -> int:
    s = 0
    for p in parts:
        s = (s * 1_000_003 + int(p)) % (1 << 62)
    return s


def device_normal_(out, sigma: float, seed: int, piece: int = 1 << 27):
    """Fill a 1-D float32/float16/bfloat16 CUDA tensor with N(0, sigma) draws, drawn
    in fp32 and cast piece by piece (bounded temporaries)."""
    import torch
    g = torch.Generator(device=out.device)
    g.manual_seed(seed)
    n = out.numel()
    for lo in range(0, n, piece):
        hi = min(n, lo + piece)
        t = torch.randn(hi - lo, generator=g, device=out.device, dtype=torch.float32)
        t.mul_(sigma)
        out[lo:hi].copy_(t)
        del t


def device_init_(w: Workload, master, half, m, v, seed_extra: int = 0):
    device_normal_(master, w.master_sigma, _torch_seed(w.wid, 0, seed_extra))
    half.copy_(master)
    m.zero_()
    if v is not None:
        v.zero_()


def device_grads_(w: Workload, grad, step: int, scale: float, offset: int = 0,
                  seed_extra: int = 0):
    """Gradient of step `step` into the CUDA tensor `grad` (fp16/bf16), which holds
    elements [offset, offset + grad.numel()) of the shard."""
    device_normal_(grad, w.grad_sigma * scale * w.grad_mult,
                   _torch_seed(w.wid, 1, step, offset, seed_extra))
    inject_(w, grad, step, offset)


def inject_(w: Workload, grad, step: int, offset: int = 0):
    import torch
    for idx, kind in w.injections.get(step, []):
        if offset <= idx < offset + grad.numel():
            bits = NONFINITE_BITS[w.hyper.dtype][kind]
            grad.view(torch.int16)[idx - offset] = bits - (1 << 16) if bits >= 1 << 15 else bits
