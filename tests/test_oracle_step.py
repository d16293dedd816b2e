"""Pins of the oracle's step against closed forms, invariants and brute force.

Nothing here re-types the oracle's update: each check is a different statement of
what one step must produce (a closed form of Adam on special inputs, an invariant of
loss scaling, an exact sum, a run-length model of the scaler), chosen so that a
dropped term, a wrong sign or index, or swapped operands fail at least one.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O

F32_EPS = 2.0 ** -23


def ulps32(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    a = np.where(a < 0, -(a & 0x7FFFFFFF), a)
    b = np.where(b < 0, -(b & 0x7FFFFFFF), b)
    return np.abs(a - b)


def make_state(n, seed=0, dtype=O.F16, wsig=0.02):
    rng = np.random.default_rng(seed)
    master = (rng.standard_normal(n) * wsig).astype(np.float32)
    return dict(master=master, half=O.float_to_half(dtype, master),
                m=np.zeros(n, np.float32), v=np.zeros(n, np.float32))


def grads_from(values, dtype=O.F16):
    return O.float_to_half(dtype, np.asarray(values, np.float32))


def run_step(cfg, st, lr, grad, s, decay=True):
    seg = dict(grad=grad, decay=decay, **s)
    return O.step(cfg, st, lr, [seg])


# ----------------------------------------------------------------------------------
# Adam closed forms
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("decay", [True, False])
def test_first_step_closed_form(decay):
    """From m = v = 0, step 1 has m_hat = g and v_hat = g^2 whatever the betas, so
    w1 = w0 - lr * (g / (|g| + eps) + wd * w0 [decay])."""
    n = 4096
    rng = np.random.default_rng(1)
    S = 1024.0
    # unscaled gradient magnitudes spanning 1e-9 .. 1e-2 so eps matters at the bottom
    g_true = rng.standard_normal(n) * 10.0 ** rng.uniform(-9, -2, n)
    grad = grads_from(g_true * S)
    g = O.half_to_double(O.F16, grad) / S           # what the step sees after unscaling
    s = make_state(n, 2)
    w0 = s["master"].astype(np.float64)
    cfg = O.Config(clip_norm=0.0, weight_decay=0.1)
    st = O.Scaler(loss_scale=S)
    lr = np.float32(1e-3)
    run_step(cfg, st, lr, grad, s, decay)
    want = w0 - float(lr) * (g / (np.abs(g) + cfg.eps) + (cfg.weight_decay * w0 if decay else 0.0))
    assert ulps32(s["master"], want.astype(np.float32)).max() <= 1
    assert st.step == 1 and st.last_skipped == 0


def test_moments_are_normalised_ema():
    """Bias-corrected moments after t steps are weighted averages of g_k and g_k^2
    with weights proportional to beta^(t-k) (weights summing to one)."""
    n, T = 512, 6
    rng = np.random.default_rng(3)
    cfg = O.Config(beta1=0.8, beta2=0.97, eps=1e-7, weight_decay=0.0, clip_norm=0.0)
    st = O.Scaler(loss_scale=256.0, good_steps=0)
    s = make_state(n, 4)
    w = s["master"].astype(np.float64)
    wmax = np.abs(w)
    gs = []
    lr = np.float32(2e-3)
    sign = np.where(rng.standard_normal(n) < 0, -1.0, 1.0)
    for t in range(1, T + 1):
        # one sign per element across steps: the moments never cancel, so the FP32
        # storage of m, v and w between steps adds at most ~1/2 ulp of w per step
        grad = grads_from(sign * (0.1 + np.abs(rng.standard_normal(n))) * 1e-3 * st.loss_scale)
        gs.append(O.half_to_double(O.F16, grad) / st.loss_scale)
        run_step(cfg, st, lr, grad, s, decay=False)
        k = np.arange(1, t + 1)
        w1 = cfg.beta1 ** (t - k)
        w2 = cfg.beta2 ** (t - k)
        G = np.array(gs)
        mhat = (w1[:, None] * G).sum(0) / w1.sum()
        vhat = (w2[:, None] * G * G).sum(0) / w2.sum()
        w = w - float(lr) * mhat / (np.sqrt(vhat) + cfg.eps)
        wmax = np.maximum(wmax, np.abs(w))
        # each step rounds the stored master once: <= 1/2 ulp of the largest |w| so far
        assert (np.abs(s["master"] - w) <= t * F32_EPS * wmax).all(), t
    assert st.step == T


def test_constant_gradient_trajectory_with_decay():
    """Constant g and no clipping: m_hat = g, v_hat = g^2 at every t, so u = g/(|g|+eps)
    is constant and w_t = (1-a)^t w0 - lr*u*(1-(1-a)^t)/a with a = lr*wd."""
    n, T = 256, 12
    rng = np.random.default_rng(5)
    S = 4096.0
    grad = grads_from(rng.standard_normal(n) * 1e-3 * S)
    g = O.half_to_double(O.F16, grad) / S
    cfg = O.Config(weight_decay=0.05, clip_norm=0.0, growth_interval=10 ** 6)
    st = O.Scaler(loss_scale=S)
    s = make_state(n, 6)
    w0 = s["master"].astype(np.float64)
    lr = np.float32(1e-2)
    for _ in range(T):
        run_step(cfg, st, lr, grad, s, decay=True)
    a = float(lr) * cfg.weight_decay
    u = g / (np.abs(g) + cfg.eps)
    want = (1 - a) ** T * w0 - float(lr) * u * (1 - (1 - a) ** T) / a
    assert ulps32(s["master"], want.astype(np.float32)).max() <= 4


def test_beta_zero_is_sign_descent():
    """beta1 = beta2 = 0: m_hat = g, v_hat = g^2 at every step (not only the first)."""
    n = 300
    rng = np.random.default_rng(7)
    cfg = O.Config(beta1=0.0, beta2=0.0, eps=0.0, weight_decay=0.0, clip_norm=0.0)
    st = O.Scaler(loss_scale=1.0)
    s = make_state(n, 8)
    lr = np.float32(1e-3)
    for _ in range(3):
        w0 = s["master"].astype(np.float64)
        # eps = 0 leaves 0/0 at g = 0, so every gradient here is nonzero
        vals = np.sign(rng.standard_normal(n)) * (1e-3 + np.abs(rng.standard_normal(n)) * 0.01)
        grad = grads_from(vals)
        g = O.half_to_double(O.F16, grad)
        run_step(cfg, st, lr, grad, s, decay=False)
        want = w0 - float(lr) * np.sign(g)
        assert ulps32(s["master"], want.astype(np.float32)).max() <= 1


def test_eps_zero_is_undefined_at_a_zero_gradient():
    """With eps = 0 Adam's direction m_hat / sqrt(v_hat) is 0 / 0 wherever the gradient
    and both moments are zero (a padding element, an unused embedding row), so the
    master weight becomes NaN: the reason the library requires eps > 0.  Elements with a
    nonzero gradient stay finite."""
    cfg = O.Config(eps=0.0, weight_decay=0.0)
    st = O.Scaler(loss_scale=1.0)
    s = make_state(4, 11)
    grad = grads_from([0.0, 1e-3, 0.0, -2e-3])
    run_step(cfg, st, np.float32(1e-3), grad, s, decay=False)
    assert st.step == 1 and not st.last_skipped
    assert np.isnan(s["master"][[0, 2]]).all()
    assert np.isfinite(s["master"][[1, 3]]).all()


@pytest.mark.parametrize("dtype", [O.F16, O.BF16])
def test_half_copy_is_the_cast_of_the_stored_master(dtype):
    """The half copy is the FP32 master as stored, rounded to the half format."""
    n = 5000
    rng = np.random.default_rng(21)
    cfg = O.Config(dtype=dtype, scaler_mode=O.STATIC)
    st = O.Scaler(loss_scale=1.0)
    s = make_state(n, 22, dtype)
    for k in range(3):
        run_step(cfg, st, np.float32(3e-3), grads_from(rng.standard_normal(n) * 1e-2, dtype), s)
        assert np.array_equal(s["half"], O.float_to_half(dtype, s["master"]))


def test_decay_only_and_identity():
    """g = 0: moments stay 0 and the update is pure decoupled decay, w*(1-lr*wd);
    a no-decay segment is left bitwise unchanged."""
    n = 1000
    cfg = O.Config(weight_decay=0.1)
    lr = np.float32(3e-3)
    for decay in (True, False):
        st = O.Scaler()
        s = make_state(n, 9)
        before = {k: v.copy() for k, v in s.items()}
        run_step(cfg, st, lr, np.zeros(n, np.uint16), s, decay)
        assert not s["m"].any() and not s["v"].any()
        if decay:
            want = before["master"].astype(np.float64) * (1 - float(lr) * cfg.weight_decay)
            assert ulps32(s["master"], want.astype(np.float32)).max() <= 1
            assert np.array_equal(s["half"], O.float_to_half(O.F16, s["master"]))
        else:
            for k in s:
                assert np.array_equal(s[k], before[k]), k
        assert st.last_norm == 0.0 and st.last_coef == 1.0 and st.step == 1


# ----------------------------------------------------------------------------------
# Norm and clip
# ----------------------------------------------------------------------------------

def test_norm_three_four_five():
    cfg = O.Config(clip_norm=0.0)
    st = O.Scaler(loss_scale=1.0)
    s = make_state(2, 10)
    run_step(cfg, st, np.float32(0.0), grads_from([3.0, 4.0]), s)
    assert st.last_norm == 5.0


def test_norm_all_equal():
    n = 1 << 16
    x = 0.375
    cfg = O.Config(clip_norm=0.0, predivide_factor=2.0, dp_world_size=8)
    st = O.Scaler(loss_scale=64.0)
    s = make_state(n, 11)
    run_step(cfg, st, np.float32(0.0), grads_from(np.full(n, x)), s)
    assert st.last_norm == x * (2.0 / (8 * 64.0)) * math.sqrt(n)


@pytest.mark.parametrize("dtype", [O.F16, O.BF16])
def test_norm_exact_sum(dtype):
    """sumsq against an exactly rounded sum (math.fsum) of the exactly unscaled
    squares; with an inexact unscale factor (D = 3) the squares are rounded once."""
    n = 50_000
    rng = np.random.default_rng(12)
    grad = grads_from(rng.standard_normal(n) * 3.0, dtype)
    inv, inv32 = 1.0 / 3.0, np.float32(1.0 / 3.0)
    sumsq, of = O.scan(dtype, grad, inv, float(inv32))
    x = O.half_to_double(dtype, grad)
    exact = math.fsum(float(Fraction(v) * Fraction(inv)) ** 2 for v in x)
    assert of == 0
    assert abs(sumsq - exact) <= 1e-12 * exact


def test_clip_norm_after_clip():
    """With clipping active the applied gradient has norm c: after step 1 from zero
    moments, ||m1|| = (1 - beta1) * c and sum(v1) = (1 - beta2) * c^2 (both moments see
    the clipped gradient)."""
    n = 20_000
    rng = np.random.default_rng(13)
    for c in (1.0, 0.3):
        cfg = O.Config(clip_norm=c)
        st = O.Scaler(loss_scale=128.0)
        grad = grads_from(rng.standard_normal(n) * 0.05 * 128.0)
        s = make_state(n, 14)
        run_step(cfg, st, np.float32(1e-4), grad, s)
        assert st.last_norm > c
        m1 = math.sqrt(math.fsum(float(v) ** 2 for v in s["m"].astype(np.float64)))
        assert abs(m1 - (1 - cfg.beta1) * c) <= 1e-5 * (1 - cfg.beta1) * c
        v1 = math.fsum(float(v) for v in s["v"].astype(np.float64))
        assert abs(v1 - (1 - cfg.beta2) * c * c) <= 1e-5 * (1 - cfg.beta2) * c * c
        assert abs(st.last_coef * st.last_norm - c) <= 1e-12


def test_clip_inactive_below_threshold_and_disabled():
    # clipping only above the threshold: a norm of exactly c (four gradients of 0.5,
    # exact in fp16) and of 0.8c keep the coefficient at 1; 1.25c gives 0.8
    for vals, c, want in (([0.5] * 4, 1.0, 1.0), ([0.4] * 4, 1.0, 1.0), ([0.625] * 4, 1.0, 0.8)):
        st = O.Scaler(loss_scale=1.0)
        g = grads_from(vals)
        s = make_state(4, 16)
        run_step(O.Config(clip_norm=c), st, np.float32(1e-3), g, s)
        assert abs(st.last_coef - want) <= 1e-15, (vals, st.last_coef)
    n = 1000
    grad = grads_from(np.full(n, 0.01))
    for c in (1.0, 0.0, -1.0):
        st = O.Scaler(loss_scale=1.0)
        s = make_state(n, 15)
        run_step(O.Config(clip_norm=c), st, np.float32(1e-3), grad, s)
        assert st.last_coef == 1.0
    grad = grads_from(np.full(n, 1.0))         # norm ~31.6
    st = O.Scaler(loss_scale=1.0)
    s = make_state(n, 15)
    run_step(O.Config(clip_norm=0.0), st, np.float32(1e-3), grad, s)
    assert st.last_coef == 1.0 and st.last_norm > 30


# ----------------------------------------------------------------------------------
# Overflow skip and the loss scaler
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [O.F16, O.BF16])
def test_skip_every_position(dtype):
    """A non-finite gradient anywhere: every array and t bitwise unchanged, scale
    halved, good_steps reset, skip counted.  Brute force over all positions."""
    n = 64
    rng = np.random.default_rng(16)
    base = grads_from(rng.standard_normal(n) * 100.0, dtype)
    bad = {O.F16: (0x7C00, 0xFC00, 0x7E00), O.BF16: (0x7F80, 0xFF80, 0x7FC0)}[dtype]
    for pos in range(n):
        for b in bad:
            grad = base.copy()
            grad[pos] = b
            s = make_state(n, 17, dtype)
            before = {k: v.copy() for k, v in s.items()}
            st = O.Scaler(loss_scale=1024.0, good_steps=5, step=7)
            run_step(O.Config(dtype=dtype), st, np.float32(1e-3), grad, s)
            for k in s:
                assert np.array_equal(s[k], before[k])
            assert (st.loss_scale, st.good_steps, st.step, st.skipped_total,
                    st.consecutive_overflows, st.last_skipped) == (512.0, 0, 7, 1, 1, 1)
            assert math.isinf(st.last_norm)


def test_fp16_largest_finite_is_not_overflow():
    grad = np.array([0x7BFF, 0xFBFF, 0x0001], np.uint16)   # +-65504 and the smallest subnormal
    st = O.Scaler(loss_scale=1.0)
    s = make_state(3, 18)
    run_step(O.Config(clip_norm=0.0), st, np.float32(1e-6), grad, s)
    assert st.last_skipped == 0 and st.step == 1
    assert st.last_norm == math.sqrt(2 * 65504.0 ** 2 + 2.0 ** -48)


def test_overflow_from_unscale_in_fp32():
    """The overflow decision is taken on the FP32 unscaled value: a finite bf16
    gradient whose unscaled value exceeds the FP32 range (scale below 1) skips."""
    big = np.array([np.float32(2.0 ** 120)], np.float32)
    grad = O.float_to_half(O.BF16, big)
    cfg = O.Config(dtype=O.BF16, min_scale=2.0 ** -20)
    st = O.Scaler(loss_scale=2.0 ** -10)                  # inv = 2^10 -> 2^130 overflows fp32
    s = make_state(1, 19, O.BF16)
    run_step(cfg, st, np.float32(1e-3), grad, s)
    assert st.last_skipped == 1 and st.loss_scale == 2.0 ** -11
    st = O.Scaler(loss_scale=2.0 ** -5)                   # inv = 2^5 -> 2^125 is finite
    run_step(cfg, st, np.float32(1e-3), grad, s)
    assert st.last_skipped == 0


# x * inv overflows FP32 when both are rounded to FP32 first, but not when the product
# is taken in double and rounded once: x = (1 + 2^-7) 2^126 (exact in bf16), inv a double
# just below the threshold whose FP32 rounding lies above it.
OVERFLOW_WINDOW_X = (1 + 2.0 ** -7) * 2.0 ** 126
OVERFLOW_WINDOW_INV = 3.9689921219219535


def test_overflow_is_decided_on_the_fp32_product():
    """Reading: the unscaled gradient is the FP32 value fp32(x) * fp32(inv); a value that
    overflows there is an overflow even where the exact product would round to a finite
    FP32 number."""
    x, inv = OVERFLOW_WINDOW_X, OVERFLOW_WINDOW_INV
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(x) * np.float32(inv)) and np.isfinite(np.float32(x * inv))
    g = O.float_to_half(O.BF16, np.array([x, 1.0], np.float32))
    assert O.half_to_double(O.BF16, g)[0] == x
    cfg = O.Config(dtype=O.BF16, scaler_mode=O.STATIC, predivide_factor=inv)
    st = O.Scaler(loss_scale=1.0)
    i, i32 = O.unscale_factor(cfg, st)
    assert i == inv and i32 == np.float32(inv)
    _, of = O.scan(O.BF16, g, i, i32)
    assert of == 1
    _, of = O.scan(O.BF16, g[1:], i, i32)
    assert of == 0


def _scaler_model(seq, S0, interval, min_scale, growth=2.0, backoff=0.5):
    """Run-length model: split the sequence at overflows; within a clean run the scale
    doubles once per full `interval` clean steps counted from the run's start (or from
    the initial counter before any overflow); each overflow halves with a floor."""
    S, good, t, skips, consec = S0, 0, 0, 0, 0
    runs = []
    cur = 0
    for o in seq:
        if o:
            runs.append(("clean", cur))
            runs.append(("of", 1))
            cur = 0
        else:
            cur += 1
    runs.append(("clean", cur))
    for kind, L in runs:
        if kind == "of":
            S = max(S * backoff, min_scale)
            good, skips, consec = 0, skips + 1, consec + 1
        elif L:
            total = good + L
            S = S * growth ** (total // interval)
            good = total % interval
            t += L
            consec = 0
    return S, good, t, skips, consec


def test_scaler_every_sequence_of_length_12():
    cfg = O.Config(growth_interval=3, min_scale=2.0 ** -2)
    for seq in itertools.product((0, 1), repeat=12):
        st = O.Scaler(loss_scale=4.0)
        for o in seq:
            O.decide(cfg, st, o, 1.0)
        want = _scaler_model(seq, 4.0, 3, 2.0 ** -2)
        got = (st.loss_scale, st.good_steps, st.step, st.skipped_total, st.consecutive_overflows)
        assert got == want, seq


def test_static_scaler_never_moves():
    # also above the floor, where a back-off would show
    for S in (1.0, 1024.0):
        cfg = O.Config(scaler_mode=O.STATIC, growth_interval=1)
        st = O.Scaler(loss_scale=S)
        for o in (0, 1, 1, 0, 0, 0, 1):
            O.decide(cfg, st, o, 0.0)
        assert st.loss_scale == S and st.skipped_total == 3 and st.step == 4


def test_scale_floor_and_collapse_counter():
    cfg = O.Config(min_scale=1.0)
    st = O.Scaler(loss_scale=2.0 ** 16)
    for k in range(20):
        O.decide(cfg, st, 1, 0.0)
        assert st.loss_scale == max(2.0 ** (15 - k), 1.0)
    assert st.consecutive_overflows == 20 and st.loss_scale == 1.0


def test_growth_stays_finite():
    cfg = O.Config(growth_interval=1)
    st = O.Scaler(loss_scale=2.0 ** 127)
    O.decide(cfg, st, 0, 0.0)
    assert st.loss_scale == 2.0 ** 127 and st.good_steps == 0


# ----------------------------------------------------------------------------------
# Invariances
# ----------------------------------------------------------------------------------

def _run_seq(cfg, S, grads, n, seed):
    st = O.Scaler(loss_scale=S, good_steps=0)
    s = make_state(n, seed)
    for g in grads:
        run_step(cfg, st, np.float32(1e-3), g, s)
    return s, st


def test_loss_scale_invariance():
    """(grad * 2^j, S * 2^j): bitwise-identical results while no fp16 value overflows
    or changes exponent range."""
    n = 4096
    rng = np.random.default_rng(20)
    raw = [rng.standard_normal(n) * 0.01 for _ in range(3)]
    cfg = O.Config(growth_interval=10 ** 6, clip_norm=0.05)
    ref_s, ref_st = _run_seq(cfg, 1024.0, [grads_from(r * 1024.0) for r in raw], n, 21)
    for j in (-2, 3):
        S = 1024.0 * 2.0 ** j
        s, st = _run_seq(cfg, S, [grads_from(r * S) for r in raw], n, 21)
        for k in s:
            assert np.array_equal(s[k], ref_s[k]), (j, k)
        assert st.last_norm == ref_st.last_norm


def test_predivide_invariance():
    """Only the ratio f / D enters the unscale: pairs with one ratio agree bitwise,
    another ratio does not (clipping off, so the magnitude is not normalised away)."""
    n = 4096
    rng = np.random.default_rng(22)
    raw = [grads_from(rng.standard_normal(n) * 10.0) for _ in range(3)]
    outs = []
    for f, D in ((1.0, 1), (8.0, 8), (16.0, 16), (128.0, 128)):
        cfg = O.Config(predivide_factor=f, dp_world_size=D, clip_norm=0.0)
        outs.append(_run_seq(cfg, 256.0, raw, n, 23))
    for s, st in outs[1:]:
        for k in s:
            assert np.array_equal(s[k], outs[0][0][k]), k
    cfg = O.Config(predivide_factor=2.0, dp_world_size=1, clip_norm=0.0)
    s, _ = _run_seq(cfg, 256.0, raw, n, 23)
    assert not np.array_equal(s["m"], outs[0][0]["m"])


def test_sharding_equals_unsharded_without_clipping():
    """Elementwise work is independent per element: with clipping off and no
    overflow, the per-rank shards concatenated equal the unsharded step bitwise."""
    tensors = [(37, True), (5, False), (120, True), (3, False), (64, True)]
    numel = [n for n, _ in tensors]
    decay = [d for _, d in tensors]
    D, A = 4, 8
    total = sum(numel)
    rng = np.random.default_rng(24)
    cfg = O.Config(clip_norm=0.0)
    lr = np.float32(1e-3)
    full = make_state(total, 25)
    grads = [grads_from(rng.standard_normal(total) * 0.01 * 65536.0) for _ in range(3)]
    shard_states = []
    segs_by_rank = []
    P = None
    for r in range(D):
        segs, P = O.partition(numel, decay, D, r, A)
        segs_by_rank.append(segs)
    padded = P * D

    def pad(a, fill=0):
        out = np.full(padded, fill, a.dtype)
        out[:a.size] = a
        return out

    # unsharded: one segment per tensor
    st_full = O.Scaler()
    for g in grads:
        segs, off = [], 0
        for n, d in tensors:
            segs.append(dict(grad=g[off:off + n], decay=d,
                             **{k: v[off:off + n] for k, v in full.items()}))
            off += n
        O.step(cfg, st_full, lr, segs)
    # sharded
    padded_state = {k: pad(v) for k, v in make_state(total, 25).items()}
    for r in range(D):
        st = O.Scaler()
        for g in grads:
            gp = pad(g)
            segs = []
            for sg in segs_by_rank[r]:
                lo = r * P + sg["shard_offset"]
                hi = lo + sg["numel"]
                segs.append(dict(grad=gp[lo:hi], decay=bool(sg["flags"] & O.DECAY),
                                 **{k: v[lo:hi] for k, v in padded_state.items()}))
            O.step(cfg, st, lr, segs)
    for k in full:
        assert np.array_equal(padded_state[k][:total], full[k]), k
    assert not padded_state["master"][total:].any()


def test_resident_bytes_per_param():
    """16 bytes of resident model state per parameter (OPT paper card, bottlenecks)."""
    import os
    here = os.path.dirname(os.path.abspath(__file__))
    vals = {}
    with open(os.path.join(here, "golden", "opt175b_state_bytes.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    s = make_state(10, 26)
    per_param = (s["master"].itemsize + s["m"].itemsize + s["v"].itemsize
                 + s["half"].itemsize + np.dtype(np.uint16).itemsize)
    assert per_param == vals["bytes_per_param"]
    assert abs(vals["params"] * per_param - vals["total_bytes_approx"]) / 2.8e12 < 0.01


# ----------------------------------------------------------------------------------
# SGD with heavy-ball momentum (the alternative optimizer the OPT card reports trying)
# ----------------------------------------------------------------------------------

def _sgd_step(cfg, st, lr, grad, s, decay):
    return O.step(cfg, st, lr, [dict(grad=grad, decay=decay, half=s["half"], master=s["master"],
                                     m=s["m"], v=None)])


@pytest.mark.parametrize("decay", [True, False])
def test_sgd_first_step_closed_form(decay):
    """From zero momentum: m1 = g and w1 = w0 - lr*(g + wd*w0 [decay])."""
    n = 2048
    rng = np.random.default_rng(50)
    S = 512.0
    grad = grads_from(rng.standard_normal(n) * 1e-2 * S)
    g = O.half_to_double(O.F16, grad) / S
    cfg = O.Config(optimizer=O.SGD, beta1=0.9, weight_decay=0.1, clip_norm=0.0)
    st = O.Scaler(loss_scale=S)
    s = make_state(n, 51)
    w0 = s["master"].astype(np.float64)
    lr = np.float32(1e-2)
    _sgd_step(cfg, st, lr, grad, s, decay)
    assert ulps32(s["m"], g.astype(np.float32)).max() <= 0
    want = w0 - float(lr) * (g + (cfg.weight_decay * w0 if decay else 0.0))
    assert ulps32(s["master"], want.astype(np.float32)).max() <= 1


def test_sgd_constant_gradient_geometric_momentum():
    """Constant g, no decay: m_t = g (1 - mu^t)/(1 - mu) and
    w_T = w0 - lr * g * sum_{t=1..T} (1 - mu^t)/(1 - mu)."""
    n, T, mu = 512, 15, 0.8
    rng = np.random.default_rng(52)
    grad = grads_from(rng.standard_normal(n) * 1e-2)
    g = O.half_to_double(O.F16, grad)
    cfg = O.Config(optimizer=O.SGD, beta1=mu, weight_decay=0.0, clip_norm=0.0,
                   growth_interval=10 ** 6)
    st = O.Scaler(loss_scale=1.0)
    s = make_state(n, 53)
    w0 = s["master"].astype(np.float64)
    wmax = np.abs(w0)
    lr = np.float32(1e-3)
    for t in range(1, T + 1):
        _sgd_step(cfg, st, lr, grad, s, False)
        mt = g * (1 - mu ** t) / (1 - mu)
        assert (np.abs(s["m"] - mt) <= t * F32_EPS * np.abs(mt)).all(), t
    want = w0 - float(lr) * g * sum((1 - mu ** t) / (1 - mu) for t in range(1, T + 1))
    wmax = np.maximum(wmax, np.abs(want))
    assert (np.abs(s["master"] - want) <= T * F32_EPS * wmax).all()


def test_sgd_zero_momentum_is_plain_sgd_and_skip_is_untouched():
    n = 300
    rng = np.random.default_rng(54)
    cfg = O.Config(optimizer=O.SGD, beta1=0.0, weight_decay=0.0, clip_norm=0.0)
    st = O.Scaler(loss_scale=1.0)
    s = make_state(n, 55)
    lr = np.float32(1e-2)
    for _ in range(3):
        w0 = s["master"].astype(np.float64)
        grad = grads_from(rng.standard_normal(n) * 0.1)
        _sgd_step(cfg, st, lr, grad, s, False)
        want = w0 - float(lr) * O.half_to_double(O.F16, grad)
        assert ulps32(s["master"], want.astype(np.float32)).max() <= 1
    grad[17] = 0x7C00
    before = {k: v.copy() for k, v in s.items()}
    _sgd_step(cfg, st, lr, grad, s, False)
    for k in s:
        assert np.array_equal(s[k], before[k])
    assert st.last_skipped == 1 and st.step == 3


def test_pieces_cover_every_element_once():
    """The all-core baseline's static partition: contiguous pieces of the concatenation,
    in order, each element exactly once, piece lengths differing by at most one."""
    rng = np.random.default_rng(12)
    for _ in range(200):
        sizes = [int(x) for x in rng.integers(1, 50, int(rng.integers(1, 8)))]
        parts = int(rng.integers(1, 12))
        got = O.pieces(sizes, parts)
        assert len(got) == parts
        flat = [(k, i) for runs in got for k, lo, hi in runs for i in range(lo, hi)]
        assert flat == [(k, i) for k, n in enumerate(sizes) for i in range(n)]
        lens = [sum(hi - lo for _, lo, hi in runs) for runs in got]
        assert max(lens) - min(lens) <= 1


@pytest.mark.parametrize("threads", [1, 3, 8])
def test_parallel_step_equals_the_serial_step(threads):
    """The threaded composition of scan / decide / update over static pieces gives the
    serial step's arrays bit for bit (clipping inactive, so the norm's summation order
    only moves its last bits) and its decisions."""
    sizes, rng = [1000, 3, 20_000, 7, 4096], np.random.default_rng(13)

    def shard():
        out = []
        for i, n in enumerate(sizes):
            s = make_state(n, 20 + i)
            s["grad"] = grads_from(rng.standard_normal(n) * 1e-4 * 65536)
            s["decay"] = i % 2 == 0
            out.append(s)
        return out

    a = shard()
    b = [{k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in s.items()} for s in a]
    sa, sb = O.Scaler(), O.Scaler()
    for _ in range(3):
        O.step(O.Config(), sa, np.float32(6e-4), a)
        O.step_parallel(O.Config(), sb, np.float32(6e-4), b, threads)
        assert (sa.step, sa.loss_scale, sa.skipped_total) == (sb.step, sb.loss_scale, sb.skipped_total)
        assert abs(sa.last_sumsq - sb.last_sumsq) <= 1e-12 * sa.last_sumsq and sa.last_coef == 1.0
        for x, y in zip(a, b):
            for k in ("half", "master", "m", "v"):
                assert np.array_equal(x[k], y[k]), k
