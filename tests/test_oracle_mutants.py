"""The oracle's pins against planted mistakes.

Each case below is one plausible slip in oracle/oracle.c (a dropped term, a wrong sign,
a swapped operand, an off-by-one, a wrong rounding rule).  The test writes the source
with that one change, builds it like the real oracle, and runs the oracle's pins against
it (tests/test_oracle_*.py, without the two exhaustive/whole-model tests that take most
of their time): some pin must fail for every mutant, and all of them must pass for the
unchanged source built the same way.  Runs on the CPU only.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import build  # noqa: E402

SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement, which occurrence: 1 = first)
MUTANTS = [
    ("first moment not bias-corrected",
     "double u = (m1 / d->bc1) / den;", "double u = m1 / den;", 1),
    ("eps inside the root",
     "double den = sqrt(v1 / d->bc2) + eps;", "double den = sqrt(v1 / d->bc2 + eps);", 1),
    ("update sign flipped",
     "double w1 = w0 - rate * u;", "double w1 = w0 + rate * u;", 1),
    ("betas swapped in the first moment",
     "double m1 = b1 * m0 + (1.0 - b1) * g;", "double m1 = b2 * m0 + (1.0 - b2) * g;", 1),
    ("clip coefficient inverted",
     "coef = cfg->clip_norm / norm;", "coef = norm / cfg->clip_norm;", 1),
    ("gradient not unscaled in the update",
     "double g = (x * d->inv) * d->coef;", "double g = x * d->coef;", 1),
    ("|g| instead of g^2 in the norm",
     "acc += g * g;", "acc += fabs(g);", 1),
    ("|g| instead of g^2 in the second moment",
     "(1.0 - b2) * (g * g);", "(1.0 - b2) * fabs(g);", 1),
    ("overflow test misses NaN",
     "return (b & 0x7F800000u) == 0x7F800000u;", "return (b & 0x7FFFFFFFu) == 0x7F800000u;", 1),
    ("bias correction one step ahead",
     "d->bc1 = 1.0 - pow(cfg->beta1, (double)t);", "d->bc1 = 1.0 - pow(cfg->beta1, (double)(t + 1));", 1),
    ("weight decay halved",
     "if (decay) u += wd * w0;", "if (decay) u += 0.5 * wd * w0;", 1),
    ("growth one clean step late",
     "st->good_steps >= cfg->growth_interval", "st->good_steps > cfg->growth_interval", 1),
    ("no floor under the loss scale",
     "st->loss_scale = s < floor_ ? floor_ : s;", "st->loss_scale = s;", 1),
    ("clean-step counter kept on overflow",
     "        st->good_steps = 0;\n        st->consecutive_overflows += 1;",
     "        st->consecutive_overflows += 1;", 1),
    ("subnormal spacing off by a factor 2",
     "v = ldexp((double)m, 1 - f.bias - f.mant_bits);", "v = ldexp((double)m, -f.bias - f.mant_bits);", 1),
    ("ties rounded away from zero",
     "double k = nearbyint(ldexp(a, -q));", "double k = round(ldexp(a, -q));", 1),
    ("skipped step still updates",
     "    if (d->skip) return;\n    const double b1", "    const double b1", 1),
    ("pre-divide factor applied upside down",
     "double v = cfg->predivide_factor / ((double)cfg->dp_world_size * (double)st->loss_scale);",
     "double v = 1.0 / (cfg->predivide_factor * (double)cfg->dp_world_size * (double)st->loss_scale);", 1),
    ("momentum SGD damped like Adam",
     "double m1 = mu * m0 + g;", "double m1 = mu * m0 + (1.0 - mu) * g;", 1),
    ("shard length not padded to D x align",
     "uint64_t padded = (total + unit - 1) / unit * unit;", "uint64_t padded = total;", 1),
    ("SGD decay dropped", "if (decay) u += wd * w0;", "if (0) u += wd * w0;", 2),
    ("SGD update sign flipped", "double w1 = w0 - rate * u;", "double w1 = w0 + rate * u;", 2),
    ("bf16 exponent bias off by one",
     "f.exp_bits = 8; f.bias = 127;", "f.exp_bits = 8; f.bias = 126;", 1),
    ("NaN encoded without the quiet bit",
     "(uint16_t)(1u << (f.mant_bits - 1));", "(uint16_t)1u;", 1),
    ("largest finite rounds to infinity",
     "if (r > max_finite) return sign | all_ones_exp;",
     "if (r >= max_finite) return sign | all_ones_exp;", 1),
    ("partition tensor offset from the rank start",
     "s->tensor_offset = e - tstart;", "s->tensor_offset = e - (uint64_t)rank * P;", 1),
    ("growth by the back-off factor",
     "scale_times(st->loss_scale, cfg->growth_factor)",
     "scale_times(st->loss_scale, cfg->backoff_factor)", 1),
    ("overflow run not reset by a clean step", "    st->consecutive_overflows = 0;\n", "", 1),
    ("skipped step reports norm 0", "st->last_norm = INFINITY;", "st->last_norm = 0.0;", 1),
    ("decay applied to no-decay elements", "if (decay) u += wd * w0;", "u += wd * w0;", 1),
    ("clip below the threshold",
     "norm > cfg->clip_norm) coef", "norm >= cfg->clip_norm * 0.5) coef", 1),
    ("m and v from the unclipped gradient",
     "double g = (x * d->inv) * d->coef;", "double g = (x * d->inv);", 1),
    ("second moment not bias-corrected",
     "double den = sqrt(v1 / d->bc2) + eps;", "double den = sqrt(v1) + eps;", 1),
    ("static scaler backs off",
     "if (cfg->scaler_mode == ORC_DYNAMIC) {\n            float s = scale_times",
     "if (1) {\n            float s = scale_times", 1),
    ("partition padding to D only",
     "uint64_t unit = (uint64_t)dp_world_size * (uint64_t)align;",
     "uint64_t unit = (uint64_t)dp_world_size;", 1),
    ("half copy cast from the unrounded master",
     "half[i] = orc_float_to_half(cfg->dtype, wf);",
     "half[i] = orc_float_to_half(cfg->dtype, (float)(w1 * (1 + 1e-7)));", 1),
    ("overflow taken on the double product",
     "float g32 = (float)x * inv32;", "float g32 = (float)(x * inv);", 1),
    ("growth past the FP32 range taken",
     "if (!f32_nonfinite(s)) st->loss_scale = s;", "st->loss_scale = s;", 1),
    ("clean-step counter kept after a growth",
     "        if (!f32_nonfinite(s)) st->loss_scale = s;\n        st->good_steps = 0;\n",
     "        if (!f32_nonfinite(s)) st->loss_scale = s;\n", 1),
    ("skipped step advances t",
     "        st->skipped_total += 1;\n", "        st->skipped_total += 1;\n        st->step += 1;\n", 1),
    ("overflow run not accumulated",
     "st->consecutive_overflows += 1;", "st->consecutive_overflows = 1;", 1),
    ("second moment from the unclipped gradient",
     "double v1 = b2 * v0 + (1.0 - b2) * (g * g);",
     "double v1 = b2 * v0 + (1.0 - b2) * ((x * d->inv) * (x * d->inv));", 1),
    ("decay on a half-updated weight",
     "if (decay) u += wd * w0;\n        double w1 = w0 - rate * u;\n\n        float wf = (float)w1;\n"
     "        exp_avg[i] = (float)m1;\n        exp_avg_sq",
     "if (decay) u += wd * (w0 - rate * u);\n        double w1 = w0 - rate * u;\n\n"
     "        float wf = (float)w1;\n        exp_avg[i] = (float)m1;\n        exp_avg_sq", 1),
    ("norm of the FP32 unscaled value",
     "double g = x * inv;\n        acc += g * g;", "double g = (double)g32;\n        acc += g * g;", 1),
    ("bias correction in single precision",
     "d->bc1 = 1.0 - pow(cfg->beta1, (double)t);",
     "d->bc1 = 1.0 - (double)powf((float)cfg->beta1, (float)t);", 1),
    ("scale floor test inverted",
     "st->loss_scale = s < floor_ ? floor_ : s;", "st->loss_scale = s > floor_ ? floor_ : s;", 1),
    ("truncating half cast",
     "double k = nearbyint(ldexp(a, -q));", "double k = trunc(ldexp(a, -q));", 1),
    ("eps added before the bias correction",
     "double den = sqrt(v1 / d->bc2) + eps;", "double den = (sqrt(v1) + eps) / sqrt(d->bc2);", 1),
    ("padding decays",
     "s->flags = (owner < ntensors && tensor_decay[owner]) ? ORC_DECAY : 0;",
     "s->flags = (owner >= ntensors || tensor_decay[owner]) ? ORC_DECAY : 0;", 1),
    ("rank of an element off by one",
     "if (e / P != (uint64_t)rank) continue;", "if (e / (P + 1) != (uint64_t)rank) continue;", 1),
    ("one tensor advanced per element",
     "while (ti < ntensors && e >= tstart + tensor_numel[ti]) {",
     "if (ti < ntensors && e >= tstart + tensor_numel[ti]) {", 1),
    ("shard offset taken in the tensor",
     "s->shard_offset = e - (uint64_t)rank * P;", "s->shard_offset = e - tstart;", 1),
    ("padding given the last tensor's id",
     "s->tensor_id = (uint32_t)owner;",
     "s->tensor_id = (uint32_t)(owner < ntensors ? owner : ntensors - 1);", 1),
]

PINS = [os.path.join(ROOT, "tests", f) for f in
        ("test_oracle_step.py", "test_oracle_formats.py", "test_oracle_partition.py")]
SKIP_SLOW = "not exhaustive and not pythia410m_layout"


def _mutate(text, old, new, which):
    at = -1
    for _ in range(which):
        at = text.index(old, at + 1)
    return text[:at] + new + text[at + len(old):]


def _build(src_text, workdir, name):
    os.makedirs(workdir, exist_ok=True)
    shutil.copy(os.path.join(ROOT, "oracle", "oracle.h"), workdir)
    c = os.path.join(workdir, f"{name}.c")
    so = os.path.join(workdir, f"{name}.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *build.CFLAGS, "-o", so, c, "-lm"], check=True,
                   capture_output=True)
    return so


def _pins(so):
    env = {**os.environ, "NEOX_ORACLE_SO": so, "PYTHONDONTWRITEBYTECODE": "1"}
    r = subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-m", "not gpu",
                        "-k", SKIP_SLOW, "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with open(SRC) as f:
        text = f.read()
    for name, old, new, which in MUTANTS:
        assert text.count(old) >= which, f"{name}: {old!r} not in oracle.c"
    jobs = [("control", text)] + [(f"m{i}", _mutate(text, old, new, which))
                                  for i, (_, old, new, which) in enumerate(MUTANTS)]
    sos = {tag: _build(src, str(tmp_path), tag) for tag, src in jobs}
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = dict(zip(sos, ex.map(_pins, sos.values())))
    rc, out = results.pop("control")
    assert rc == 0, "the unchanged oracle must pass its pins:\n" + out
    survived = [MUTANTS[int(tag[1:])][0] for tag, (rc, _) in results.items() if rc != 1]
    assert not survived, f"mistakes no pin catches: {survived}"
