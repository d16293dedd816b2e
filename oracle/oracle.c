/*
 * oracle.c -- plain CPU reference of the ZeRO-1 mixed-precision Adam step.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): used by tests/, the smoke check and the
 * benchmark's CPU-baseline leg, never by the library.  Scalar loops, double
 * arithmetic, no blocking, no reordering.  Build without fast-math and without FP
 * contraction so every line means what it says:
 *     gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math oracle.c -lm
 */
#include "oracle.h"

#include <math.h>
#include <string.h>

/* ------------------------------------------------------------------------------ */
/* Number formats                                                                  */
/* ------------------------------------------------------------------------------ */

/* Field widths of the two half formats (IEEE-754 binary16; bfloat16 = the top 16
 * bits of binary32).  Both have the sign in bit 15. */
typedef struct { int mant_bits, exp_bits, bias; } fmt_t;
static fmt_t fmt_of(int32_t dtype) {
    fmt_t f;
    if (dtype == ORC_BF16) { f.mant_bits = 7;  f.exp_bits = 8; f.bias = 127; }
    else                   { f.mant_bits = 10; f.exp_bits = 5; f.bias = 15;  }
    return f;
}

/* Decode: value = (-1)^s * 2^(e - bias) * (1 + m / 2^p) for normal numbers,
 * (-1)^s * 2^(1 - bias) * (m / 2^p) for subnormals, all-ones exponent = inf / NaN. */
double orc_half_to_double(int32_t dtype, uint16_t bits) {
    fmt_t f = fmt_of(dtype);
    int s = bits >> 15;
    int e = (bits >> f.mant_bits) & ((1 << f.exp_bits) - 1);
    int m = bits & ((1 << f.mant_bits) - 1);
    double v;
    if (e == (1 << f.exp_bits) - 1) v = m ? NAN : INFINITY;
    else if (e == 0)                v = ldexp((double)m, 1 - f.bias - f.mant_bits);
    else                            v = ldexp((double)((1 << f.mant_bits) + m), e - f.bias - f.mant_bits);
    return s ? -v : v;
}

/* Encode with round-to-nearest, ties to even: find the spacing 2^q of representable
 * numbers around |x| (fixed at the subnormal spacing below the smallest normal),
 * round |x| / 2^q to the nearest integer (nearbyint honours the default
 * round-to-nearest-even mode), and map values above the largest finite number to
 * infinity.  NaN becomes the quiet NaN with the input's sign. */
uint16_t orc_float_to_half(int32_t dtype, float x) {
    fmt_t f = fmt_of(dtype);
    const int emin = 1 - f.bias, emax = f.bias;
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    const uint16_t all_ones_exp = (uint16_t)(((1u << f.exp_bits) - 1u) << f.mant_bits);
    double a = fabs((double)x);
    if (isnan(x)) return sign | all_ones_exp | (uint16_t)(1u << (f.mant_bits - 1));
    if (isinf(a)) return sign | all_ones_exp;
    if (a == 0.0) return sign;

    int e2;
    frexp(a, &e2);                     /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    int q = (E > emin ? E : emin) - f.mant_bits;
    double k = nearbyint(ldexp(a, -q)); /* exact scaling, then one RNE rounding */
    double r = ldexp(k, q);
    double max_finite = ldexp(2.0 - ldexp(1.0, -f.mant_bits), emax);
    if (r > max_finite) return sign | all_ones_exp;
    if (r < ldexp(1.0, emin)) return sign | (uint16_t)k;   /* subnormal: k < 2^p */
    frexp(r, &e2);
    E = e2 - 1;
    uint32_t mant = (uint32_t)ldexp(r, f.mant_bits - E) - (1u << f.mant_bits);
    return sign | (uint16_t)((uint32_t)(E + f.bias) << f.mant_bits) | (uint16_t)mant;
}

void orc_float_to_half_array(int32_t dtype, const float* x, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_float_to_half(dtype, x[i]);
}

void orc_half_to_double_array(int32_t dtype, const uint16_t* bits, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_half_to_double(dtype, bits[i]);
}

static int f32_nonfinite(float x) {
    uint32_t b;
    memcpy(&b, &x, sizeof b);
    return (b & 0x7F800000u) == 0x7F800000u;
}

/* ------------------------------------------------------------------------------ */
/* The step                                                                        */
/* ------------------------------------------------------------------------------ */

/* Unscale factor.  The stored gradient is the sum over D ranks of each rank's
 * gradient of the loss scaled by S and pre-divided by f [OPT paper card, section
 * "方法适配": pre-divide factor; section "计算设置": dynamic loss scaling].  The
 * mean unscaled gradient is therefore stored * f / (D * S). */
void orc_unscale_factor(const orc_config* cfg, const orc_scaler* st, double* inv, float* inv32) {
    double v = cfg->predivide_factor / ((double)cfg->dp_world_size * (double)st->loss_scale);
    *inv = v;
    *inv32 = (float)v;
}

/* Overflow test and global squared L2 norm of the unscaled gradient.  The overflow
 * decision is integer-valued, so it is taken in the precision the method keeps the
 * unscaled gradient in (FP32): any non-finite fp32(float(x) * fp32(inv)).  The norm
 * is the exact definition: sum of (x * inv)^2, x * inv in double, summed in index
 * order. */
void orc_scan(int32_t dtype, const uint16_t* grad, int64_t n, double inv, float inv32,
              double* sumsq, int32_t* overflow) {
    double acc = *sumsq;
    int32_t of = *overflow;
    for (int64_t i = 0; i < n; ++i) {
        double x = orc_half_to_double(dtype, grad[i]);
        float g32 = (float)x * inv32;
        if (f32_nonfinite(g32)) of = 1;
        double g = x * inv;
        acc += g * g;
    }
    *sumsq = acc;
    *overflow = of;
}

static float scale_times(float s, double factor) {
    return (float)((double)s * factor);
}

/* Finalize one step.
 *  - Overflow: skip the update, leave t alone, back the scale off (dynamic mode) but
 *    not below min_scale, reset the clean-step counter, count the skip.  A run of
 *    these is the "scale collapse" the OPT card calls a divergence symptom
 *    [OPT paper card, sections "瓶颈" and "方法适配"].
 *  - Clean: clip coefficient min(1, c / ||g||) for c > 0 (clip thresholds 1.0 and 0.3,
 *    section "方法适配"), t += 1, bias corrections 1 - beta^t (Kingma & Ba), and the
 *    scale grows by the growth factor after growth_interval clean steps in a row
 *    (Micikevicius et al. 2018).  A growth that would leave FP32 range is not taken. */
void orc_decide(const orc_config* cfg, orc_scaler* st, int32_t overflow, double sumsq,
                orc_decision* d) {
    orc_unscale_factor(cfg, st, &d->inv, &d->inv32);
    if (overflow) {
        d->skip = 1;
        d->coef = 1.0;
        d->bc1 = d->bc2 = 0.0;
        d->t = st->step;
        if (cfg->scaler_mode == ORC_DYNAMIC) {
            float s = scale_times(st->loss_scale, cfg->backoff_factor);
            float floor_ = (float)cfg->min_scale;
            st->loss_scale = s < floor_ ? floor_ : s;
        }
        st->good_steps = 0;
        st->consecutive_overflows += 1;
        st->skipped_total += 1;
        st->last_skipped = 1;
        st->last_sumsq = 0.0;
        st->last_norm = INFINITY;
        st->last_coef = 1.0;
        return;
    }
    double norm = sqrt(sumsq);
    double coef = 1.0;
    if (cfg->clip_norm > 0.0 && norm > cfg->clip_norm) coef = cfg->clip_norm / norm;
    int64_t t = st->step + 1;
    d->skip = 0;
    d->coef = coef;
    d->t = t;
    d->bc1 = 1.0 - pow(cfg->beta1, (double)t);
    d->bc2 = 1.0 - pow(cfg->beta2, (double)t);

    st->step = t;
    st->good_steps += 1;
    if (cfg->scaler_mode == ORC_DYNAMIC && st->good_steps >= cfg->growth_interval) {
        float s = scale_times(st->loss_scale, cfg->growth_factor);
        if (!f32_nonfinite(s)) st->loss_scale = s;
        st->good_steps = 0;
    }
    st->consecutive_overflows = 0;
    st->last_skipped = 0;
    st->last_sumsq = sumsq;
    st->last_norm = norm;
    st->last_coef = coef;
}

static double dmax(double a, double b) { return a > b ? a : b; }

/* AdamW on one run of elements [Kingma & Ba 2015 with decoupled decay, Loshchilov &
 * Hutter]: the unscaled, clipped gradient g updates the FP32 moments; the update
 * direction is the bias-corrected first moment over the root of the bias-corrected
 * second moment plus eps; decaying elements add wd * (pre-update weight); the FP32
 * master moves by -lr times that; the half copy is the master rounded to the half
 * format [OPT paper card, section "计算设置": FP32 Adam state, FP16 weights]. */
void orc_update(const orc_config* cfg, const orc_decision* d, float lr,
                const uint16_t* grad, uint16_t* half, float* master, float* exp_avg,
                float* exp_avg_sq, int64_t n, int32_t decay,
                double* s_m, double* s_v, double* s_w) {
    if (d->skip) return;
    const double b1 = cfg->beta1, b2 = cfg->beta2, eps = cfg->eps, wd = cfg->weight_decay;
    const double rate = (double)lr;
    for (int64_t i = 0; i < n; ++i) {
        double x = orc_half_to_double(cfg->dtype, grad[i]);
        double g = (x * d->inv) * d->coef;
        double m0 = exp_avg[i], v0 = exp_avg_sq[i], w0 = master[i];
        double m1 = b1 * m0 + (1.0 - b1) * g;
        double v1 = b2 * v0 + (1.0 - b2) * (g * g);
        double den = sqrt(v1 / d->bc2) + eps;
        double u = (m1 / d->bc1) / den;
        if (decay) u += wd * w0;
        double w1 = w0 - rate * u;

        float wf = (float)w1;
        exp_avg[i] = (float)m1;
        exp_avg_sq[i] = (float)v1;
        master[i] = wf;
        half[i] = orc_float_to_half(cfg->dtype, wf);

        double sm = dmax(fabs(m1), dmax(b1 * fabs(m0), (1.0 - b1) * fabs(g)));
        double sv = dmax(v1, dmax(b2 * v0, (1.0 - b2) * g * g));
        double su = (sm / d->bc1) / den + (decay ? wd * fabs(w0) : 0.0);
        if (s_m) s_m[i] = sm;
        if (s_v) s_v[i] = sv;
        if (s_w) s_w[i] = dmax(fabs(w1), dmax(fabs(w0), rate * su));
    }
}

/* Heavy-ball momentum SGD (Polyak; the form m = beta*m + g of Sutskever et al. 2013)
 * with the same decoupled decay as the AdamW path; the OPT card (section "方法适配")
 * reports SGD being tried in place of Adam.  The unscale, clip and skip are shared with
 * AdamW; no bias correction. */
void orc_update_sgd(const orc_config* cfg, const orc_decision* d, float lr,
                    const uint16_t* grad, uint16_t* half, float* master, float* exp_avg,
                    int64_t n, int32_t decay, double* s_m, double* s_w) {
    if (d->skip) return;
    const double mu = cfg->beta1, wd = cfg->weight_decay, rate = (double)lr;
    for (int64_t i = 0; i < n; ++i) {
        double x = orc_half_to_double(cfg->dtype, grad[i]);
        double g = (x * d->inv) * d->coef;
        double m0 = exp_avg[i], w0 = master[i];
        double m1 = mu * m0 + g;
        double u = m1;
        if (decay) u += wd * w0;
        double w1 = w0 - rate * u;

        float wf = (float)w1;
        exp_avg[i] = (float)m1;
        master[i] = wf;
        half[i] = orc_float_to_half(cfg->dtype, wf);

        double sm = dmax(fabs(m1), dmax(mu * fabs(m0), fabs(g)));
        double su = sm + (decay ? wd * fabs(w0) : 0.0);
        if (s_m) s_m[i] = sm;
        if (s_w) s_w[i] = dmax(fabs(w1), dmax(fabs(w0), rate * su));
    }
}

void orc_step(const orc_config* cfg, orc_scaler* st, float lr,
              const orc_segment* segs, int64_t nseg) {
    double inv;
    float inv32;
    orc_unscale_factor(cfg, st, &inv, &inv32);
    double sumsq = 0.0;
    int32_t overflow = 0;
    for (int64_t s = 0; s < nseg; ++s)
        orc_scan(cfg->dtype, segs[s].grad, segs[s].numel, inv, inv32, &sumsq, &overflow);
    orc_decision d;
    orc_decide(cfg, st, overflow, sumsq, &d);
    for (int64_t s = 0; s < nseg; ++s) {
        if (cfg->optimizer == ORC_SGD)
            orc_update_sgd(cfg, &d, lr, segs[s].grad, segs[s].half, segs[s].master,
                           segs[s].exp_avg, segs[s].numel, segs[s].flags & ORC_DECAY, NULL, NULL);
        else
            orc_update(cfg, &d, lr, segs[s].grad, segs[s].half, segs[s].master, segs[s].exp_avg,
                       segs[s].exp_avg_sq, segs[s].numel, segs[s].flags & ORC_DECAY,
                       NULL, NULL, NULL);
    }
}

/* ------------------------------------------------------------------------------ */
/* Shard layout                                                                    */
/* ------------------------------------------------------------------------------ */

/* Element-by-element: element e of the padded flat concat belongs to rank e / P and
 * to the tensor whose range contains it (or to the padding past the last tensor);
 * consecutive elements of one rank with the same owner form one segment.
 * [GPT-NeoX article "GPT-NeoX：如何为开源社区打开千亿级大模型训练的“民主化”之门",
 * section "技术深度解析": each device updates only
 * the shard it owns; parallelism table: DP + ZeRO uses reduce-scatter / all-gather.] */
int64_t orc_partition(const uint64_t* tensor_numel, const uint8_t* tensor_decay,
                      int64_t ntensors, int64_t dp_world_size, int64_t rank, int64_t align,
                      orc_shard_segment* out, int64_t cap, uint64_t* shard_numel) {
    uint64_t total = 0;
    for (int64_t i = 0; i < ntensors; ++i) total += tensor_numel[i];
    uint64_t unit = (uint64_t)dp_world_size * (uint64_t)align;
    uint64_t padded = (total + unit - 1) / unit * unit;
    uint64_t P = padded / (uint64_t)dp_world_size;
    *shard_numel = P;

    int64_t nseg = 0;
    int64_t cur_tensor = -2;            /* owner of the previous element of this rank */
    int64_t ti = 0;                      /* tensor containing element e               */
    uint64_t tstart = 0;                 /* first element of tensor ti                */
    for (uint64_t e = 0; e < padded; ++e) {
        while (ti < ntensors && e >= tstart + tensor_numel[ti]) {
            tstart += tensor_numel[ti];
            ++ti;
        }
        if (e / P != (uint64_t)rank) continue;
        int64_t owner = ti;              /* == ntensors in the padding */
        if (owner != cur_tensor) {
            if (nseg < cap) {
                orc_shard_segment* s = &out[nseg];
                s->shard_offset = e - (uint64_t)rank * P;
                s->numel = 0;
                s->tensor_offset = e - tstart;
                s->tensor_id = (uint32_t)owner;
                s->flags = (owner < ntensors && tensor_decay[owner]) ? ORC_DECAY : 0;
            }
            ++nseg;
            cur_tensor = owner;
        }
        if (nseg - 1 < cap) out[nseg - 1].numel += 1;
    }
    return nseg;
}
