/*
 * oracle.h -- plain CPU reference of the ZeRO-1 mixed-precision Adam step on one
 * data-parallel shard.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path includes, links
 * or calls this code; only the test-suite, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no source with the GPU path.
 *
 * What it computes, and which passage of the pages it follows:
 *   - Each data-parallel rank updates only its own shard of the Adam state; the
 *     optimizer memory is divided by the DP degree.
 *       [GPT-NeoX article "GPT-NeoX：如何为开源社区打开千亿级大模型训练的“民主化”之门"
 *        (ainews.cool), section "技术深度解析" (technical deep dive),
 *        ZeRO stage-1 paragraph and the parallelism-strategy table]
 *   - Adam state kept in FP32, model weights kept in FP16, dynamic loss scaling.
 *       [OPT: Open Pre-trained Transformer Language Models (paper card),
 *        section "计算设置" (compute setup)]
 *   - 16 bytes of model state per parameter for mixed-precision Adam (2 B half weight,
 *     2 B half gradient, 4 B FP32 master, 4 B + 4 B FP32 moments).
 *       [OPT paper card, section "瓶颈" (bottlenecks), memory-arithmetic paragraph]
 *   - A gradient pre-divide factor, and gradient clipping at 1.0 then 0.3; a
 *     loss-scale collapse counts as a divergence symptom.
 *       [OPT paper card, sections "瓶颈" and "方法适配" (method adaptation)]
 *   The pages give no formula for Adam, the scaler or the clip.  The oracle takes the
 *   plainest published readings: Adam with bias correction (Kingma & Ba, 2015),
 *   decoupled weight decay (Loshchilov & Hutter, AdamW), loss scaling with
 *   skip / back-off / growth (Micikevicius et al., "Mixed Precision Training", 2018),
 *   and clipping by the global L2 norm.
 *
 * Precision.  The pages fix the storage types (FP32 state, FP16 or BF16 half copy and
 * gradients).  Every per-element quantity is evaluated here in double from the stored
 * inputs and rounded ONCE to its storage type, so the oracle's outputs are the exact
 * result of one step up to that final rounding.  Two decisions are integer-valued and
 * are taken in the storage precision the method uses, FP32: the loss-scale update and
 * the overflow test on the unscaled FP32 gradient.
 *
 * Parity pins: every function is pinned by tests under tests/ (closed forms,
 * invariants, brute force, library routines).  The last-ulp choice among valid FP32
 * evaluations of m, v and master is only bounded by the tolerance, not pinned.
 */
#ifndef NEOX_ORACLE_H
#define NEOX_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F16 = 1, ORC_BF16 = 2 };
enum { ORC_ADAMW = 0, ORC_SGD = 1 };
enum { ORC_DYNAMIC = 0, ORC_STATIC = 1 };
enum { ORC_DECAY = 1 };

typedef struct {
    double beta1, beta2, eps, weight_decay;
    double clip_norm;          /* <= 0 disables clipping                              */
    double predivide_factor;   /* f: each rank divided its gradient by f before the sum */
    int32_t dp_world_size;     /* D: number of ranks whose gradients were summed        */
    int32_t dtype;             /* ORC_F16 / ORC_BF16: gradient and half-copy format     */
    int32_t scaler_mode;       /* ORC_DYNAMIC / ORC_STATIC                              */
    int32_t growth_interval;   /* clean steps between growths (dynamic mode)            */
    double growth_factor, backoff_factor, min_scale;
    int32_t optimizer;         /* ORC_ADAMW, or ORC_SGD (momentum beta1, decoupled decay) */
    int32_t pad_;
} orc_config;

typedef struct {
    float   loss_scale;        /* S, stored in FP32                                     */
    int32_t last_skipped;
    int64_t good_steps;
    int64_t step;              /* t: applied steps only                                 */
    int64_t skipped_total;
    int64_t consecutive_overflows;
    double  last_sumsq;        /* sum of squares of the unscaled gradient (0 on a skip) */
    double  last_norm;         /* +inf on a skipped step                                */
    double  last_coef;         /* 1 on a skipped step                                   */
} orc_scaler;

/* What the finalize decides for one step; consumed by orc_update. */
typedef struct {
    int32_t skip;
    double  inv;               /* f / (D * S) with S the pre-step scale, in double      */
    float   inv32;             /* the same rounded once to FP32 (overflow test)         */
    double  coef;              /* clip coefficient                                      */
    double  bc1, bc2;          /* 1 - beta^t                                            */
    int64_t t;                 /* step number of this update (after the increment)      */
} orc_decision;

typedef struct {
    const uint16_t* grad;      /* half-precision gradient bits                          */
    uint16_t* half;            /* half-precision model copy bits                        */
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    int64_t numel;
    int32_t flags;             /* ORC_DECAY */
    int32_t pad_;
} orc_segment;

typedef struct {
    uint64_t shard_offset;
    uint64_t numel;
    uint64_t tensor_offset;
    uint32_t tensor_id;        /* ntensors for the trailing zero padding               */
    uint32_t flags;            /* ORC_DECAY                                              */
} orc_shard_segment;

/* ---- number formats (IEEE-754 binary16 and bfloat16, round to nearest even) ---- */
double   orc_half_to_double(int32_t dtype, uint16_t bits);
uint16_t orc_float_to_half(int32_t dtype, float x);
void     orc_float_to_half_array(int32_t dtype, const float* x, uint16_t* out, int64_t n);
void     orc_half_to_double_array(int32_t dtype, const uint16_t* bits, double* out, int64_t n);

/* ---- the step, in three parts that compose to orc_step ---- */
/* Scan: adds sum_i (x_i * inv)^2 in double (index order) into *sumsq and ORs into
 * *overflow whether any FP32 unscaled value fp32(float(x_i) * inv32) is non-finite. */
void orc_scan(int32_t dtype, const uint16_t* grad, int64_t n, double inv, float inv32,
              double* sumsq, int32_t* overflow);
/* The unscale factor for the state's current scale. */
void orc_unscale_factor(const orc_config* cfg, const orc_scaler* st, double* inv, float* inv32);
/* Finalize: skip decision, clip coefficient, step count, bias corrections and the
 * scaler update.  Updates *st and fills *d. */
void orc_decide(const orc_config* cfg, orc_scaler* st, int32_t overflow, double sumsq,
                orc_decision* d);
/* Elementwise AdamW update of n elements under decision d (no-op when d->skip).
 * s_m, s_v, s_w (optional, may be NULL) receive the magnitude of the largest term
 * that entered each output, the scale of its rounding error. */
void orc_update(const orc_config* cfg, const orc_decision* d, float lr,
                const uint16_t* grad, uint16_t* half, float* master, float* exp_avg,
                float* exp_avg_sq, int64_t n, int32_t decay,
                double* s_m, double* s_v, double* s_w);
/* SGD with heavy-ball momentum on one run of elements (the optimizer the OPT card
 * reports trying instead of Adam): m = beta1*m + g, w -= lr*(m + wd*w) for decaying
 * elements.  exp_avg holds the momentum.  s_m, s_w as for orc_update. */
void orc_update_sgd(const orc_config* cfg, const orc_decision* d, float lr,
                    const uint16_t* grad, uint16_t* half, float* master, float* exp_avg,
                    int64_t n, int32_t decay, double* s_m, double* s_w);
/* One whole step over the segment list. */
void orc_step(const orc_config* cfg, orc_scaler* st, float lr,
              const orc_segment* segs, int64_t nseg);

/* ---- shard layout: element-by-element assignment of the flat concat ---- */
/* Tensors are concatenated in order, the total padded with zero elements to a multiple
 * of dp_world_size * align, and rank r owns elements [r*P, (r+1)*P).  Returns the
 * number of segments (runs of one tensor) of rank r, writes up to cap of them, and
 * the shard length P into *shard_numel.  Walks every element: slow by design. */
int64_t orc_partition(const uint64_t* tensor_numel, const uint8_t* tensor_decay,
                      int64_t ntensors, int64_t dp_world_size, int64_t rank, int64_t align,
                      orc_shard_segment* out, int64_t cap, uint64_t* shard_numel);

#ifdef __cplusplus
}
#endif
#endif
