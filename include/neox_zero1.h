/*
 * neox_zero1.h -- C ABI of the MI355X (gfx950) ZeRO-1 mixed-precision Adam step.
 *
 * One call runs the optimizer step that one data-parallel rank performs on its own
 * flat shard after the gradients have been reduced: FP32 Adam moments and FP32
 * master weights, FP16 or BF16 gradients and model copy, dynamic loss scaling that
 * skips the step on an inf/NaN gradient, a gradient pre-divide factor, clipping by
 * the global L2 norm, decoupled weight decay, and the write-back of the half copy.
 *
 * Sources (web pages on GPT-NeoX and OPT training):
 *   [NeoX] "GPT-NeoX：如何为开源社区打开千亿级大模型训练的“民主化”之门"
 *          (ainews.cool article; roughly "GPT-NeoX: how it opens the door to
 *          democratised 100B-scale training for the open-source community"),
 *          section 技术深度解析 (technical deep dive): with
 *          ZeRO stage 1 the Adam moments are split over the data-parallel GPUs and
 *          each device updates only the shard it owns; parallelism-strategy table:
 *          DP + ZeRO communicates by reduce-scatter / all-gather.
 *   [OPT]  "OPT: Open Pre-trained Transformer Language Models" (paper card),
 *          section 计算设置 (compute setup): Adam state in FP32, sharded; FP16
 *          weights; dynamic loss scaling.  Section 瓶颈 (bottlenecks): about 16
 *          bytes of model state per parameter; loss-scale collapse accompanies
 *          divergence.  Section 方法适配 (method adaptation): gradient pre-divide
 *          factor; clipping changed from 1.0 to 0.3; scaler reset / restart.
 * The pages give no formulas.  The step computes Adam with bias correction (Kingma &
 * Ba 2015), decoupled weight decay (Loshchilov & Hutter), loss scaling with skip /
 * back-off / growth (Micikevicius et al. 2018) and clipping by min(1, c / ||g||).
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are HIP device pointers (e.g. torch tensors' data_ptr()
 *     on a ROCm build); everything else is host memory.
 *   - hip_stream is a hipStream_t passed as void* (NULL = the null stream).
 *   - Return value: NEOX_OK (0) or a negative NEOX_E* code.  Nothing throws or aborts
 *     across the ABI.  Arguments are validated before any work is enqueued; on error
 *     nothing is enqueued and neox_zero1_last_error() describes the failure.
 *   - A handle may be used by one host thread at a time.
 *   - A handle belongs to the device current at neox_zero1_create(); every segment array
 *     must live on it, and later calls must pass a stream of that device (or NULL with
 *     that device current).
 */
#ifndef NEOX_ZERO1_H
#define NEOX_ZERO1_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NEOX_OK       0
#define NEOX_EINVAL  (-1)   /* bad argument: null, misaligned, zero size, out of range */
#define NEOX_EHIP    (-2)   /* a HIP runtime call failed                               */
#define NEOX_ENOMEM  (-3)   /* device or host allocation failed                        */

#define NEOX_F16  1         /* IEEE-754 binary16 gradients and model copy */
#define NEOX_BF16 2         /* bfloat16 gradients and model copy          */

#define NEOX_SCALER_DYNAMIC 0   /* back off on overflow, grow after clean runs */
#define NEOX_SCALER_STATIC  1   /* fixed scale; overflow still skips the step  */

#define NEOX_OPT_ADAMW 0         /* Adam with bias correction, decoupled decay   */
#define NEOX_OPT_SGD   1         /* heavy-ball momentum SGD, decoupled decay     */

#define NEOX_PATH_CHUNKED 0     /* update driven by the per-chunk work table    */
#define NEOX_PATH_FLAT    1     /* update addresses a flat partition's tiles    */

#define NEOX_CHUNK_DECAY 1u     /* chunk's elements receive decoupled decay     */
#define NEOX_CHUNK_VEC   2u     /* all five arrays 16-byte aligned at its start */

#define NEOX_SEG_DECAY 1u       /* segment receives decoupled weight decay      */
#define NEOX_PAD_TENSOR 0xFFFFFFFFu

/* Create-time configuration.  neox_zero1_default_config() fills the values the
 * OPT-style recipe uses (betas 0.9 / 0.95, eps 1e-8, decay 0.01, clip 1.0, f = D = 1,
 * fp16, dynamic scaler starting at 2^16, x0.5 on overflow, x2 after 1000 clean steps,
 * floor 1.0). */
typedef struct neox_zero1_config {
    double  beta1, beta2;          /* in [0, 1)                                         */
    double  eps;                   /* > 0 (also after rounding to FP32), added to
                                      sqrt(v_hat); 0 would make a zero gradient with zero
                                      moments compute 0/0                               */
    double  weight_decay;          /* >= 0, decoupled: w -= lr * wd * w (DECAY segments) */
    double  clip_norm;             /* > 0: clip to this global L2 norm; <= 0: no clip   */
    double  predivide_factor;      /* f > 0: each rank divided its gradient by f        */
    int32_t dp_world_size;         /* D >= 1: ranks whose gradients were summed         */
    int32_t dtype;                 /* NEOX_F16 or NEOX_BF16 (gradients and half copy)   */
    int32_t scaler_mode;           /* NEOX_SCALER_DYNAMIC or NEOX_SCALER_STATIC         */
    int32_t growth_interval;       /* >= 1 clean steps between growths                  */
    double  init_scale;            /* > 0, finite in FP32: scale of the first step       */
    double  growth_factor;         /* >= 1                                              */
    double  backoff_factor;        /* in (0, 1]                                         */
    double  min_scale;             /* > 0: floor of the dynamic scale                   */
    /* Resume: state of a previous run as read by neox_scaler_state(). */
    int64_t init_step;             /* applied steps so far (t), >= 0                    */
    int64_t init_skipped;          /* skipped steps so far, >= 0                        */
    int32_t init_good_steps;       /* clean steps since the last growth / overflow      */
    int32_t init_consecutive_overflows;
    /* Launch shape; 0 selects the default.  Results other than the norm's last bits
     * do not depend on either. */
    uint32_t chunk_elems;          /* elements per work chunk: multiple of 8, 256..2^24 */
    uint32_t norm_blocks;          /* norm pass grid: 0 = one block per chunk, else this
                                      many blocks striding over the chunks              */
    /* Optimizer: NEOX_OPT_ADAMW, or NEOX_OPT_SGD (m = beta1*m + g; w -= lr*(m + wd*w);
     * exp_avg holds the momentum, exp_avg_sq is unused and may be NULL).  The OPT card
     * (方法适配) reports SGD being tried in place of Adam and reverted. */
    int32_t  optimizer;
    /* 1: also keep each segment's squared gradient norm of the last step on the device
     * (neox_zero1_segment_sumsq); needs norm_blocks == 0.  Gradient-norm spikes per
     * tensor are how the OPT card (瓶颈, 方法适配) diagnoses instability. */
    uint32_t segment_norms;
    /* Update kernel.  0: when chunk_elems is 0 and the segments, in order, tile five
     * contiguous arrays whose first elements are 16-byte aligned (one flat ZeRO-1
     * partition, as neox_zero1_partition lays it out), the update computes each tile's
     * addresses from its index and loads its data without first reading a work
     * descriptor; any other layout uses the per-chunk work table.  1: always the work
     * table.  Results do not depend on the choice. */
    uint32_t chunked_update;
} neox_zero1_config;

/* One contiguous run of parameters of the shard, with its five device arrays, each
 * holding numel elements:
 *   grad        device, read-only: gradient in `dtype`, already summed over the D
 *               ranks after each rank divided by f, still multiplied by the loss scale
 *               of the step it is used in.  2-byte aligned.
 *   half        device, written on applied steps: model copy in `dtype`.  2-byte aligned.
 *   master      device FP32 master weights.           4-byte aligned.
 *   exp_avg     device FP32 first moment m.           4-byte aligned.
 *   exp_avg_sq  device FP32 second moment v.          4-byte aligned.
 * 16-byte alignment of all five (at the same element) is the fast path; any other
 * alignment is handled.  Segments must not overlap one another.  flags: NEOX_SEG_DECAY.
 * tensor_id and tensor_offset are informational (as produced by neox_zero1_partition). */
typedef struct neox_segment {
    const void* grad;
    void*       half;
    float*      master;
    float*      exp_avg;
    float*      exp_avg_sq;
    uint64_t    numel;
    uint32_t    flags;
    uint32_t    tensor_id;
    uint64_t    tensor_offset;
} neox_segment;

/* Scaler / step state after the last enqueued step. */
typedef struct neox_scaler_state_t {
    float    loss_scale;           /* scale the next step's gradient must carry          */
    int32_t  good_steps;           /* clean steps since the last growth or overflow      */
    int64_t  step;                 /* applied steps (t)                                  */
    int64_t  skipped_total;        /* skipped steps                                      */
    int32_t  consecutive_overflows;/* overflows in a row; a climbing count at the scale
                                      floor is the loss-scale collapse [OPT, 瓶颈]       */
    int32_t  last_skipped;         /* 1 if the last step was skipped                     */
    float    last_grad_norm;       /* global L2 norm of the unscaled gradient; +inf on a
                                      skipped step                                       */
    float    last_clip_coef;       /* applied clip coefficient (1 when not clipped)      */
    double   last_sumsq;           /* squared norm in double (0 on a skipped step)       */
    const float* device_loss_scale;/* device address of loss_scale, for scaling the next
                                      loss on the device without a host sync             */
} neox_scaler_state_t;

/* Segment of a rank's shard as produced by neox_zero1_partition(). */
typedef struct neox_shard_segment {
    uint64_t shard_offset;         /* first element within the rank's flat shard         */
    uint64_t numel;
    uint64_t tensor_offset;        /* first element within the tensor                    */
    uint32_t tensor_id;            /* index into the tensor list; NEOX_PAD_TENSOR for the
                                      zero padding at the end of the flat concat          */
    uint32_t flags;                /* NEOX_SEG_DECAY if the tensor decays                */
} neox_shard_segment;

typedef struct neox_zero1 neox_zero1;

/* Fill *cfg with the defaults listed above.  Host only. */
int neox_zero1_default_config(neox_zero1_config* cfg);

/* ZeRO-1 shard layout [NeoX, 技术深度解析 and its parallelism table]: the tensors
 * (host arrays tensor_numel[ntensors], tensor_decay[ntensors] with 0 / 1) are
 * concatenated in order, the total is padded with zero elements to a multiple of
 * dp_world_size * align, and rank `rank` owns elements [rank*P, (rank+1)*P) with
 * P = padded / dp_world_size.  Writes up to `cap` segments (the intersections of each
 * tensor, then the padding, with that range, in order) to the host array `out`, the
 * number of segments to *nseg_out and P to *shard_numel_out.  Call with cap = 0 to size
 * `out`.  Host only; never touches the GPU.
 * Errors: NEOX_EINVAL for null outputs, dp_world_size or align of 0, rank out of range,
 * a null input with ntensors > 0, or a 64-bit overflow of the total. */
int neox_zero1_partition(const uint64_t* tensor_numel, const uint8_t* tensor_decay,
                         uint64_t ntensors, uint32_t dp_world_size, uint32_t rank,
                         uint32_t align, neox_shard_segment* out, uint64_t cap,
                         uint64_t* nseg_out, uint64_t* shard_numel_out);

/* Create a step handle for one data-parallel rank's shard of the optimizer state: the
 * rank keeps and updates only its own piece of the FP32 master weights and Adam moments
 * [NeoX, 技术深度解析: ZeRO stage 1], which the OPT card keeps in FP32 next to FP16
 * weights [OPT, 计算设置], 16 bytes per parameter in all [OPT, 瓶颈].
 * cfg and segs[nseg] are host memory, copied
 * (the caller may free them on return).  The caller keeps ownership of every device
 * array; they must stay valid, and not be written by anyone else while a step runs,
 * until neox_zero1_destroy().  The library allocates its own device scratch (work
 * table, per-block partial sums, a state block) and uploads it on hip_stream, then
 * synchronizes that stream.  *out receives the handle.
 * Errors: NEOX_EINVAL (null pointers, nseg == 0, a zero-length or misaligned segment,
 * written arrays that overlap one another, a gradient that overlaps a written array, a
 * config field out of the ranges above), NEOX_ENOMEM, NEOX_EHIP. */
int neox_zero1_create(const neox_zero1_config* cfg, const neox_segment* segs, uint64_t nseg,
                      void* hip_stream, neox_zero1** out);

/* One optimizer step with dynamic loss scaling [OPT, 计算设置]: skip on an inf/NaN
 * gradient and back off the scale, the pre-divide factor folded into the unscale, and
 * clipping by the global L2 norm (1.0, later 0.3 in the OPT run) [OPT, 方法适配].
 * Enqueue it on hip_stream and return without waiting: a norm/overflow pass
 * over every gradient, a one-block finalize (skip decision, clip coefficient, step
 * count, bias corrections, loss-scale update, all on the device), and the fused
 * unscale + clip + AdamW + cast update, which returns before loading its data when the
 * finalize decided to skip.  When the norm pass has at most 256 blocks there is no
 * separate finalize: every update block sums the partials in the finalize's order and
 * takes the same decisions itself (same bits), and one of them writes the state.  That
 * is the case for every flat partition up to ~6.8e10 elements (a norm pass of at most
 * 64 blocks below ~2M elements, else of at most 256 large blocks cutting the whole
 * gradient; with segment_norms the chunks follow the segments, which keeps this for
 * fewer than 128 segments) and for other layouts below ~2M elements whose segments add
 * few norm chunks; neox_zero1_plan reports which.  The
 * gradient must be complete in stream order before this call.
 * On a skipped step master, exp_avg, exp_avg_sq and half are not written.
 * Errors: NEOX_EINVAL (null handle, non-finite lr), NEOX_EHIP (launch failure). */
int neox_zero1_step(neox_zero1* h, float lr, void* hip_stream);

/* The loss scaler's state: the scale, its clean-step and overflow counters (a climbing
 * overflow count at the floor is the scale collapse the OPT card describes [OPT, 瓶颈]),
 * the step count and the last step's norm and clip coefficient.
 * Wait for the stream of the last call that enqueued work on this handle and copy the
 * state to *out.  A step replayed from a captured HIP graph is not such a call: wait for
 * the replay's stream before reading the state.  Errors: NEOX_EINVAL (null), NEOX_EHIP. */
int neox_scaler_state(neox_zero1* h, neox_scaler_state_t* out);

/* End of a shard's optimizer (the caller keeps the FP32 state it owns [NeoX,
 * 技术深度解析]).  Wait for outstanding work and free the library's scratch (never caller
 * memory).
 * A graph that captured a step of this handle must not be replayed afterwards.
 * NULL is a no-op returning NEOX_OK. */
int neox_zero1_destroy(neox_zero1* h);

/* Split step for data-parallel ranks [NeoX, 技术深度解析 parallelism table: DP + ZeRO].
 * The clip coefficient and the skip decision need the squared norm over every rank's
 * gradient shard, so a rank can run its step in two halves around an exchange:
 *   neox_zero1_step_local  enqueues the norm pass and writes this rank's squared norm
 *                          of the unscaled gradient to the device double *local_sumsq
 *                          (non-finite if any of its unscaled values overflowed);
 *   (caller)               gathers the D ranks' values, in rank order, into a device
 *                          array rank_sumsq[D] on every rank (an all-gather: data
 *                          movement only);
 *   neox_zero1_step_apply  adds rank_sumsq[0 .. nranks) in a fixed order, so every rank
 *                          gets the same bits and takes the same skip and clip decisions
 *                          (a non-finite value from any rank skips the step everywhere),
 *                          and enqueues the update.  With at most 256 ranks on a handle
 *                          whose update can decide (a flat partition, or a shard whose
 *                          neox_zero1_step has no finalize launch) the update kernel adds
 *                          the values and decides itself; otherwise a one-block finalize
 *                          does it first.  The bits are the same either way.
 * The step's scaler state is the one its step_local started from (the norm pass saves
 * it): call neox_scaler_set between steps, not between a step_local and its step_apply,
 * and give every step_apply its own step_local.
 * neox_zero1_step is step_local followed by step_apply on the local value alone
 * (nranks = 1), bit for bit.  Both return without waiting.  Errors: NEOX_EINVAL (null
 * handle or pointer, pointer not 8-byte aligned, nranks 0 or above 2^24, non-finite lr),
 * NEOX_EHIP. */
int neox_zero1_step_local(neox_zero1* h, double* local_sumsq, void* hip_stream);
int neox_zero1_step_apply(neox_zero1* h, const double* rank_sumsq, uint32_t nranks, float lr,
                          void* hip_stream);

/* Overwrite the persistent scaler state in stream order: loss_scale, good_steps, step,
 * skipped_total and consecutive_overflows of *st (host) replace the device copy; the
 * last_* fields and device_loss_scale are ignored.  This is the OPT card's remedy of
 * resetting the dynamic loss scaler or restarting from a checkpoint whose scaler is
 * healthy (方法适配).  Errors: NEOX_EINVAL (null, loss_scale not finite and > 0, negative
 * counters), NEOX_EHIP. */
int neox_scaler_set(neox_zero1* h, const neox_scaler_state_t* st, void* hip_stream);

/* Per-segment telemetry (handle created with segment_norms = 1): waits for the last
 * step and writes each segment's squared norm of the unscaled gradient of that step to
 * the host array out[nseg] (nseg = the number of segments given to create), in segment
 * order; a non-finite value marks the segment that overflowed.  Errors: NEOX_EINVAL
 * (null, wrong nseg, telemetry off), NEOX_EHIP. */
int neox_zero1_segment_sumsq(neox_zero1* h, double* out, uint64_t nseg);

/* Per-kernel timing for profiling.  neox_zero1_timing_begin(h, max_steps, update_only)
 * makes the next max_steps calls of neox_zero1_step time their kernels: each of the
 * three kernels, or (update_only = 1) the update kernel only, is launched with a pair of
 * HIP events that its own dispatch stamps with its start and end (no marker packets are
 * added to the stream).  The events skip the system-scope fence at completion: they
 * give elapsed times only and order nothing.  neox_zero1_timing_end() waits, writes
 * the summed kernel durations in milliseconds of the norm pass, the finalize and the
 * update to ms_sums[3] (host; the first two are 0 with update_only, the finalize's is 0
 * when the update takes the decisions itself), the number of
 * recorded steps to *steps, and, when step_cap > 0, each of the first step_cap recorded
 * steps' duration to the host array step_ms (from the norm pass's start to the update's
 * end, launch gaps included; the update kernel alone with update_only), then stops
 * recording.  max_steps is 1 .. 1,000,000; a new begin discards an unfinished recording;
 * if an event cannot be created, nothing is recorded and later steps run untimed.
 * Errors: NEOX_EINVAL (null handle or outputs, step_cap < 0, step_ms NULL with
 * step_cap > 0), NEOX_ENOMEM, NEOX_EHIP. */
int neox_zero1_timing_begin(neox_zero1* h, int32_t max_steps, int32_t update_only);
int neox_zero1_timing_end(neox_zero1* h, double* ms_sums, int64_t* steps, double* step_ms,
                          int64_t step_cap);

/* Which update kernel the handle runs: NEOX_PATH_FLAT or NEOX_PATH_CHUNKED (see
 * chunked_update).  Errors: NEOX_EINVAL (null handle). */
int neox_zero1_update_path(const neox_zero1* h);

/* The work decomposition neox_zero1_create() builds for a segment list — the segment /
 * chunk bookkeeping of the multi-tensor step [NeoX, 技术深度解析: each rank updates the
 * shard it owns, held as a list of tensor pieces] — computed on the host with the same
 * validation and no device call, for inspection and tests.  Chunks never straddle a
 * segment: a segment whose five arrays become 16-byte aligned after h < 8 elements
 * starts with an h-element chunk without NEOX_CHUNK_VEC, then takes chunks of
 * chunk_elems (the last one shorter), all with NEOX_CHUNK_VEC; a segment whose arrays
 * can never be aligned together gets chunks without it.  Chunks are listed in segment
 * order.  On the flat path tile_words[flat_tiles + 1] and changes[flat_changes] hold the
 * tile table: word T = (index in changes of tile T's first decay-flag change) << 1 |
 * decay flag of the tile's first element; changes holds in-tile offsets where the flag
 * flips; word flat_tiles closes the last list. */
typedef struct neox_chunk_info {
    uint64_t offset;               /* first element of the chunk within its segment      */
    uint32_t seg;                  /* index in segs                                      */
    uint32_t len;                  /* elements, 1 .. chunk_elems                         */
    uint32_t flags;                /* NEOX_CHUNK_DECAY | NEOX_CHUNK_VEC                  */
    uint32_t reserved;             /* 0                                                  */
} neox_chunk_info;

typedef struct neox_zero1_plan_t {
    uint64_t numel;                /* elements over all segments                        */
    uint64_t update_chunks;        /* entries of the update chunk table                 */
    uint64_t norm_chunks;          /* entries of the norm pass's table (on a flat       */
                                   /*    partition without segment_norms they cut the  */
                                   /*    whole gradient, across segment bounds)         */
    uint64_t flat_tiles;           /* tiles of the flat update; 0 on the chunked path   */
    uint64_t flat_changes;         /* in-tile decay-flag changes (flat path)            */
    uint32_t chunk_elems;          /* update chunk length                               */
    uint32_t norm_chunk_elems;     /* norm chunk length                                 */
    uint32_t tile_elems;           /* flat tile length                                  */
    int32_t  update_path;          /* NEOX_PATH_FLAT or NEOX_PATH_CHUNKED               */
    uint32_t norm_block_threads;   /* threads per block of the norm pass                */
    uint32_t update_decides;       /* 1: the update takes the step's decisions itself  */
                                   /*    from the norm pass's partials (no finalize    */
                                   /*    launch); 0: a one-block finalize decides       */
} neox_zero1_plan_t;

/* Fills *out (host) and the first min(cap, size) entries of each host table; a table
 * may be NULL with capacity 0.  The segments' pointers are only compared, never
 * dereferenced.  Errors: as neox_zero1_create's validation (NEOX_EINVAL), NEOX_EINVAL
 * for a NULL out or a NULL table with nonzero capacity, NEOX_ENOMEM. */
int neox_zero1_plan(const neox_zero1_config* cfg, const neox_segment* segs, uint64_t nseg,
                    neox_zero1_plan_t* out, neox_chunk_info* chunks, uint64_t chunk_cap,
                    uint32_t* tile_words, uint64_t word_cap, uint32_t* changes,
                    uint64_t change_cap);

/* For callers that cannot allocate device memory (tight serving loops, harnesses that
 * forbid hipMalloc; the call synchronizes its stream, so it is not one to record inside
 * a HIP graph capture): one whole step -- the same kernels and
 * launch shapes as neox_zero1_step, so the same bits for the same inputs -- with no
 * handle and no device allocation.  cfg and segs[nseg] are as for neox_zero1_create
 * (host memory; segment_norms must be 0).  *state (host) is read for the scaler state
 * before the step (loss_scale, good_steps, step, skipped_total, consecutive_overflows;
 * the other fields are ignored) and overwritten with the state after it, as
 * neox_scaler_state reports it (device_loss_scale = NULL).  The call waits for hip_stream
 * before it returns.
 * The library's side of the step (state block, per-block partial sums, work tables) lives
 * in a fixed device array of NEOX_NOALLOC_SCRATCH_BYTES that each device holds for the
 * life of the process: about 2 bytes per 1,000 elements on a flat partition (its tile
 * table; up to ~8.5e9 elements) and 33 per 1,000 on other layouts (up to ~5e8).  A
 * larger shard is
 * rejected with NEOX_EINVAL.  Every call on one device uses the same array: calls on one
 * device from several host threads are serialized by the library; calls from several
 * processes each have their own array.
 * Errors: NEOX_EINVAL (as neox_zero1_create, plus null state, bad state values,
 * non-finite lr, segment_norms, a shard beyond the scratch size), NEOX_ENOMEM (host),
 * NEOX_EHIP. */
#define NEOX_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
int neox_zero1_step_noalloc(const neox_zero1_config* cfg, const neox_segment* segs, uint64_t nseg,
                            neox_scaler_state_t* state, float lr, void* hip_stream);

/* Text of the last error raised on the calling thread (never NULL). */
const char* neox_zero1_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
