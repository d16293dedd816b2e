// zero1_kernels.hip -- gfx950 kernels of the ZeRO-1 mixed-precision Adam step.
//
// Two or three launches per step, all on the caller's stream:
//   norm      one block per chunk (or a smaller grid striding over the chunks);
//             each block sums the squares of its unscaled FP32 gradient in double and
//             writes one partial.  A non-finite unscaled value makes its square, and so
//             the sum, non-finite; finite values cannot overflow a double sum (|g| <
//             2^128 so g^2 < 2^256), so "sum not finite" is exactly "some gradient
//             overflowed".
//   finalize  one block; fixed-order sum of the per-block partials, then the skip
//             decision, clip coefficient, step count, bias corrections and the loss
//             scale update, written to the device state block.  Not launched when the
//             norm pass has at most kFuseMaxParts blocks: then every update block sums
//             the partials in the finalize's order and decides itself (fused_decide).
//   update    unscale + clip + AdamW + cast with 16-byte loads and stores, nothing
//             written on a skipped step: flat_update_kernel (one block per 2,048-element
//             tile of a flat partition, addresses from the block index) or update_kernel
//             (one block per entry of the chunk table, any layout).
// Sources: FP32 Adam state with FP16 weights and dynamic loss scaling [OPT: Open
// Pre-trained Transformer Language Models, paper card, 计算设置]; pre-divide factor
// and clipping at 1.0 / 0.3 [same card, 方法适配]; each rank updates only its shard
// [GPT-NeoX article "GPT-NeoX：如何为开源社区打开千亿级大模型训练的“民主化”之门",
// 技术深度解析].  Formulas: Adam with bias
// correction (Kingma & Ba), decoupled decay (Loshchilov & Hutter), loss scaling
// (Micikevicius et al. 2018).
#include "zero1_internal.h"

#include <hip/hip_ext.h>

namespace nz1 {

// ------------------------------------------------------------------------------------
// Half formats.  Decoding is exact; encoding rounds to nearest even in hardware
// (v_cvt_f16_f32 under the default rounding mode, v_cvt_pk_bf16_f32 on gfx950).
// ------------------------------------------------------------------------------------
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The half copy must be the stored FP32 master rounded to the half format.  Left alone,
// the backend folds "FMA then convert" into one mixed-precision FMA that rounds the
// exact result straight to FP16 (one rounding instead of two), which differs in rare
// ties.  An empty register-only asm makes the FP32 value opaque, so the conversion
// starts from the rounded FP32 number.  (No memory access is involved.)
__device__ __forceinline__ float materialized(float x) {
    asm("" : "+v"(x));
    return x;
}

template <int DT>
struct Fmt;

template <>
struct Fmt<1> {
    static __device__ __forceinline__ float lo(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
    }
    static __device__ __forceinline__ float hi(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
    static __device__ __forceinline__ float one(uint16_t b) {
        return (float)__builtin_bit_cast(_Float16, b);
    }
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        f16x2 p = {(_Float16)materialized(a), (_Float16)materialized(b)};
        return __builtin_bit_cast(uint32_t, p);
    }
    static __device__ __forceinline__ uint16_t enc(float a) {
        return __builtin_bit_cast(uint16_t, (_Float16)materialized(a));
    }
};

template <>
struct Fmt<2> {
    static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
    static __device__ __forceinline__ float one(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        bf16x2 p = {(__bf16)materialized(a), (__bf16)materialized(b)};
        return __builtin_bit_cast(uint32_t, p);
    }
    static __device__ __forceinline__ uint16_t enc(float a) {
        return __builtin_bit_cast(uint16_t, (__bf16)materialized(a));
    }
};

// ------------------------------------------------------------------------------------
// 16-byte global accesses, optionally non-temporal (streamed data is touched once).
// Compile-time tuning knobs; the defaults are the measured best on MI355X.
// ------------------------------------------------------------------------------------
#ifndef NZ1_NORM_UNROLL
#define NZ1_NORM_UNROLL 8
#endif
constexpr int kNormUnroll = NZ1_NORM_UNROLL;   // 16-byte loads in flight per norm thread
// The update reads the gradient with non-temporal loads (it is read once and not written)
// and the FP32 state, which it writes back in place, with ordinary ones.  Measured on
// MI355X, same arrays, alternating builds, median us per update, ordinary / non-temporal
// gradient loads: 215M shard 992-1017 / 985-994 (momentum SGD 704-722 / 695-700, chunk
// table 1070-1077 / 1060-1063), a Pythia-410M rank 214 / 208-209, the 5,000-tensor
// layout 5059-5077 / 5012-5021, the 6e9 shard 29.05-29.07 / 28.06-28.08 ms;
// non-temporal loads of the state too: 215M 1182-1188.
#ifndef NZ1_UPDATE_NT_GRAD
#define NZ1_UPDATE_NT_GRAD 1
#endif
#ifndef NZ1_UPDATE_NT_STATE
#define NZ1_UPDATE_NT_STATE 0
#endif
// Non-temporal stores of the update's results: measured 1-2% faster at the update's low
// occupancy (they were neutral at full occupancy).
#ifndef NZ1_UPDATE_NT_STORE
#define NZ1_UPDATE_NT_STORE 1
#endif
// Chunked update: each block touches the descriptor of the block this many places later
// (0 = off), so that block's first load hits the cache instead of HBM.
#ifndef NZ1_DESC_AHEAD
#define NZ1_DESC_AHEAD 512
#endif
// Chunked update: threads per block (with NZ1_UPDATE_CHUNK = 2048 and two vectors per
// thread, one pass per chunk).
#ifndef NZ1_UPDATE_BLOCK
#define NZ1_UPDATE_BLOCK 128
#endif
constexpr int kUpdateBlock = NZ1_UPDATE_BLOCK;   // threads per block of the chunked update
#ifndef NZ1_UPDATE_UNROLL
#define NZ1_UPDATE_UNROLL 2
#endif
#ifndef NZ1_UPDATE_REVERSE
#define NZ1_UPDATE_REVERSE 1
#endif
// 1: the flat update issues its tile's loads before it knows the finalize's decision (a
// skipped step then reads the tile and drops it).  0: it waits for the decision first.
// At 2 blocks per CU the other block hides that wait and the two measure the same, so
// the default keeps skipped steps cheap.
#ifndef NZ1_FLAT_SPECULATE
#define NZ1_FLAT_SPECULATE 0
#endif
#ifndef NZ1_UPDATE_FAST_DIV
#define NZ1_UPDATE_FAST_DIV 0
#endif
// Pause of a deciding AdamW flat-update block after its loads, in units of 64 clocks
// (s_sleep); 0 = none.  See flat_update_kernel.
#ifndef NZ1_FLAT_PAUSE
#define NZ1_FLAT_PAUSE 8
#endif

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// The arrays are device (global) memory; the pointers come out of the work table, so
// the compiler cannot prove it and would emit generic flat accesses.  Accessing them
// through address-space-1 pointers gives global_load / global_store.
typedef __attribute__((address_space(1))) u32x4 g_u32x4;
typedef __attribute__((address_space(1))) f32x4 g_f32x4;

template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint4* p) {
    const g_u32x4* q = (const g_u32x4*)p;
    u32x4 r;
    if constexpr (NT) r = __builtin_nontemporal_load(q);
    else r = *q;
    return make_uint4(r.x, r.y, r.z, r.w);
}
template <bool NT>
__device__ __forceinline__ float4 ld16(const float4* p) {
    const g_f32x4* q = (const g_f32x4*)p;
    f32x4 r;
    if constexpr (NT) r = __builtin_nontemporal_load(q);
    else r = *q;
    return make_float4(r.x, r.y, r.z, r.w);
}
template <bool NT>
__device__ __forceinline__ void st16(uint4* p, uint4 v) {
    g_u32x4* q = (g_u32x4*)p;
    const u32x4 r = {v.x, v.y, v.z, v.w};
    if constexpr (NT) __builtin_nontemporal_store(r, q);
    else *q = r;
}
template <bool NT>
__device__ __forceinline__ void st16(float4* p, float4 v) {
    g_f32x4* q = (g_f32x4*)p;
    const f32x4 r = {v.x, v.y, v.z, v.w};
    if constexpr (NT) __builtin_nontemporal_store(r, q);
    else *q = r;
}

// ------------------------------------------------------------------------------------
// Deterministic block reduction of a double: xor-butterfly inside each wave64 (every
// lane ends with the same, order-fixed value), then wave 0..3 partials in index order.
// ------------------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ double block_sum(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    __shared__ double ws[NT / 64];
    if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = ws[0];
#pragma unroll
    for (int k = 1; k < NT / 64; ++k) r += ws[k];
    return r;
}

// ------------------------------------------------------------------------------------
// norm: sum over the shard of fp64(fp32(x * inv))^2
// ------------------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ void sq8(const uint4 q, float inv, double& a0, double& a1) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const double x = (double)(Fmt<DT>::lo(w[k]) * inv);
        const double y = (double)(Fmt<DT>::hi(w[k]) * inv);
        a0 = __builtin_fma(x, x, a0);
        a1 = __builtin_fma(y, y, a1);
    }
}

// This block's sum of squares over its chunks (every thread gets the value); NB threads
// per block.  NTL:
// non-temporal loads (the gradient is not kept in the caches for the update's re-read).
template <int DT, bool NTL, int NB>
__device__ __forceinline__ double norm_block(const Chunk* __restrict__ chunks, uint32_t nchunks,
                                             float inv) {
    double a0 = 0.0, a1 = 0.0;
    for (uint32_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const Chunk* ch = chunks + c;
        const uint16_t* __restrict__ g = ch->grad;
        const uint32_t len = ch->len;
        uint32_t done = 0;
        if (ch->flags & CH_VEC) {
            const uint4* __restrict__ g4 = reinterpret_cast<const uint4*>(g);
            const uint32_t nvec = len / kVec;
            uint32_t i = threadIdx.x;
            // kNormUnroll loads in flight per thread, then their sums in order
            for (; i + (kNormUnroll - 1) * NB < nvec; i += kNormUnroll * NB) {
                uint4 q[kNormUnroll];
#pragma unroll
                for (int u = 0; u < kNormUnroll; ++u) q[u] = ld16<NTL>(g4 + i + u * NB);
#pragma unroll
                for (int u = 0; u < kNormUnroll; ++u) sq8<DT>(q[u], inv, a0, a1);
            }
            for (; i < nvec; i += NB) sq8<DT>(ld16<NTL>(g4 + i), inv, a0, a1);
            done = nvec * kVec;
        }
        for (uint32_t i = done + threadIdx.x; i < len; i += NB) {
            const double x = (double)(Fmt<DT>::one(g[i]) * inv);
            a0 = __builtin_fma(x, x, a0);
        }
    }
    return block_sum<NB>(a0 + a1);
}

// snap (optional): block 0 copies the scaler state the step starts from, for an update
// that takes the step's decisions itself (see fused_decide).
template <int DT, bool NTL, int NB>
__global__ __launch_bounds__(NB) void norm_kernel(const Chunk* __restrict__ chunks,
                                                      uint32_t nchunks,
                                                      const DevState* __restrict__ st,
                                                      double* __restrict__ partial,
                                                      DevState* __restrict__ snap) {
    if (snap && blockIdx.x == 0 && threadIdx.x == 0) {
        snap->loss_scale = st->loss_scale;
        snap->inv = st->inv;
        snap->good_steps = st->good_steps;
        snap->consecutive_overflows = st->consecutive_overflows;
        snap->step = st->step;
        snap->skipped_total = st->skipped_total;
    }
    const double s = norm_block<DT, NTL, NB>(chunks, nchunks, st->inv);
    if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

// ------------------------------------------------------------------------------------
// finalize: one block
// ------------------------------------------------------------------------------------
__device__ __forceinline__ bool f64_finite(double x) {
    return (__double_as_longlong(x) & 0x7FF0000000000000ll) != 0x7FF0000000000000ll;
}
__device__ __forceinline__ bool f32_finite(float x) {
    return (__float_as_uint(x) & 0x7F800000u) != 0x7F800000u;
}

// Block size of every fixed-order sum of the partials (the finalize and the split step's
// reduce), so both add in the same order.
constexpr int kFinalizeBlock = kBlock;

// Fixed-order sum of the norm pass's partials by one block of kFinalizeBlock threads:
// thread t owns partials t, t + kFinalizeBlock, ... in that order; eight independent
// loads per round keep the one-block read latency-tolerant.
__device__ __forceinline__ double sum_partials(const double* __restrict__ partial, uint32_t nparts) {
    constexpr int R = 8;
    double acc = 0.0;
    uint32_t i = threadIdx.x;
    for (; i + (R - 1) * kFinalizeBlock < nparts; i += R * kFinalizeBlock) {
        double p[R];
#pragma unroll
        for (int r = 0; r < R; ++r) p[r] = partial[i + r * kFinalizeBlock];
#pragma unroll
        for (int r = 0; r < R; ++r) acc += p[r];
    }
    for (; i < nparts; i += kFinalizeBlock) acc += partial[i];
    return block_sum<kFinalizeBlock>(acc);
}

// This rank's squared norm, for a caller that sums it over the data-parallel ranks.
__global__ __launch_bounds__(kFinalizeBlock) void reduce_kernel(const double* __restrict__ partial,
                                                                uint32_t nparts,
                                                                double* __restrict__ out) {
    const double s = sum_partials(partial, nparts);
    if (threadIdx.x == 0) *out = s;
}

// Squared norm of each segment: the norm chunks of segment k are the contiguous range
// [range[2k], range[2k+1]) of the norm table, one partial each.
__global__ __launch_bounds__(kBlock) void segment_sumsq_kernel(const double* __restrict__ partial,
                                                               const uint32_t* __restrict__ range,
                                                               double* __restrict__ out) {
    const uint32_t lo = range[2 * blockIdx.x], hi = range[2 * blockIdx.x + 1];
    double acc = 0.0;
    for (uint32_t i = lo + threadIdx.x; i < hi; i += kBlock) acc += partial[i];
    const double s = block_sum<kBlock>(acc);
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

// Stream-ordered overwrite of the persistent scaler state.
__global__ void set_state_kernel(DevState* __restrict__ st, float scale, int32_t good_steps,
                                 int64_t step, int64_t skipped, int32_t consecutive,
                                 double predivide, double dp) {
    if (threadIdx.x != 0) return;
    st->loss_scale = scale;
    st->good_steps = good_steps;
    st->step = step;
    st->skipped_total = skipped;
    st->consecutive_overflows = consecutive;
    st->inv = unscale_factor(predivide, dp, scale);
}

// b^t for an integer t >= 1 by binary exponentiation: at most ~2 log2(t) roundings
// (a few ulps), and a short dependent chain for the one thread that runs it.
__device__ __forceinline__ double ipow(double b, int64_t t) {
    double r = 1.0;
    while (t) {
        if (t & 1) r *= b;
        b *= b;
        t >>= 1;
    }
    return r;
}

// The scaler state a step starts from.
struct PreState {
    float scale;
    float inv;                   // unscale factor the norm pass used
    int32_t good;
    int32_t consecutive;
    int64_t step;
    int64_t skipped;
};
__device__ __forceinline__ PreState read_pre(const DevState* __restrict__ st) {
    return PreState{st->loss_scale, st->inv, st->good_steps, st->consecutive_overflows,
                    st->step, st->skipped_total};
}

// The step's decisions from its squared norm: skip, clip coefficient, step count, bias
// corrections and the loss-scale state machine.  A pure function of its inputs, so every
// thread that evaluates it gets the same bits.
struct Decision {
    DevState next;               // the state block after the step
};
__device__ __forceinline__ Decision decide(double sumsq, const PreState& p, const FinalizeArgs& a) {
    Decision d;
    DevState& n = d.next;
    float scale = p.scale;
    if (!f64_finite(sumsq)) {
        // overflow: skip, back off (not below the floor), restart the clean count
        n.skip = 1;
        n.gscale = 0.0f;
        n.rbc1 = 0.0f;
        n.rsbc2 = 0.0f;
        if (a.dynamic) {
            float s = (float)((double)scale * a.backoff_factor);
            scale = s < a.min_scale ? a.min_scale : s;
        }
        n.good_steps = 0;
        n.consecutive_overflows = p.consecutive + 1;
        n.skipped_total = p.skipped + 1;
        n.step = p.step;
        n.last_skipped = 1;
        n.last_sumsq = 0.0;
        n.last_grad_norm = __builtin_inff();
        n.last_clip_coef = 1.0f;
    } else {
        const double norm = __builtin_sqrt(sumsq);
        double coef = 1.0;
        if (a.clip_norm > 0.0 && norm > a.clip_norm) coef = a.clip_norm / norm;
        const int64_t t = p.step + 1;
        const double bc1 = 1.0 - ipow(a.beta1, t);
        const double bc2 = 1.0 - ipow(a.beta2, t);
        n.skip = 0;
        n.gscale = (float)((double)p.inv * coef);
        n.rbc1 = (float)(1.0 / bc1);
        n.rsbc2 = (float)(1.0 / __builtin_sqrt(bc2));
        n.step = t;
        int32_t good = p.good + 1;
        if (a.dynamic && good >= a.growth_interval) {
            const float s = (float)((double)scale * a.growth_factor);
            if (f32_finite(s)) scale = s;
            good = 0;
        }
        n.good_steps = good;
        n.consecutive_overflows = 0;
        n.skipped_total = p.skipped;
        n.last_skipped = 0;
        n.last_sumsq = sumsq;
        n.last_grad_norm = (float)norm;
        n.last_clip_coef = (float)coef;
    }
    n.loss_scale = scale;
    n.inv = unscale_factor(a.predivide_factor, a.dp_world_size, scale);
    n.pad_[0] = n.pad_[1] = n.pad_[2] = 0;
    return d;
}

__device__ __forceinline__ void write_state(DevState* __restrict__ st, const DevState& n) {
    st->loss_scale = n.loss_scale;
    st->good_steps = n.good_steps;
    st->step = n.step;
    st->skipped_total = n.skipped_total;
    st->consecutive_overflows = n.consecutive_overflows;
    st->last_skipped = n.last_skipped;
    st->last_sumsq = n.last_sumsq;
    st->last_grad_norm = n.last_grad_norm;
    st->last_clip_coef = n.last_clip_coef;
    st->inv = n.inv;
    st->skip = n.skip;
    st->gscale = n.gscale;
    st->rbc1 = n.rbc1;
    st->rsbc2 = n.rsbc2;
}

// The squared norm is the fixed-order sum of nparts values: this handle's per-block
// partials, or the data-parallel ranks' squared norms (the same order on every rank).
__global__ __launch_bounds__(kFinalizeBlock) void finalize_kernel(const double* __restrict__ partial,
                                                                  uint32_t nparts,
                                                                  DevState* __restrict__ st,
                                                                  FinalizeArgs a) {
    const double sumsq = sum_partials(partial, nparts);
    if (threadIdx.x == 0) write_state(st, decide(sumsq, read_pre(st), a).next);
}

// For a norm pass of at most kFuseMaxParts blocks the update takes the step's decisions
// itself and the finalize launch is not made.  Every wave of every update block sums the
// partials exactly as sum_partials does with kFinalizeBlock threads: thread t < nparts
// holds 0 + partial[t], the others 0; each wave of the finalize adds its 64 values by the
// xor-butterfly, and the wave sums are added in wave order.  One wave here walks the
// finalize's waves in turn with the same butterfly, so the squared norm and every
// decision have the bits the finalize kernel would give.  The pre-step state comes from
// the norm pass's snapshot, and block 0 writes the state block.
static_assert(kFuseMaxParts == kFinalizeBlock && kFinalizeBlock % 64 == 0,
              "a fused update covers the finalize's whole first pass");
struct Fuse {
    const double* partial;       // null: the finalize kernel ran, read the state block
    uint32_t nparts;
    const DevState* snap;
    DevState* st;                // written by block 0
    FinalizeArgs fin;
};
// The loads of fused_decide, so that a caller can issue them ahead of its data loads and
// let the decision's arithmetic overlap the data's latency.
struct FusedIn {
    double p[kFinalizeBlock / 64];   // this lane's partial of each finalize wave (0 if none)
    PreState pre;
};
__device__ __forceinline__ FusedIn fused_load(const Fuse& f) {
    const uint32_t lane = threadIdx.x & 63;
    FusedIn in;
    // unconditional loads (a lane past the partials reads partial[0], which fused_finish
    // ignores), so they issue back to back without a wait between them
#pragma unroll
    for (int w = 0; w < kFinalizeBlock / 64; ++w) {
        const uint32_t i = w * 64 + lane;
        in.p[w] = f.partial[i < f.nparts ? i : 0];
    }
    in.pre = read_pre(f.snap);
    return in;
}
// Issued after a block's data loads: the decision's arithmetic cannot be scheduled above
// this point (it depends on the values passed through), and the data loads cannot sink
// below it, so the arithmetic overlaps the data's latency.  Register operands only.
__device__ __forceinline__ void after_data(FusedIn& in) {
    static_assert(kFinalizeBlock / 64 == 4, "four partial registers");
    asm volatile("" : "+v"(in.p[0]), "+v"(in.p[1]), "+v"(in.p[2]), "+v"(in.p[3]) : : "memory");
}
__device__ __forceinline__ Decision fused_finish(const FusedIn& in, const Fuse& f) {
    const uint32_t lane = threadIdx.x & 63;
    // finalize waves holding partials; the others sum to +0, which is added as such
    const uint32_t waves = (f.nparts + 63) / 64;
    double r = 0.0;
#pragma unroll
    for (uint32_t w = 0; w < kFinalizeBlock / 64; ++w) {
        double v = 0.0;
        if (w < waves) {
            if (w * 64 + lane < f.nparts) v = 0.0 + in.p[w];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
        }
        r = w == 0 ? v : r + v;
    }
    return decide(r, in.pre, f.fin);
}
__device__ __forceinline__ Decision fused_decide(const Fuse& f) {
    return fused_finish(fused_load(f), f);
}

// ------------------------------------------------------------------------------------
// update: fused unscale + clip + AdamW + cast, one block per chunk or flat tile
// ------------------------------------------------------------------------------------
struct Coefs {
    float gs, rbc1, rsbc2;
};

// heavy-ball momentum SGD with decoupled decay: m = beta1*m + g; w -= lr*(m + wd*w)
__device__ __forceinline__ void sgd(float h, float& w, float& m, const Coefs& c,
                                    const UpdateArgs& a, bool decay) {
    const float g = h * c.gs;
    m = __builtin_fmaf(a.b1, m, g);
    float u = m;
    if (decay) u = __builtin_fmaf(a.wd, w, u);
    w = __builtin_fmaf(-a.lr, u, w);
}

// Square root and reciprocal with the hardware's ~1-ulp instructions.  v_sqrt_f32 is
// given a normal input: a subnormal v is scaled by 2^64 first and the root by 2^-32
// (exact powers of two).  The reciprocal's input sqrt(v)/sqrt(bc2) + eps is never
// subnormal (sqrt of the smallest FP32 subnormal is ~3.7e-23), so v_rcp_f32 sees
// normal numbers, zero or infinity.
__device__ __forceinline__ float sqrt_hw(float v) {
    const bool tiny = v < 0x1p-126f;
    const float r = __builtin_amdgcn_sqrtf(tiny ? v * 0x1p64f : v);
    return tiny ? r * 0x1p-32f : r;
}

__device__ __forceinline__ void adam(float h, float& w, float& m, float& v, const Coefs& c,
                                     const UpdateArgs& a, bool decay) {
    const float g = h * c.gs;
    m = __builtin_fmaf(a.b1, m, a.omb1 * g);
    v = __builtin_fmaf(a.b2, v, a.omb2 * (g * g));
#if NZ1_UPDATE_FAST_DIV
    const float den = __builtin_fmaf(sqrt_hw(v), c.rsbc2, a.eps);
    float u = (m * c.rbc1) * __builtin_amdgcn_rcpf(den);
#else
    const float den = __builtin_fmaf(__builtin_sqrtf(v), c.rsbc2, a.eps);
    float u = (m * c.rbc1) / den;
#endif
    if (decay) u = __builtin_fmaf(a.wd, w, u);
    w = __builtin_fmaf(-a.lr, u, w);
}

// One thread-vector: 8 consecutive elements whose gradient, master, m and v are already
// in registers; updates them, stores the FP32 state and the half copy.  Bit e of dmask
// set: element e receives decoupled weight decay.
template <int DT, int OPT>
__device__ __forceinline__ void update8(const uint4& G, const float4 (&W)[2], const float4 (&M)[2],
                                        const float4 (&V)[2], const Coefs& c, const UpdateArgs& a,
                                        uint32_t dmask, uint4* __restrict__ h4,
                                        float4* __restrict__ w4, float4* __restrict__ m4,
                                        float4* __restrict__ v4, uint64_t i) {
    constexpr bool ADAM = OPT == 0;
    const uint32_t gw[4] = {G.x, G.y, G.z, G.w};
    float w[8] = {W[0].x, W[0].y, W[0].z, W[0].w, W[1].x, W[1].y, W[1].z, W[1].w};
    float m[8] = {M[0].x, M[0].y, M[0].z, M[0].w, M[1].x, M[1].y, M[1].z, M[1].w};
    float v[8];
    if constexpr (ADAM) {
        v[0] = V[0].x; v[1] = V[0].y; v[2] = V[0].z; v[3] = V[0].w;
        v[4] = V[1].x; v[5] = V[1].y; v[6] = V[1].z; v[7] = V[1].w;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const bool d0 = (dmask >> (2 * k)) & 1u, d1 = (dmask >> (2 * k + 1)) & 1u;
        if constexpr (ADAM) {
            adam(Fmt<DT>::lo(gw[k]), w[2 * k], m[2 * k], v[2 * k], c, a, d0);
            adam(Fmt<DT>::hi(gw[k]), w[2 * k + 1], m[2 * k + 1], v[2 * k + 1], c, a, d1);
        } else {
            sgd(Fmt<DT>::lo(gw[k]), w[2 * k], m[2 * k], c, a, d0);
            sgd(Fmt<DT>::hi(gw[k]), w[2 * k + 1], m[2 * k + 1], c, a, d1);
        }
    }
    constexpr bool NTS = NZ1_UPDATE_NT_STORE;
    st16<NTS>(w4 + 2 * i, make_float4(w[0], w[1], w[2], w[3]));
    st16<NTS>(w4 + 2 * i + 1, make_float4(w[4], w[5], w[6], w[7]));
    st16<NTS>(m4 + 2 * i, make_float4(m[0], m[1], m[2], m[3]));
    st16<NTS>(m4 + 2 * i + 1, make_float4(m[4], m[5], m[6], m[7]));
    if constexpr (ADAM) {
        st16<NTS>(v4 + 2 * i, make_float4(v[0], v[1], v[2], v[3]));
        st16<NTS>(v4 + 2 * i + 1, make_float4(v[4], v[5], v[6], v[7]));
    }
    st16<NTS>(h4 + i, make_uint4(Fmt<DT>::pack(w[0], w[1]), Fmt<DT>::pack(w[2], w[3]),
                                 Fmt<DT>::pack(w[4], w[5]), Fmt<DT>::pack(w[6], w[7])));
}

// One element on the scalar path.
template <int DT, int OPT>
__device__ __forceinline__ void update1(const uint16_t* __restrict__ gp, uint16_t* __restrict__ hp,
                                        float* __restrict__ wp, float* __restrict__ mp,
                                        float* __restrict__ vp, uint64_t i, const Coefs& c,
                                        const UpdateArgs& a, bool decay) {
    float w = wp[i], m = mp[i];
    if constexpr (OPT == 0) {
        float v = vp[i];
        adam(Fmt<DT>::one(gp[i]), w, m, v, c, a, decay);
        vp[i] = v;
    } else {
        sgd(Fmt<DT>::one(gp[i]), w, m, c, a, decay);
    }
    wp[i] = w;
    mp[i] = m;
    hp[i] = Fmt<DT>::enc(w);
}

// Loads of thread-vector i (8 elements) of the five arrays.
template <int OPT>
__device__ __forceinline__ void load8(const uint4* __restrict__ g4, const float4* __restrict__ w4,
                                      const float4* __restrict__ m4, const float4* __restrict__ v4,
                                      uint64_t i, uint4& G, float4 (&W)[2], float4 (&M)[2],
                                      float4 (&V)[2]) {
    constexpr bool NTG = NZ1_UPDATE_NT_GRAD, NTL = NZ1_UPDATE_NT_STATE;
    G = ld16<NTG>(g4 + i);
    W[0] = ld16<NTL>(w4 + 2 * i);
    W[1] = ld16<NTL>(w4 + 2 * i + 1);
    M[0] = ld16<NTL>(m4 + 2 * i);
    M[1] = ld16<NTL>(m4 + 2 * i + 1);
    if constexpr (OPT == 0) {
        V[0] = ld16<NTL>(v4 + 2 * i);
        V[1] = ld16<NTL>(v4 + 2 * i + 1);
    }
}

// The update of one chunk whose descriptor fields are in registers.
template <int DT, int U, int OPT>
__device__ __forceinline__ void run_chunk(const uint16_t* __restrict__ gp, uint16_t* __restrict__ hp,
                                          float* __restrict__ wp, float* __restrict__ mp,
                                          float* __restrict__ vp, uint32_t len, uint32_t flags,
                                          const Coefs& c, const UpdateArgs& a,
                                          const uint32_t* touch) {
    const uint32_t dmask = (flags & CH_DECAY) ? 0xFFu : 0u;
    uint32_t done = 0;
    // Optional: one lane reads *touch behind this block's first data loads (vector loads
    // complete in order, so the data does not wait for it); an empty asm at the end
    // consumes it.
    uint32_t touched = 0;
    bool pending = touch != nullptr && threadIdx.x == 0;
    if (flags & CH_VEC) {
        const uint4* __restrict__ g4 = reinterpret_cast<const uint4*>(gp);
        uint4* __restrict__ h4 = reinterpret_cast<uint4*>(hp);
        float4* __restrict__ w4 = reinterpret_cast<float4*>(wp);
        float4* __restrict__ m4 = reinterpret_cast<float4*>(mp);
        float4* __restrict__ v4 = reinterpret_cast<float4*>(vp);
        const uint32_t nvec = len / kVec;
        for (uint32_t base = 0; base < nvec; base += U * kUpdateBlock) {
            uint4 G[U];
            float4 W[U][2], M[U][2], V[U][2];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = base + u * kUpdateBlock + threadIdx.x;
                if (i < nvec) load8<OPT>(g4, w4, m4, v4, i, G[u], W[u], M[u], V[u]);
            }
            if (pending) {
                touched = __hip_atomic_load(touch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                pending = false;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = base + u * kUpdateBlock + threadIdx.x;
                if (i < nvec) update8<DT, OPT>(G[u], W[u], M[u], V[u], c, a, dmask, h4, w4, m4, v4, i);
            }
        }
        done = nvec * kVec;
    }
    if (pending) touched = __hip_atomic_load(touch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    // scalar path: chunks that are not 16-byte aligned, and the last < 8 elements
    for (uint32_t i = done + threadIdx.x; i < len; i += kUpdateBlock)
        update1<DT, OPT>(gp, hp, wp, mp, vp, i, c, a, (flags & CH_DECAY) != 0);
    asm volatile("" ::"v"(touched));
}

// NZ1_UPDATE_REVERSE walks the chunks last-to-first, so the first gradients the update
// reads are the ones the norm pass read last.
__device__ __forceinline__ const Chunk* chunk_at(const Chunk* chunks, uint32_t nchunks, uint32_t k) {
    return chunks + (NZ1_UPDATE_REVERSE ? nchunks - 1 - k : k);
}

// Generic layout: one block per entry of the chunk table.  FUSE: the block takes the
// step's decisions from the norm pass's partials itself (small norm grids, no finalize).
template <int DT, int U, int OPT, bool FUSE>
__global__ __launch_bounds__(kUpdateBlock) void update_kernel(const Chunk* __restrict__ chunks,
                                                              uint32_t nchunks,
                                                              const DevState* __restrict__ st,
                                                              UpdateArgs a, Fuse f) {
    const Chunk* ch = chunk_at(chunks, nchunks, blockIdx.x);
    // The descriptor and the finalize's decision are fetched together: the early exit
    // below tests both, so neither load waits for the other.
    const uint32_t len = ch->len;
    const uint32_t flags = ch->flags;
    const uint16_t* __restrict__ gp = ch->grad;
    uint16_t* __restrict__ hp = ch->half;
    float* __restrict__ wp = ch->master;
    float* __restrict__ mp = ch->m;
    float* __restrict__ vp = ch->v;
    int32_t skip;
    Coefs c;
    if constexpr (FUSE) {
        const Decision d = fused_decide(f);
        if (blockIdx.x == 0 && threadIdx.x == 0) write_state(f.st, d.next);
        skip = d.next.skip;
        c = Coefs{d.next.gscale, d.next.rbc1, d.next.rsbc2};
    } else {
        skip = st->skip;
        c = Coefs{st->gscale, st->rbc1, st->rsbc2};
    }
    // Chunks are never empty, their pointers are at least 2-byte aligned and flags use
    // the low bits only, so the last two terms never fire; they make the branch wait for
    // the whole descriptor at once.
    const uint32_t odd = (uint32_t)(((uintptr_t)gp | (uintptr_t)hp | (uintptr_t)wp |
                                     (uintptr_t)mp | (uintptr_t)vp) & 1u) | (flags >> 31);
    if (skip | (len == 0) | odd) return;
    // Touch the descriptor of the block NZ1_DESC_AHEAD places later (a multiple of 8, so
    // on the same XCD under round-robin dispatch), so that block finds it in cache.
    const uint32_t ahead = blockIdx.x + NZ1_DESC_AHEAD;
    const uint32_t* touch =
        (NZ1_DESC_AHEAD && ahead < nchunks) ? &chunk_at(chunks, nchunks, ahead)->len : nullptr;
    run_chunk<DT, U, OPT>(gp, hp, wp, mp, vp, len, flags, c, a, touch);
}

// Decay bits of the n <= 8 consecutive elements starting at offset o of a tile: the
// tile's starting flag, flipped at each of the tile's change offsets that is <= the
// element's offset.  change[first, end) is uniform across the block.
__device__ __forceinline__ uint32_t decay_bits(const uint32_t* __restrict__ change, uint32_t first,
                                               uint32_t end, uint32_t o, uint32_t start_mask) {
    uint32_t mask = start_mask;
    for (uint32_t j = first; j < end; ++j) {
        const int d = (int)change[j] - (int)o;
        if (d <= 0) mask ^= 0xFFu;
        else if (d < kVec) mask ^= (0xFFu << d) & 0xFFu;
    }
    return mask;
}

// Uses loaded values (register operands of an empty asm).  Placed on the skip branch
// after the loads, it gives them a user on both sides of that branch, so the compiler
// cannot sink them below it (with NZ1_FLAT_SPECULATE they are in flight while the block
// waits for the decision).
template <int OPT>
__device__ __forceinline__ void keep_loaded(const uint4& G, const float4 (&W)[2],
                                            const float4 (&M)[2], const float4 (&V)[2]) {
    asm volatile("" ::"v"(G.x), "v"(W[0].x), "v"(W[1].x), "v"(M[0].x), "v"(M[1].x));
    if constexpr (OPT == 0) asm volatile("" ::"v"(V[0].x), "v"(V[1].x));
}

// What a flat-update block reads besides its data: the finalize's decision and
// coefficients, and its tile's two decay words.  Read with relaxed atomic loads: those
// are vector-memory loads, which return in issue order, and the compiler keeps them in
// program order after the data loads, so the block issues its whole tile before it
// waits for them.  (Plain loads of these uniform values would become scalar loads,
// whose out-of-order completion makes the compiler wait for all of them before the data
// loads go out.)  Workgroup scope suffices: the values were written by an earlier
// kernel, complete before this one started.
struct StepWords {
    int32_t skip;
    float gscale, rbc1, rsbc2;
    uint32_t w0, w1;
};
__device__ __forceinline__ StepWords ld_after(const DevState* st, const uint32_t* word) {
    const uint64_t a = __hip_atomic_load(reinterpret_cast<const uint64_t*>(&st->skip),
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint64_t b = __hip_atomic_load(reinterpret_cast<const uint64_t*>(&st->rbc1),
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    StepWords r;
    r.skip = (int32_t)(uint32_t)a;
    r.gscale = __uint_as_float((uint32_t)(a >> 32));
    r.rbc1 = __uint_as_float((uint32_t)b);
    r.rsbc2 = __uint_as_float((uint32_t)(b >> 32));
    r.w0 = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    r.w1 = __hip_atomic_load(word + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return r;
}

// The decision, coefficients and tile words of a flat-update block: from the state block
// behind the data (ld_after), or, with FUSE, taken by the block itself (block 0 also
// writes the state block).
template <bool FUSE>
__device__ __forceinline__ StepWords step_words(const DevState* st, const uint32_t* word, const Fuse& f,
                                                const FusedIn& in) {
    if constexpr (FUSE) {
        const Decision d = fused_finish(in, f);
        if (blockIdx.x == 0 && threadIdx.x == 0) write_state(f.st, d.next);
        StepWords r;
        r.skip = d.next.skip;
        r.gscale = d.next.gscale;
        r.rbc1 = d.next.rbc1;
        r.rsbc2 = d.next.rsbc2;
        r.w0 = word[0];
        r.w1 = word[1];
        return r;
    } else {
        return ld_after(st, word);
    }
}

// Flat layout: the segments tile five contiguous 16-byte-aligned arrays (a flat
// partition), so tile T's addresses follow from T alone: a block needs no work
// descriptor (a per-block load that streaming has evicted to HBM) before its first data
// load, only the finalize's decision, which every block reads and the L2 keeps.  The
// tile's decay words and the coefficients are fetched behind the data.
template <int DT, int OPT, bool FUSE>
__global__ __launch_bounds__(kFlatBlock) void flat_update_kernel(FlatSpan s,
                                                             const uint32_t* __restrict__ tile_word,
                                                             const uint32_t* __restrict__ change,
                                                             const DevState* __restrict__ st,
                                                             UpdateArgs a, Fuse f) {
    constexpr int U = kFlatUnroll;
    const uint32_t T = s.ntiles - 1 - blockIdx.x;     // last tile first, as above
    const uint64_t nvec = s.n / kVec;
    const uint64_t v0 = (uint64_t)T * (U * kFlatBlock);
    const uint4* __restrict__ g4 = reinterpret_cast<const uint4*>(s.grad);
    uint4* __restrict__ h4 = reinterpret_cast<uint4*>(s.half);
    float4* __restrict__ w4 = reinterpret_cast<float4*>(s.master);
    float4* __restrict__ m4 = reinterpret_cast<float4*>(s.m);
    float4* __restrict__ v4 = reinterpret_cast<float4*>(s.v);

#if !NZ1_FLAT_SPECULATE
    // Wait for the decision before loading: a skipped step then reads nothing here.  The
    // base pointers are 16-byte aligned, so their low-bit term never fires; it makes the
    // branch wait for them too, so they are fetched with the state pointer, not after.
    // (With FUSE the decision is not made yet: the block issues its tile's loads first and
    // decides behind them, so a skipped step still reads every tile.)
    if constexpr (!FUSE) {
        const uintptr_t low = ((uintptr_t)s.grad | (uintptr_t)s.half | (uintptr_t)s.master |
                               (uintptr_t)s.m | (uintptr_t)s.v) & 1u;
        if (st->skip | (int32_t)low) return;
    }
#endif
    // With FUSE the decision's inputs are loaded first, so its arithmetic overlaps the
    // data loads' latency.
    FusedIn fin_in{};
    if constexpr (FUSE) fin_in = fused_load(f);
    if (T + 1 < s.ntiles || s.n % kFlatTile == 0) {
        // a full tile: every thread owns U whole vectors
        uint4 G[U];
        float4 W[U][2], M[U][2], V[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u)
            load8<OPT>(g4, w4, m4, v4, v0 + u * kFlatBlock + threadIdx.x, G[u], W[u], M[u], V[u]);
        // Then the decision, the coefficients and the tile words, as vector loads issued
        // behind the data (see ld_after), or the block's own decision (FUSE).
        if constexpr (FUSE) after_data(fin_in);
        // A deciding AdamW block pauses briefly after issuing its tile's loads, before it
        // takes the decision and computes.  Measured on MI355X (215M-element shard, same
        // process, alternating builds, us per update): no pause 1026-1031, 6 x 64 clocks
        // 1013-1016, 8 x 64 1005-1009, 12 x 64 1013-1017, 16 x 64 1024-1027, 24 x 64
        // 1055-1057; a Pythia-410M rank, 16M and 1M shards and momentum SGD unchanged.
        // (Extra ALU work in the same place gives the same gain at the same length: the
        // gain is the timing, not the work.)
        if constexpr (FUSE && OPT == 0 && NZ1_FLAT_PAUSE > 0) __builtin_amdgcn_s_sleep(NZ1_FLAT_PAUSE);
        const StepWords sw = step_words<FUSE>(st, tile_word + T, f, fin_in);
        const Coefs c{sw.gscale, sw.rbc1, sw.rsbc2};
        const uint32_t first = sw.w0 >> 1, end = sw.w1 >> 1;
        const uint32_t start_mask = (sw.w0 & 1u) ? 0xFFu : 0u;
        // words are non-decreasing, so (end < first) never holds; it keeps the tile-word
        // loads above the branch with the decision
        if (sw.skip | (end < first)) {
#pragma unroll
            for (int u = 0; u < U; ++u) keep_loaded<OPT>(G[u], W[u], M[u], V[u]);
            return;
        }
        if (first == end) {
            // one decay flag for the whole tile
#pragma unroll
            for (int u = 0; u < U; ++u)
                update8<DT, OPT>(G[u], W[u], M[u], V[u], c, a, start_mask, h4, w4, m4, v4,
                                 v0 + u * kFlatBlock + threadIdx.x);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t o = (uint32_t)(u * kFlatBlock + threadIdx.x) * kVec;
                update8<DT, OPT>(G[u], W[u], M[u], V[u], c, a,
                                 decay_bits(change, first, end, o, start_mask), h4, w4, m4, v4,
                                 v0 + u * kFlatBlock + threadIdx.x);
            }
        }
        return;
    }

    // the last tile, shorter than kFlatTile: guarded vectors, then the last n % 8
    // elements on the scalar path
    const StepWords sw = step_words<FUSE>(st, tile_word + T, f, fin_in);
    if (sw.skip) return;
    const Coefs c{sw.gscale, sw.rbc1, sw.rsbc2};
    const uint32_t first = sw.w0 >> 1, end = sw.w1 >> 1;
    const uint32_t start_mask = (sw.w0 & 1u) ? 0xFFu : 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t i = v0 + u * kFlatBlock + threadIdx.x;
        if (i < nvec) {
            uint4 G;
            float4 W[2], M[2], V[2];
            load8<OPT>(g4, w4, m4, v4, i, G, W, M, V);
            const uint32_t o = (uint32_t)(u * kFlatBlock + threadIdx.x) * kVec;
            update8<DT, OPT>(G, W, M, V, c, a, decay_bits(change, first, end, o, start_mask), h4,
                             w4, m4, v4, i);
        }
    }
    const uint64_t e = nvec * kVec + threadIdx.x;
    if (e < s.n) {
        const uint32_t o = (uint32_t)(e - (uint64_t)T * kFlatTile);
        const bool decay = decay_bits(change, first, end, o, start_mask) & 1u;
        update1<DT, OPT>(s.grad, s.half, s.master, s.m, s.v, e, c, a, decay);
    }
}

// ------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------
constexpr int kUpdateUnroll = NZ1_UPDATE_UNROLL;

// One launch, timed through its own dispatch when t carries events.
template <typename... Params, typename... Args>
static void launch(void (*kernel)(Params...), dim3 grid, dim3 block, uint32_t lds,
                   hipStream_t stream, const KernelTiming& t, Args... args) {
    if (t.start)
        hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, t.start, t.stop, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
}

hipError_t launch_norm(int dtype, bool nt_loads, bool big, const Chunk* chunks, uint32_t nchunks,
                       uint32_t blocks, const DevState* st, double* partial, DevState* snap,
                       uint32_t lds_reserve, hipStream_t stream, const KernelTiming& t) {
    if (big) {
        auto k = dtype == 1 ? (nt_loads ? norm_kernel<1, true, kNormBigBlock> : norm_kernel<1, false, kNormBigBlock>)
                            : (nt_loads ? norm_kernel<2, true, kNormBigBlock> : norm_kernel<2, false, kNormBigBlock>);
        launch(k, dim3(blocks), dim3(kNormBigBlock), lds_reserve, stream, t, chunks, nchunks, st,
               partial, snap);
    } else {
        auto k = dtype == 1 ? (nt_loads ? norm_kernel<1, true, kBlock> : norm_kernel<1, false, kBlock>)
                            : (nt_loads ? norm_kernel<2, true, kBlock> : norm_kernel<2, false, kBlock>);
        launch(k, dim3(blocks), dim3(kBlock), lds_reserve, stream, t, chunks, nchunks, st, partial,
               snap);
    }
    return hipGetLastError();
}

hipError_t launch_finalize(const double* partial, uint32_t nparts, DevState* st,
                           const FinalizeArgs& a, hipStream_t stream, const KernelTiming& t) {
    launch(finalize_kernel, dim3(1), dim3(kFinalizeBlock), 0, stream, t, partial, nparts, st, a);
    return hipGetLastError();
}

hipError_t launch_reduce(const double* partial, uint32_t nparts, double* out, hipStream_t stream) {
    reduce_kernel<<<1, kFinalizeBlock, 0, stream>>>(partial, nparts, out);
    return hipGetLastError();
}

hipError_t launch_segment_sumsq(const double* partial, const uint32_t* range, uint32_t nseg,
                                double* out, hipStream_t stream) {
    segment_sumsq_kernel<<<nseg, kBlock, 0, stream>>>(partial, range, out);
    return hipGetLastError();
}

hipError_t launch_set_state(DevState* st, float scale, int32_t good_steps, int64_t step,
                            int64_t skipped, int32_t consecutive, double predivide, double dp,
                            hipStream_t stream) {
    set_state_kernel<<<1, 64, 0, stream>>>(st, scale, good_steps, step, skipped, consecutive,
                                           predivide, dp);
    return hipGetLastError();
}

template <int OPT, bool FUSE>
static void launch_update_opt(int dtype, const Chunk* chunks, uint32_t nchunks, const DevState* st,
                              const UpdateArgs& a, const Fuse& f, uint32_t lds, hipStream_t stream,
                              const KernelTiming& t) {
    launch(dtype == 1 ? update_kernel<1, kUpdateUnroll, OPT, FUSE> : update_kernel<2, kUpdateUnroll, OPT, FUSE>,
           dim3(nchunks), dim3(kUpdateBlock), lds, stream, t, chunks, nchunks, st, a, f);
}

template <int OPT, bool FUSE>
static void launch_flat_opt(int dtype, const FlatSpan& sp, const DevState* st, const UpdateArgs& a,
                            const Fuse& f, uint32_t lds, hipStream_t stream, const KernelTiming& t) {
    launch(dtype == 1 ? flat_update_kernel<1, OPT, FUSE> : flat_update_kernel<2, OPT, FUSE>,
           dim3(sp.ntiles), dim3(kFlatBlock), lds, stream, t, sp, sp.tile_word, sp.change, st, a, f);
}

static Fuse fuse_args(const FuseIn* in) {
    Fuse f{};
    if (in) {
        f.partial = in->partial;
        f.nparts = in->nparts;
        f.snap = in->snap;
        f.st = in->st;
        f.fin = in->fin;
    }
    return f;
}

hipError_t launch_flat_update(int dtype, int optimizer, const FlatSpan& sp, const DevState* st,
                              const UpdateArgs& a, const FuseIn* fuse, uint32_t lds_reserve,
                              hipStream_t stream, const KernelTiming& t) {
    const Fuse f = fuse_args(fuse);
    if (optimizer == 1)
        fuse ? launch_flat_opt<1, true>(dtype, sp, st, a, f, lds_reserve, stream, t)
             : launch_flat_opt<1, false>(dtype, sp, st, a, f, lds_reserve, stream, t);
    else
        fuse ? launch_flat_opt<0, true>(dtype, sp, st, a, f, lds_reserve, stream, t)
             : launch_flat_opt<0, false>(dtype, sp, st, a, f, lds_reserve, stream, t);
    return hipGetLastError();
}

// lds_reserve: dynamic LDS the kernel never touches, requested only to cap how many
// blocks share a CU (fewer tiles in flight keep the chip's open DRAM rows few).
hipError_t launch_update(int dtype, int optimizer, const Chunk* chunks, uint32_t nchunks,
                         const DevState* st, const UpdateArgs& a, const FuseIn* fuse,
                         uint32_t lds_reserve, hipStream_t stream, const KernelTiming& t) {
    const Fuse f = fuse_args(fuse);
    if (optimizer == 1)
        fuse ? launch_update_opt<1, true>(dtype, chunks, nchunks, st, a, f, lds_reserve, stream, t)
             : launch_update_opt<1, false>(dtype, chunks, nchunks, st, a, f, lds_reserve, stream, t);
    else
        fuse ? launch_update_opt<0, true>(dtype, chunks, nchunks, st, a, f, lds_reserve, stream, t)
             : launch_update_opt<0, false>(dtype, chunks, nchunks, st, a, f, lds_reserve, stream, t);
    return hipGetLastError();
}

hipError_t norm_static_lds(uint32_t* bytes, uint32_t* big_bytes) {
    hipFuncAttributes a{}, b{};
    hipError_t e = hipFuncGetAttributes(&a, reinterpret_cast<const void*>(&norm_kernel<1, true, kBlock>));
    if (e == hipSuccess)
        e = hipFuncGetAttributes(&b, reinterpret_cast<const void*>(&norm_kernel<1, true, kNormBigBlock>));
    *bytes = e == hipSuccess ? (uint32_t)a.sharedSizeBytes : 0u;
    *big_bytes = e == hipSuccess ? (uint32_t)b.sharedSizeBytes : 0u;
    return e;
}

}  // namespace nz1
