// zero1_api.hip -- host side of the C ABI declared in include/neox_zero1.h:
// argument validation, the ZeRO-1 shard partition, the chunk table, device scratch,
// kernel launches and state readback.
#include "neox_zero1.h"
#include "zero1_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

using namespace nz1;

namespace nz1 {

static thread_local std::string g_last_error = "no error";

int set_error(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    try {
        g_last_error = buf;
    } catch (...) {
        // keep the previous message rather than let an exception cross the C ABI
    }
    return code;
}

int set_hip_error(hipError_t e, const char* what) {
    return set_error(NEOX_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

}  // namespace nz1

namespace {

// Work-unit sizes (elements), measured best on MI355X: the update wants small blocks
// (2,048 elements: 128 threads x two 16-byte vectors per array) at 2 blocks per CU on
// long grids, the
// read-only norm pass more bytes per block (32K elements, 8 loads in flight per thread)
// at 4 blocks per CU.
#ifndef NZ1_UPDATE_CHUNK
#define NZ1_UPDATE_CHUNK 2048
#endif
#ifndef NZ1_NORM_CHUNK
#define NZ1_NORM_CHUNK 32768
#endif
// Blocks per CU for each pass (0 = as many as registers allow).  The cap is enforced by
// reserving an equal share of the CU's LDS per block.
#ifndef NZ1_UPDATE_BLOCKS_PER_CU
#define NZ1_UPDATE_BLOCKS_PER_CU 2
#endif
// The norm pass: 4 blocks per CU measured 62.8-63.2 us on the 215M shard against
// 64.9-65.0 at 3 and 79.5-79.7 at 2 (same process, alternating builds).
#ifndef NZ1_NORM_BLOCKS_PER_CU
#define NZ1_NORM_BLOCKS_PER_CU 4
#endif
// Longest norm chunk of the large-block norm pass: 2^28 elements, so that every shard
// one GPU can hold (~1.8e10 elements at 16 bytes each) fits 256 chunks.
#ifndef NZ1_NORM_BIG_MAX_CHUNK
#define NZ1_NORM_BIG_MAX_CHUNK (1u << 28)
#endif
#ifndef NZ1_FLAT_BLOCKS_PER_CU
#define NZ1_FLAT_BLOCKS_PER_CU 2
#endif
// Momentum SGD (20 B/param over seven streams, both update kernels): 4 blocks per CU
// on grids of at most NZ1_SGD_SHORT_GRID blocks per CU, 2 on longer ones.  Measured on
// MI355X, flat one-segment shards, same arrays, alternating builds, median us per
// update at 4 / 2 blocks per CU: 2M elements 7.4 / 8.8, 8M 27.4 / 30.9, 16M 49.4 / 55.1,
// 32M 103 / 112, 44M 157.5 / 150.2, 64M 230 / 218, 128M 460 / 427, the 215M shard
// 756-760 / 707-710 (the grid has 61 blocks per CU at 32M and 84 at 44M).
#ifndef NZ1_SGD_BLOCKS_PER_CU_SHORT
#define NZ1_SGD_BLOCKS_PER_CU_SHORT 4
#endif
#ifndef NZ1_SGD_BLOCKS_PER_CU_LONG
#define NZ1_SGD_BLOCKS_PER_CU_LONG 2
#endif
#ifndef NZ1_SGD_SHORT_GRID
#define NZ1_SGD_SHORT_GRID 64
#endif
// Short update grids want more blocks in flight: a pass of a few blocks per CU is
// dominated by its ramp-up and drain, while on long grids more tiles in flight mean more
// open DRAM rows.  Up to NZ1_SHORT_GRID blocks per CU of grid the AdamW update runs 4
// blocks per CU, beyond that the defaults above.  Measured on MI355X, one-segment shards,
// same arrays, alternating builds, two rounds, median us per update at 2 / 4 / 8 blocks
// per CU; flat (deciding) update: 4M 24.8-26.0 / 21.3-21.6 / 22.6-22.7, 8M 42.0-42.3 /
// 37.1 / 39.3-39.4, 12M 60.8-62.0 / 54.7 / 55.4-56.0, 16M 77.6-77.8 / 71.5-71.6 /
// 73.4-73.5, 20M 103.3-103.7 / 96.7-96.9 / 98.4-98.9, 24M 114.1-115.3 / 110.7-111.1 /
// 112.1-112.2, 28M 135.3-135.8 / 143.2-143.8 / 143.6-143.7, 32M 155.3 / 165.7-166.4 /
// 168.3-168.4, 44M 206.5-207.3 / 222.9-223.5 / 229.4-229.5; chunk-table update: 8M
// 50.8-51.7 / 40.8-41.0 / 40.9-41.3, 16M 68.2-68.3 / 68.8-69.0 / 73.8-74.0, 24M
// 115.5-115.7 / 107.7-108.0 / 107.2-107.4, 28M 141.8-142.5 / 139.7-140.5 / 141.8-142.1,
// 32M 158.9-159.1 / 161.7-161.8 / 169.5-169.9 (on 256 CUs the grid has 15 blocks per CU
// at 8M, 46 at 24M, 53 at 28M; M = 1e6 elements).
#ifndef NZ1_SHORT_GRID
#define NZ1_SHORT_GRID 48
#endif
// Timing events skip the system-scope fence an event otherwise performs when it
// completes (an L2 write-back and invalidate that slows the kernels after it): they are
// only read for elapsed times, and every readback of results synchronizes by itself.
#ifndef NZ1_TIMING_EVENT_FLAGS
#define NZ1_TIMING_EVENT_FLAGS hipEventDisableSystemFence
#endif
constexpr uint32_t kDefaultChunk = NZ1_UPDATE_CHUNK;
constexpr uint32_t kNormChunk = NZ1_NORM_CHUNK;

// start / stop of the norm, finalize and update kernels of one recorded step
struct TimingSlot {
    hipEvent_t ev[6];
};

}  // namespace

struct neox_zero1 {
    neox_zero1_config cfg;
    int device = 0;
    StepLaunch sl;                 // the step's launches, device addresses resolved
    // library-owned device memory
    uint32_t* d_tile_word = nullptr;
    uint32_t* d_change = nullptr;
    Chunk* d_chunks = nullptr;
    Chunk* d_norm_chunks = nullptr;
    uint32_t* d_seg_range = nullptr;   // per segment: [first, end) norm chunk (telemetry)
    double* d_seg_sumsq = nullptr;     // per segment squared norm of the last step
    double* d_partial = nullptr;
    DevState* d_state = nullptr;       // [0] the state block, [1] the pre-step snapshot
    uint32_t nseg = 0;
    hipStream_t last_stream = nullptr;
    // profiling
    std::vector<TimingSlot> timing;
    int64_t timing_used = 0;
    bool timing_update_only = false;
};

// ------------------------------------------------------------------------------------
// configuration
// ------------------------------------------------------------------------------------
extern "C" int neox_zero1_default_config(neox_zero1_config* cfg) {
    if (!cfg) return set_error(NEOX_EINVAL, "cfg is NULL");
    std::memset(cfg, 0, sizeof *cfg);
    cfg->beta1 = 0.9;
    cfg->beta2 = 0.95;
    cfg->eps = 1e-8;
    cfg->weight_decay = 0.01;
    cfg->clip_norm = 1.0;
    cfg->predivide_factor = 1.0;
    cfg->dp_world_size = 1;
    cfg->dtype = NEOX_F16;
    cfg->scaler_mode = NEOX_SCALER_DYNAMIC;
    cfg->growth_interval = 1000;
    cfg->init_scale = 65536.0;
    cfg->growth_factor = 2.0;
    cfg->backoff_factor = 0.5;
    cfg->min_scale = 1.0;
    return NEOX_OK;
}

static bool finite_pos(double x) { return std::isfinite(x) && x > 0.0; }

static int validate_config(const neox_zero1_config* c) {
    if (!(c->beta1 >= 0.0 && c->beta1 < 1.0)) return set_error(NEOX_EINVAL, "beta1 %g not in [0,1)", c->beta1);
    if (!(c->beta2 >= 0.0 && c->beta2 < 1.0)) return set_error(NEOX_EINVAL, "beta2 %g not in [0,1)", c->beta2);
    // eps = 0 would make a zero-gradient element with zero moments compute 0 / 0
    if (!(std::isfinite(c->eps) && c->eps > 0.0 && (float)c->eps > 0.0f))
        return set_error(NEOX_EINVAL, "eps %g: must be > 0 in FP32", c->eps);
    if (!(std::isfinite(c->weight_decay) && c->weight_decay >= 0.0))
        return set_error(NEOX_EINVAL, "weight_decay %g", c->weight_decay);
    if (std::isnan(c->clip_norm) || std::isinf(c->clip_norm))
        return set_error(NEOX_EINVAL, "clip_norm %g", c->clip_norm);
    if (!finite_pos(c->predivide_factor)) return set_error(NEOX_EINVAL, "predivide_factor %g", c->predivide_factor);
    if (c->dp_world_size < 1) return set_error(NEOX_EINVAL, "dp_world_size %d", c->dp_world_size);
    if (c->dtype != NEOX_F16 && c->dtype != NEOX_BF16) return set_error(NEOX_EINVAL, "dtype %d", c->dtype);
    if (c->scaler_mode != NEOX_SCALER_DYNAMIC && c->scaler_mode != NEOX_SCALER_STATIC)
        return set_error(NEOX_EINVAL, "scaler_mode %d", c->scaler_mode);
    if (c->growth_interval < 1) return set_error(NEOX_EINVAL, "growth_interval %d", c->growth_interval);
    if (!finite_pos(c->init_scale) || !std::isfinite((float)c->init_scale) || (float)c->init_scale <= 0.0f)
        return set_error(NEOX_EINVAL, "init_scale %g", c->init_scale);
    if (!(std::isfinite(c->growth_factor) && c->growth_factor >= 1.0))
        return set_error(NEOX_EINVAL, "growth_factor %g", c->growth_factor);
    if (!(c->backoff_factor > 0.0 && c->backoff_factor <= 1.0))
        return set_error(NEOX_EINVAL, "backoff_factor %g", c->backoff_factor);
    if (!finite_pos(c->min_scale) || (float)c->min_scale <= 0.0f || !std::isfinite((float)c->min_scale))
        return set_error(NEOX_EINVAL, "min_scale %g", c->min_scale);
    if (c->init_step < 0 || c->init_skipped < 0 || c->init_good_steps < 0 ||
        c->init_consecutive_overflows < 0)
        return set_error(NEOX_EINVAL, "negative resume counter");
    if (c->chunk_elems != 0 &&
        (c->chunk_elems % kVec != 0 || c->chunk_elems < 256 || c->chunk_elems > (1u << 24)))
        return set_error(NEOX_EINVAL, "chunk_elems %u: multiple of 8 in [256, 2^24]", c->chunk_elems);
    if (c->norm_blocks > (1u << 20)) return set_error(NEOX_EINVAL, "norm_blocks %u too large", c->norm_blocks);
    if (c->optimizer != NEOX_OPT_ADAMW && c->optimizer != NEOX_OPT_SGD)
        return set_error(NEOX_EINVAL, "optimizer %d", c->optimizer);
    if (c->segment_norms > 1) return set_error(NEOX_EINVAL, "segment_norms %u", c->segment_norms);
    if (c->chunked_update > 1) return set_error(NEOX_EINVAL, "chunked_update %u", c->chunked_update);
    if (c->segment_norms && c->norm_blocks)
        return set_error(NEOX_EINVAL, "segment_norms needs the one-block-per-chunk norm pass (norm_blocks 0)");
    return NEOX_OK;
}

// ------------------------------------------------------------------------------------
// shard partition: interval intersection of each tensor with the rank's range
// ------------------------------------------------------------------------------------
extern "C" int neox_zero1_partition(const uint64_t* tensor_numel, const uint8_t* tensor_decay,
                                    uint64_t ntensors, uint32_t dp_world_size, uint32_t rank,
                                    uint32_t align, neox_shard_segment* out, uint64_t cap,
                                    uint64_t* nseg_out, uint64_t* shard_numel_out) {
    if (!nseg_out || !shard_numel_out) return set_error(NEOX_EINVAL, "null output pointer");
    if (ntensors && (!tensor_numel || !tensor_decay)) return set_error(NEOX_EINVAL, "null tensor list");
    if (cap && !out) return set_error(NEOX_EINVAL, "out is NULL with cap > 0");
    if (dp_world_size == 0 || align == 0) return set_error(NEOX_EINVAL, "dp_world_size and align must be >= 1");
    if (rank >= dp_world_size) return set_error(NEOX_EINVAL, "rank %u >= dp_world_size %u", rank, dp_world_size);
    uint64_t total = 0;
    for (uint64_t i = 0; i < ntensors; ++i) {
        if (tensor_numel[i] > UINT64_MAX - total) return set_error(NEOX_EINVAL, "total numel overflows");
        total += tensor_numel[i];
    }
    const unsigned __int128 unit = (unsigned __int128)dp_world_size * align;
    const unsigned __int128 padded128 = ((unsigned __int128)total + unit - 1) / unit * unit;
    if (padded128 > UINT64_MAX) return set_error(NEOX_EINVAL, "padded numel overflows");
    const uint64_t padded = (uint64_t)padded128;
    const uint64_t P = padded / dp_world_size;
    const uint64_t lo = (uint64_t)rank * P, hi = lo + P;

    uint64_t n = 0;
    auto emit = [&](uint64_t a, uint64_t b, uint64_t tensor_start, uint32_t tid, uint32_t flags) {
        if (n < cap) {
            out[n].shard_offset = a - lo;
            out[n].numel = b - a;
            out[n].tensor_offset = a - tensor_start;
            out[n].tensor_id = tid;
            out[n].flags = flags;
        }
        ++n;
    };
    uint64_t off = 0;
    for (uint64_t i = 0; i < ntensors && off < hi; ++i) {
        const uint64_t a = off > lo ? off : lo;
        const uint64_t end = off + tensor_numel[i];
        const uint64_t b = end < hi ? end : hi;
        if (a < b) emit(a, b, off, (uint32_t)i, tensor_decay[i] ? NEOX_SEG_DECAY : 0u);
        off = end;
    }
    {
        const uint64_t a = total > lo ? total : lo;
        const uint64_t b = padded < hi ? padded : hi;
        if (a < b) emit(a, b, total, NEOX_PAD_TENSOR, 0u);
    }
    *nseg_out = n;
    *shard_numel_out = P;
    return NEOX_OK;
}

// ------------------------------------------------------------------------------------
// chunk table
// ------------------------------------------------------------------------------------
static bool aligned16(uintptr_t p) { return (p & 15u) == 0; }

// Smallest head h in [0, 8) after which all five arrays are 16-byte aligned, or -1.
static int vector_head(const neox_segment& s) {
    for (int h = 0; h < kVec; ++h) {
        if (aligned16((uintptr_t)s.grad + 2u * h) && aligned16((uintptr_t)s.half + 2u * h) &&
            aligned16((uintptr_t)s.master + 4u * h) && aligned16((uintptr_t)s.exp_avg + 4u * h) &&
            (!s.exp_avg_sq || aligned16((uintptr_t)s.exp_avg_sq + 4u * h)))
            return h;
    }
    return -1;
}

static void push_chunk(std::vector<Chunk>& t, const neox_segment& s, uint32_t seg, uint64_t start,
                       uint32_t len, bool vec) {
    Chunk c{};
    c.grad = static_cast<const uint16_t*>(s.grad) + start;
    c.half = static_cast<uint16_t*>(s.half) + start;
    c.master = s.master + start;
    c.m = s.exp_avg + start;
    c.v = s.exp_avg_sq ? s.exp_avg_sq + start : nullptr;
    c.len = len;
    c.flags = ((s.flags & NEOX_SEG_DECAY) ? CH_DECAY : 0u) | (vec ? CH_VEC : 0u);
    c.seg = seg;
    t.push_back(c);
}

// Entries build_chunks makes for chunk length C.
static uint64_t count_chunks(const neox_segment* segs, uint64_t nseg, uint32_t C) {
    uint64_t n = 0;
    for (uint64_t s = 0; s < nseg; ++s) {
        const int head = vector_head(segs[s]);
        const uint64_t h = head > 0 ? ((uint64_t)head < segs[s].numel ? (uint64_t)head : segs[s].numel) : 0;
        n += (h ? 1 : 0) + (segs[s].numel - h + C - 1) / C;
    }
    return n;
}

static void build_chunks(const neox_segment* segs, uint64_t nseg, uint32_t C, std::vector<Chunk>& t) {
    t.reserve(count_chunks(segs, nseg, C));
    for (uint64_t s = 0; s < nseg; ++s) {
        const neox_segment& sg = segs[s];
        const int head = vector_head(sg);
        uint64_t off = 0;
        if (head > 0) {
            const uint64_t h = (uint64_t)head < sg.numel ? (uint64_t)head : sg.numel;
            push_chunk(t, sg, (uint32_t)s, 0, (uint32_t)h, false);
            off = h;
        }
        while (off < sg.numel) {
            const uint64_t len = sg.numel - off < C ? sg.numel - off : C;
            push_chunk(t, sg, (uint32_t)s, off, (uint32_t)len, head >= 0);
            off += len;
        }
    }
}

// The segments, in order, tile five contiguous arrays (exp_avg_sq too when has_v)
// whose first elements are 16-byte aligned: one flat partition.  *n gets its length.
static bool flat_layout(const neox_segment* segs, uint64_t nseg, bool has_v, uint64_t* n) {
    const neox_segment& s0 = segs[0];
    if (!aligned16((uintptr_t)s0.grad) || !aligned16((uintptr_t)s0.half) ||
        !aligned16((uintptr_t)s0.master) || !aligned16((uintptr_t)s0.exp_avg) ||
        (has_v && !aligned16((uintptr_t)s0.exp_avg_sq)))
        return false;
    uint64_t off = 0;
    for (uint64_t k = 0; k < nseg; ++k) {
        const neox_segment& s = segs[k];
        if ((uintptr_t)s.grad != (uintptr_t)s0.grad + 2 * off ||
            (uintptr_t)s.half != (uintptr_t)s0.half + 2 * off ||
            (uintptr_t)s.master != (uintptr_t)s0.master + 4 * off ||
            (uintptr_t)s.exp_avg != (uintptr_t)s0.exp_avg + 4 * off ||
            (has_v && (uintptr_t)s.exp_avg_sq != (uintptr_t)s0.exp_avg_sq + 4 * off))
            return false;
        off += s.numel;
    }
    *n = off;
    return true;
}

// Per-tile decay description of a flat partition of n elements: word[T] = (index in
// `change` of tile T's first in-tile flag change) << 1 | flag of the tile's first
// element; word[ntiles] closes the last list; change holds in-tile offsets.
static void build_flat_tables(const neox_segment* segs, uint64_t nseg, uint64_t n,
                              std::vector<uint32_t>& word, std::vector<uint32_t>& change) {
    std::vector<uint64_t> at;   // element indices where the decay flag differs from the previous one
    uint64_t off = 0;
    for (uint64_t k = 0; k < nseg; ++k) {
        if (k && (segs[k].flags & NEOX_SEG_DECAY) != (segs[k - 1].flags & NEOX_SEG_DECAY))
            at.push_back(off);
        off += segs[k].numel;
    }
    const uint64_t ntiles = (n + kFlatTile - 1) / kFlatTile;
    word.assign(ntiles + 1, 0);
    change.clear();
    uint32_t flag = (segs[0].flags & NEOX_SEG_DECAY) ? 1u : 0u;
    size_t j = 0;
    for (uint64_t T = 0; T < ntiles; ++T) {
        const uint64_t lo = T * kFlatTile, hi = lo + kFlatTile;
        for (; j < at.size() && at[j] <= lo; ++j) flag ^= 1u;
        word[T] = (uint32_t)(change.size() << 1) | flag;
        for (size_t k = j; k < at.size() && at[k] < hi; ++k) change.push_back((uint32_t)(at[k] - lo));
    }
    word[ntiles] = (uint32_t)(change.size() << 1);
}

static bool overlaps(uintptr_t a, uint64_t abytes, uintptr_t b, uint64_t bbytes) {
    return a < b + bbytes && b < a + abytes;
}

// Every array of every segment: the written ones (half, master, exp_avg, exp_avg_sq) must
// not overlap one another, and no gradient may overlap a written array (a block would
// read gradients another block is overwriting).  Gradients may overlap each other.
static int validate_segments(const neox_segment* segs, uint64_t nseg, bool need_v) {
    if (!segs) return set_error(NEOX_EINVAL, "segs is NULL");
    if (nseg == 0) return set_error(NEOX_EINVAL, "nseg is 0");
    if (nseg > (1u << 31)) return set_error(NEOX_EINVAL, "too many segments");
    struct Range { uintptr_t p; uint64_t bytes; uint64_t seg; };
    std::vector<Range> written, grads;
    try {
        written.reserve(nseg * (need_v ? 4 : 3));
        grads.reserve(nseg);
    } catch (const std::exception&) {
        return set_error(NEOX_ENOMEM, "host allocation of the overlap check (%llu segments)",
                         (unsigned long long)nseg);
    }
    for (uint64_t i = 0; i < nseg; ++i) {
        const neox_segment& s = segs[i];
        if (!s.grad || !s.half || !s.master || !s.exp_avg || (need_v && !s.exp_avg_sq))
            return set_error(NEOX_EINVAL, "segment %llu: null array", (unsigned long long)i);
        if (s.numel == 0) return set_error(NEOX_EINVAL, "segment %llu: numel is 0", (unsigned long long)i);
        if (s.numel > (UINT64_MAX >> 3)) return set_error(NEOX_EINVAL, "segment %llu: numel too large", (unsigned long long)i);
        if (((uintptr_t)s.grad & 1u) || ((uintptr_t)s.half & 1u))
            return set_error(NEOX_EINVAL, "segment %llu: grad/half not 2-byte aligned", (unsigned long long)i);
        if (((uintptr_t)s.master & 3u) || ((uintptr_t)s.exp_avg & 3u) || ((uintptr_t)s.exp_avg_sq & 3u))
            return set_error(NEOX_EINVAL, "segment %llu: FP32 array not 4-byte aligned", (unsigned long long)i);
        if (s.flags & ~NEOX_SEG_DECAY) return set_error(NEOX_EINVAL, "segment %llu: unknown flags", (unsigned long long)i);
        // capacity was reserved above, so these never allocate
        written.push_back({(uintptr_t)s.half, 2 * s.numel, i});
        written.push_back({(uintptr_t)s.master, 4 * s.numel, i});
        written.push_back({(uintptr_t)s.exp_avg, 4 * s.numel, i});
        if (need_v) written.push_back({(uintptr_t)s.exp_avg_sq, 4 * s.numel, i});
        grads.push_back({(uintptr_t)s.grad, 2 * s.numel, i});
    }
    // written arrays must not overlap each other (sorted sweep)
    auto by_start = [](const Range& a, const Range& b) { return a.p < b.p; };
    std::sort(written.begin(), written.end(), by_start);
    for (size_t k = 1; k < written.size(); ++k)
        if (overlaps(written[k - 1].p, written[k - 1].bytes, written[k].p, written[k].bytes))
            return set_error(NEOX_EINVAL, "segments %llu and %llu: written arrays overlap",
                             (unsigned long long)written[k - 1].seg, (unsigned long long)written[k].seg);
    // the written ranges are now disjoint and sorted by start, so of those starting before a
    // gradient's end the last one also ends last: it alone decides an overlap
    for (const Range& g : grads) {
        auto it = std::lower_bound(written.begin(), written.end(), g.p + g.bytes,
                                   [](const Range& r, uintptr_t end) { return r.p < end; });
        if (it == written.begin()) continue;
        const Range& r = *(it - 1);
        if (overlaps(r.p, r.bytes, g.p, g.bytes))
            return set_error(NEOX_EINVAL, "segment %llu: grad overlaps a written array of segment %llu",
                             (unsigned long long)g.seg, (unsigned long long)r.seg);
    }
    return NEOX_OK;
}

// ------------------------------------------------------------------------------------
// create / step / state / destroy
// ------------------------------------------------------------------------------------
static void free_handle(neox_zero1* h) {
    if (!h) return;
    for (auto& s : h->timing)
        for (auto& e : s.ev)
            if (e) (void)hipEventDestroy(e);
    if (h->d_chunks) (void)hipFree(h->d_chunks);
    if (h->d_norm_chunks) (void)hipFree(h->d_norm_chunks);
    if (h->d_seg_range) (void)hipFree(h->d_seg_range);
    if (h->d_seg_sumsq) (void)hipFree(h->d_seg_sumsq);
    if (h->d_partial) (void)hipFree(h->d_partial);
    if (h->d_state) (void)hipFree(h->d_state);
    if (h->d_tile_word) (void)hipFree(h->d_tile_word);
    if (h->d_change) (void)hipFree(h->d_change);
    delete h;
}

namespace nz1 {

int make_plan(const neox_zero1_config* cfg, const neox_segment* segs, uint64_t nseg, Plan& p,
              bool want_table) {
    if (!cfg) return set_error(NEOX_EINVAL, "cfg is NULL");
    int rc = validate_config(cfg);
    if (rc) return rc;
    rc = validate_segments(segs, nseg, cfg->optimizer == NEOX_OPT_ADAMW);
    if (rc) return rc;
    if (cfg->segment_norms && nseg >= (1u << 24))
        return set_error(NEOX_EINVAL, "segment_norms supports fewer than 2^24 segments");

    // update chunks of C elements; norm chunks of the smallest multiple of C that is at
    // least kNormChunk, or, on a small shard, at least numel / kNormTargetBlocks (so its
    // norm pass still spreads over the chip)
    p.C = cfg->chunk_elems ? cfg->chunk_elems : kDefaultChunk;
    for (uint64_t k = 0; k < nseg; ++k) p.numel += segs[k].numel;
    const bool has_v = cfg->optimizer == NEOX_OPT_ADAMW;
    uint64_t flat_n = 0;
    p.flat = !cfg->chunked_update && cfg->chunk_elems == 0 &&
             flat_layout(segs, nseg, has_v, &flat_n) &&
             (flat_n + kFlatTile - 1) / kFlatTile * kFlatBlock < (1ull << 32);
    const uint64_t spread = (p.numel + kNormTargetBlocks - 1) / kNormTargetBlocks;
    uint64_t target = spread < kNormChunk ? (spread > p.C ? spread : p.C) : kNormChunk;
    // Above that, a flat partition runs its norm pass as at most kFuseMaxParts large
    // blocks (one per CU, kNormBigBlock threads each), so that the update takes the step's
    // decisions itself and the finalize launch goes.  Its gradient is one contiguous array,
    // so the chunks cut it into kFuseMaxParts equal pieces whatever its segments -- unless
    // per-segment norms are asked for: then the chunks follow the segments, numel /
    // (kFuseMaxParts - nseg) elements each (each segment adds at most one short chunk), for
    // fewer than kFuseMaxParts / 2 segments.  A chunk holds at most NZ1_NORM_BIG_MAX_CHUNK
    // elements; a longer shard keeps the many short chunks.  Measured on MI355X, us per
    // step (short chunks and a finalize / large blocks): 215M 1115 / 1101, a Pythia-410M
    // rank 237 / 230, 64M 336 / 327, 16M 84.8 / 82.1, 24M 123.3 / 124.2; 6e9 31.53 / 31.15
    // ms (capped at 2^24 elements the 385 large blocks leave the chip half idle in a last
    // round: 31.7 ms); the 5,000-tensor list carved into one flat partition 5.41 / 5.36 ms.
    // Chunks across segments instead of along them: 6e9 norm pass 1.81 -> 1.77 ms, 215M
    // and a Pythia rank unchanged.  The chunk-table update reads its descriptor before its
    // data, so deciding there as well is slower on large grids (215M 1145 / 1345): other
    // layouts keep the finalize.
    const bool span = p.flat && !cfg->segment_norms;
    if (kUpdateDecides && p.flat && spread >= kNormChunk && (span || nseg < kFuseMaxParts / 2)) {
        const uint64_t parts = span ? kFuseMaxParts : kFuseMaxParts - nseg;
        const uint64_t few = ((p.numel + parts - 1) / parts + p.C - 1) / p.C * p.C;
        if (few <= (uint64_t)NZ1_NORM_BIG_MAX_CHUNK) {
            target = few;
            p.norm_big = true;
        }
    }
    const uint64_t C1_64 = (target + p.C - 1) / p.C * p.C;
    p.C1 = C1_64 > (p.norm_big ? (uint64_t)NZ1_NORM_BIG_MAX_CHUNK : (1u << 24)) ? p.C : (uint32_t)C1_64;
    p.nchunks = count_chunks(segs, nseg, p.C);
    // one block per chunk of the chunked update; the grid's x size in work-items is 32-bit
    if (!p.flat && p.nchunks >= (1ull << 24))
        return set_error(NEOX_EINVAL, "%llu chunks: raise chunk_elems", (unsigned long long)p.nchunks);
    try {
        if (!p.flat || want_table) build_chunks(segs, nseg, p.C, p.table);
        if (span) {
            // the whole gradient as one segment (the norm pass reads only the gradient)
            neox_segment whole = segs[0];
            whole.numel = flat_n;
            build_chunks(&whole, 1, p.C1, p.norm_table);
        } else {
            build_chunks(segs, nseg, p.C1, p.norm_table);
        }
    } catch (const std::exception&) {
        return set_error(NEOX_ENOMEM, "host allocation of the chunk table");
    }
#if NZ1_SORT_CHUNKS
    std::stable_sort(p.table.begin(), p.table.end(),
                     [](const Chunk& a, const Chunk& b) { return (uintptr_t)a.master < (uintptr_t)b.master; });
#endif

    if (p.flat) {
        try {
            build_flat_tables(segs, nseg, flat_n, p.tile_word, p.change);
        } catch (const std::exception&) {
            return set_error(NEOX_ENOMEM, "host allocation of the tile table");
        }
    }
    return NEOX_OK;
}

FinalizeArgs finalize_args(const neox_zero1_config& cfg) {
    FinalizeArgs f{};
    f.clip_norm = cfg.clip_norm;
    f.beta1 = cfg.beta1;
    f.beta2 = cfg.beta2;
    f.growth_factor = cfg.growth_factor;
    f.backoff_factor = cfg.backoff_factor;
    f.predivide_factor = cfg.predivide_factor;
    f.dp_world_size = (double)cfg.dp_world_size;
    f.min_scale = (float)cfg.min_scale;
    f.dynamic = cfg.scaler_mode == NEOX_SCALER_DYNAMIC;
    f.growth_interval = cfg.growth_interval;
    return f;
}

UpdateArgs update_args(const neox_zero1_config& cfg) {
    UpdateArgs u{};
    u.b1 = (float)cfg.beta1;
    u.omb1 = (float)(1.0 - cfg.beta1);
    u.b2 = (float)cfg.beta2;
    u.omb2 = (float)(1.0 - cfg.beta2);
    u.eps = (float)cfg.eps;
    u.wd = (float)cfg.weight_decay;
    u.lr = 0.0f;
    return u;
}

DevState initial_state(const neox_zero1_config& cfg, float scale, int32_t good_steps,
                       int64_t step, int64_t skipped, int32_t consecutive) {
    DevState st{};
    st.loss_scale = scale;
    st.good_steps = good_steps;
    st.step = step;
    st.skipped_total = skipped;
    st.consecutive_overflows = consecutive;
    st.last_skipped = 0;
    st.last_sumsq = 0.0;
    st.last_grad_norm = 0.0f;
    st.last_clip_coef = 1.0f;
    st.inv = unscale_factor(cfg.predivide_factor, (double)cfg.dp_world_size, scale);
    st.skip = 1;
    return st;
}

// Dynamic LDS to request so that exactly per_cu blocks of a kernel with `fixed` bytes of
// static LDS fit on a CU (0 = no cap).  A block's LDS is allocated in granules, so the
// total per block (static + dynamic) is made a multiple of 2 KiB, which every allocation
// granularity up to 2 KiB keeps as it is: per_cu such totals fit, per_cu + 1 do not.
static uint32_t reserve_for(int lds_per_cu, uint32_t per_cu, uint32_t fixed) {
    if (!per_cu) return 0u;
    const uint32_t total = ((uint32_t)lds_per_cu / per_cu) & ~2047u;
    return total > fixed ? total - fixed : 0u;
}

// Blocks per CU for an update grid of `blocks` blocks on `cus` CUs.
static uint32_t update_per_cu(uint64_t blocks, int cus, uint32_t long_grid) {
    const uint64_t per = (blocks + (uint64_t)cus - 1) / (uint64_t)cus;
    if (per <= NZ1_SHORT_GRID) return long_grid > 4u ? long_grid : 4u;
    return long_grid;
}

int lds_reserve(int device, int optimizer, uint64_t update_blocks, LdsReserve* out) {
    int lds_per_cu = 0, cus = 0;
    hipError_t e = hipDeviceGetAttribute(&lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                         device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return set_hip_error(e, "hipDeviceGetAttribute");
    if (cus < 1) cus = 1;
    uint32_t norm_fixed = 0, norm_big_fixed = 0;
    e = norm_static_lds(&norm_fixed, &norm_big_fixed);
    if (e != hipSuccess) return set_hip_error(e, "hipFuncGetAttributes");
    out->norm = reserve_for(lds_per_cu, NZ1_NORM_BLOCKS_PER_CU, norm_fixed);
    out->norm_big = reserve_for(lds_per_cu, 1, norm_big_fixed);   // one large block per CU
    // the update kernels declare no static LDS
    if (optimizer == NEOX_OPT_SGD) {
        // momentum SGD never takes 8 per CU (measured slower at every size: 16M elements
        // 66.8 against 64.5 us at 4 per CU)
        const uint64_t per = (update_blocks + (uint64_t)cus - 1) / (uint64_t)cus;
        const uint32_t sgd = per <= NZ1_SGD_SHORT_GRID ? NZ1_SGD_BLOCKS_PER_CU_SHORT
                                                       : NZ1_SGD_BLOCKS_PER_CU_LONG;
        out->update = reserve_for(lds_per_cu, sgd, 0);
        out->flat = reserve_for(lds_per_cu, sgd, 0);
    } else {
        out->update = reserve_for(lds_per_cu, update_per_cu(update_blocks, cus, NZ1_UPDATE_BLOCKS_PER_CU), 0);
        out->flat = reserve_for(lds_per_cu, update_per_cu(update_blocks, cus, NZ1_FLAT_BLOCKS_PER_CU), 0);
    }
    return NEOX_OK;
}

}  // namespace nz1

extern "C" int neox_zero1_plan(const neox_zero1_config* cfg, const neox_segment* segs, uint64_t nseg,
                               neox_zero1_plan_t* out, neox_chunk_info* chunks, uint64_t chunk_cap,
                               uint32_t* tile_words, uint64_t word_cap, uint32_t* changes,
                               uint64_t change_cap) {
    if (!out) return set_error(NEOX_EINVAL, "out is NULL");
    if ((chunk_cap && !chunks) || (word_cap && !tile_words) || (change_cap && !changes))
        return set_error(NEOX_EINVAL, "NULL table with a nonzero capacity");
    Plan p;
    const int rc = make_plan(cfg, segs, nseg, p, chunk_cap > 0);
    if (rc) return rc;
    std::memset(out, 0, sizeof *out);
    out->numel = p.numel;
    out->update_chunks = p.nchunks;
    out->norm_chunks = p.norm_table.size();
    out->flat_tiles = p.flat ? p.tile_word.size() - 1 : 0;
    out->flat_changes = p.change.size();
    out->chunk_elems = p.C;
    out->norm_chunk_elems = p.C1;
    out->tile_elems = kFlatTile;
    out->update_path = p.flat ? NEOX_PATH_FLAT : NEOX_PATH_CHUNKED;
    out->norm_block_threads = p.norm_big ? kNormBigBlock : kBlock;
    uint64_t nb = cfg->norm_blocks ? cfg->norm_blocks : p.norm_table.size();
    if (nb > p.norm_table.size()) nb = p.norm_table.size();
    out->update_decides = kUpdateDecides && nb <= kFuseMaxParts ? 1 : 0;
    for (uint64_t i = 0; i < chunk_cap && i < p.table.size(); ++i) {   // built when chunk_cap > 0
        const Chunk& c = p.table[i];
        const neox_segment& sg = segs[c.seg];
        chunks[i].offset = (uint64_t)(c.master - sg.master);
        chunks[i].seg = c.seg;
        chunks[i].len = c.len;
        chunks[i].flags = ((c.flags & CH_DECAY) ? NEOX_CHUNK_DECAY : 0u) |
                          ((c.flags & CH_VEC) ? NEOX_CHUNK_VEC : 0u);
        chunks[i].reserved = 0;
    }
    for (uint64_t i = 0; i < word_cap && i < p.tile_word.size(); ++i) tile_words[i] = p.tile_word[i];
    for (uint64_t i = 0; i < change_cap && i < p.change.size(); ++i) changes[i] = p.change[i];
    return NEOX_OK;
}

extern "C" int neox_zero1_create(const neox_zero1_config* cfg, const neox_segment* segs,
                                 uint64_t nseg, void* hip_stream, neox_zero1** out) {
    if (!out) return set_error(NEOX_EINVAL, "out is NULL");
    *out = nullptr;
    Plan plan;
    const int rc = make_plan(cfg, segs, nseg, plan);
    if (rc) return rc;
    std::vector<Chunk>& table = plan.table;
    std::vector<Chunk>& norm_table = plan.norm_table;
    std::vector<uint32_t>& tile_word = plan.tile_word;
    std::vector<uint32_t>& change = plan.change;
    const bool flat = plan.flat;
    const bool has_v = cfg->optimizer == NEOX_OPT_ADAMW;
    const uint64_t flat_n = plan.numel;

    neox_zero1* h = new (std::nothrow) neox_zero1();
    if (!h) return set_error(NEOX_ENOMEM, "host allocation of the handle");
    h->cfg = *cfg;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    StepLaunch& sl = h->sl;

    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) { free_handle(h); return set_hip_error(e, "hipGetDevice"); }
    int rc2 = lds_reserve(h->device, cfg->optimizer,
                          flat ? (uint64_t)tile_word.size() - 1 : (uint64_t)table.size(), &sl.lds);
    if (rc2) { free_handle(h); return rc2; }
    const uint32_t nnorm = (uint32_t)norm_table.size();
    // norm pass: one block per norm chunk unless a smaller striding grid is requested
    uint32_t nb = cfg->norm_blocks ? cfg->norm_blocks : nnorm;
    if (nb > nnorm) nb = nnorm;
    if (nb == 0) nb = 1;

    h->nseg = (uint32_t)nseg;
    std::vector<uint32_t> seg_range;
    if (cfg->segment_norms) {
        // norm chunks are built segment by segment, so each segment owns a contiguous range
        try {
            seg_range.assign(2 * nseg, 0);
        } catch (const std::exception&) {
            free_handle(h);
            return set_error(NEOX_ENOMEM, "host allocation of the segment ranges");
        }
        for (uint32_t c = 0; c < nnorm; ++c) {
            const uint32_t sg = norm_table[c].seg;
            if (c == 0 || norm_table[c - 1].seg != sg) seg_range[2 * sg] = c;
            seg_range[2 * sg + 1] = c + 1;
        }
    }

    // the update chunk table is uploaded only when the chunked update runs
    e = flat ? hipSuccess : hipMalloc(&h->d_chunks, table.size() * sizeof(Chunk));
    if (e == hipSuccess) e = hipMalloc(&h->d_norm_chunks, norm_table.size() * sizeof(Chunk));
    if (e == hipSuccess && cfg->segment_norms) e = hipMalloc(&h->d_seg_range, seg_range.size() * sizeof(uint32_t));
    if (e == hipSuccess && cfg->segment_norms) e = hipMalloc(&h->d_seg_sumsq, nseg * sizeof(double));
    if (e == hipSuccess) e = hipMalloc(&h->d_partial, nb * sizeof(double));
    if (e == hipSuccess) e = hipMalloc(&h->d_state, 2 * sizeof(DevState));
    if (e == hipSuccess && flat) e = hipMalloc(&h->d_tile_word, tile_word.size() * sizeof(uint32_t));
    if (e == hipSuccess && flat) e = hipMalloc(&h->d_change, (change.size() + 1) * sizeof(uint32_t));
    if (e != hipSuccess) {
        free_handle(h);
        return e == hipErrorOutOfMemory ? set_error(NEOX_ENOMEM, "hipMalloc of library scratch")
                                        : set_hip_error(e, "hipMalloc");
    }

    const DevState st[2] = {initial_state(*cfg, (float)cfg->init_scale, cfg->init_good_steps,
                                          cfg->init_step, cfg->init_skipped,
                                          cfg->init_consecutive_overflows),
                            DevState{}};

    if (!flat)
        e = hipMemcpyAsync(h->d_chunks, table.data(), table.size() * sizeof(Chunk), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(h->d_norm_chunks, norm_table.data(), norm_table.size() * sizeof(Chunk),
                           hipMemcpyHostToDevice, stream);
    if (e == hipSuccess && cfg->segment_norms)
        e = hipMemcpyAsync(h->d_seg_range, seg_range.data(), seg_range.size() * sizeof(uint32_t),
                           hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(h->d_state, st, sizeof st, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess && flat)
        e = hipMemcpyAsync(h->d_tile_word, tile_word.data(), tile_word.size() * sizeof(uint32_t),
                           hipMemcpyHostToDevice, stream);
    if (e == hipSuccess && flat && !change.empty())
        e = hipMemcpyAsync(h->d_change, change.data(), change.size() * sizeof(uint32_t),
                           hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) { free_handle(h); return set_hip_error(e, "upload of the chunk table"); }

    sl.dtype = cfg->dtype;
    sl.optimizer = cfg->optimizer;
    sl.norm_nt = plan.numel > kNormCachedMax;
    sl.norm_big = plan.norm_big;
    sl.norm_chunks = h->d_norm_chunks;
    sl.nnorm = nnorm;
    sl.norm_blocks = nb;
    sl.partial = h->d_partial;
    sl.st = h->d_state;
    sl.snap = h->d_state + 1;
    sl.fused = kUpdateDecides && nb <= kFuseMaxParts;
    sl.fin = finalize_args(*cfg);
    sl.upd = update_args(*cfg);
    sl.flat = flat;
    if (flat) {
        FlatSpan& sp = sl.span;
        sp.grad = static_cast<const uint16_t*>(segs[0].grad);
        sp.half = static_cast<uint16_t*>(segs[0].half);
        sp.master = segs[0].master;
        sp.m = segs[0].exp_avg;
        sp.v = has_v ? segs[0].exp_avg_sq : nullptr;
        sp.n = flat_n;
        sp.tile_word = h->d_tile_word;
        sp.change = h->d_change;
        sp.ntiles = (uint32_t)(tile_word.size() - 1);
    } else {
        sl.chunks = h->d_chunks;
        sl.nchunks = (uint32_t)table.size();
    }
    if (cfg->segment_norms) {
        sl.seg_range = h->d_seg_range;
        sl.seg_sumsq = h->d_seg_sumsq;
        sl.nseg = (uint32_t)nseg;
    }

    h->last_stream = stream;
    *out = h;
    return NEOX_OK;
}

namespace nz1 {

// norm pass (+ per-segment sums when enabled); with snap it also copies the pre-step
// state to s.snap, for an update that takes the step's decisions itself
static hipError_t enqueue_norm(const StepLaunch& s, bool snap, hipStream_t stream,
                               const KernelTiming& t) {
    hipError_t e = launch_norm(s.dtype, s.norm_nt, s.norm_big, s.norm_chunks, s.nnorm,
                               s.norm_blocks, s.st, s.partial, snap ? s.snap : nullptr,
                               s.norm_big ? s.lds.norm_big : s.lds.norm, stream, t);
    if (e == hipSuccess && s.seg_sumsq)
        e = launch_segment_sumsq(s.partial, s.seg_range, s.nseg, s.seg_sumsq, stream);
    return e;
}

static hipError_t enqueue_update(const StepLaunch& s, float lr, const FuseIn* fuse,
                                 hipStream_t stream, const KernelTiming& t) {
    UpdateArgs u = s.upd;
    u.lr = lr;
    if (s.flat)
        return launch_flat_update(s.dtype, s.optimizer, s.span, s.st, u, fuse, s.lds.flat, stream, t);
    return launch_update(s.dtype, s.optimizer, s.chunks, s.nchunks, s.st, u, fuse, s.lds.update,
                         stream, t);
}

hipError_t enqueue_step(const StepLaunch& s, float lr, hipStream_t stream, const KernelTiming* t3) {
    const KernelTiming none{};
    hipError_t e = enqueue_norm(s, s.fused, stream, t3 ? t3[0] : none);
    if (s.fused) {
        const FuseIn f{s.partial, s.norm_blocks, s.snap, s.st, s.fin};
        if (e == hipSuccess) e = enqueue_update(s, lr, &f, stream, t3 ? t3[2] : none);
    } else {
        if (e == hipSuccess) e = launch_finalize(s.partial, s.norm_blocks, s.st, s.fin, stream, t3 ? t3[1] : none);
        if (e == hipSuccess) e = enqueue_update(s, lr, nullptr, stream, t3 ? t3[2] : none);
    }
    return e;
}

bool split_update_decides(const StepLaunch& s, uint32_t nranks) {
    return kUpdateDecides && nranks <= kFuseMaxParts && (s.flat || s.fused);
}

hipError_t enqueue_update_only(const StepLaunch& s, float lr, hipStream_t stream) {
    return enqueue_update(s, lr, nullptr, stream, KernelTiming{});
}

}  // namespace nz1

extern "C" int neox_zero1_step(neox_zero1* h, float lr, void* hip_stream) {
    if (!h) return set_error(NEOX_EINVAL, "handle is NULL");
    if (!std::isfinite(lr)) return set_error(NEOX_EINVAL, "lr %g is not finite", (double)lr);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    TimingSlot* ts = nullptr;
    if (h->timing_used < (int64_t)h->timing.size()) ts = &h->timing[h->timing_used++];
    KernelTiming t3[3];
    if (ts && !h->timing_update_only) {
        t3[0] = {ts->ev[0], ts->ev[1]};
        t3[1] = {ts->ev[2], ts->ev[3]};
    }
    if (ts) t3[2] = {ts->ev[4], ts->ev[5]};
    const hipError_t e = enqueue_step(h->sl, lr, stream, ts ? t3 : nullptr);
    h->last_stream = stream;
    if (e != hipSuccess) return set_hip_error(e, "step launch");
    return NEOX_OK;
}

extern "C" int neox_zero1_step_local(neox_zero1* h, double* local_sumsq, void* hip_stream) {
    if (!h || !local_sumsq) return set_error(NEOX_EINVAL, "null argument");
    if ((uintptr_t)local_sumsq & 7u) return set_error(NEOX_EINVAL, "local_sumsq not 8-byte aligned");
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    hipError_t e = enqueue_norm(h->sl, true, stream, KernelTiming{});
    if (e == hipSuccess) e = launch_reduce(h->sl.partial, h->sl.norm_blocks, local_sumsq, stream);
    h->last_stream = stream;
    if (e != hipSuccess) return set_hip_error(e, "step_local launch");
    return NEOX_OK;
}

extern "C" int neox_zero1_step_apply(neox_zero1* h, const double* rank_sumsq, uint32_t nranks,
                                     float lr, void* hip_stream) {
    if (!h || !rank_sumsq) return set_error(NEOX_EINVAL, "null argument");
    if (nranks == 0 || nranks > (1u << 24)) return set_error(NEOX_EINVAL, "nranks %u not in [1, 2^24]", nranks);
    if ((uintptr_t)rank_sumsq & 7u) return set_error(NEOX_EINVAL, "rank_sumsq not 8-byte aligned");
    if (!std::isfinite(lr)) return set_error(NEOX_EINVAL, "lr %g is not finite", (double)lr);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    hipError_t e;
    if (split_update_decides(h->sl, nranks)) {
        // the update adds the ranks' values in the finalize's order and decides itself,
        // from the pre-step state the norm pass of step_local saved
        const FuseIn f{rank_sumsq, nranks, h->sl.snap, h->sl.st, h->sl.fin};
        e = enqueue_update(h->sl, lr, &f, stream, KernelTiming{});
    } else {
        e = launch_finalize(rank_sumsq, nranks, h->sl.st, h->sl.fin, stream);
        if (e == hipSuccess) e = enqueue_update_only(h->sl, lr, stream);
    }
    h->last_stream = stream;
    if (e != hipSuccess) return set_hip_error(e, "step_apply launch");
    return NEOX_OK;
}

extern "C" int neox_scaler_set(neox_zero1* h, const neox_scaler_state_t* st, void* hip_stream) {
    if (!h || !st) return set_error(NEOX_EINVAL, "null argument");
    if (!(std::isfinite(st->loss_scale) && st->loss_scale > 0.0f))
        return set_error(NEOX_EINVAL, "loss_scale %g", (double)st->loss_scale);
    if (st->good_steps < 0 || st->step < 0 || st->skipped_total < 0 || st->consecutive_overflows < 0)
        return set_error(NEOX_EINVAL, "negative counter");
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    hipError_t e = launch_set_state(h->d_state, st->loss_scale, st->good_steps, st->step,
                                    st->skipped_total, st->consecutive_overflows,
                                    h->sl.fin.predivide_factor, h->sl.fin.dp_world_size, stream);
    h->last_stream = stream;
    if (e != hipSuccess) return set_hip_error(e, "scaler_set launch");
    return NEOX_OK;
}

extern "C" int neox_zero1_segment_sumsq(neox_zero1* h, double* out, uint64_t nseg) {
    if (!h || !out) return set_error(NEOX_EINVAL, "null argument");
    if (!h->cfg.segment_norms) return set_error(NEOX_EINVAL, "handle created without segment_norms");
    if (nseg != h->nseg) return set_error(NEOX_EINVAL, "nseg %llu != %u", (unsigned long long)nseg, h->nseg);
    hipError_t e = hipStreamSynchronize(h->last_stream);
    if (e == hipSuccess) e = hipMemcpy(out, h->d_seg_sumsq, nseg * sizeof(double), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return set_hip_error(e, "segment_sumsq readback");
    return NEOX_OK;
}

extern "C" int neox_scaler_state(neox_zero1* h, neox_scaler_state_t* out) {
    if (!h || !out) return set_error(NEOX_EINVAL, "null argument");
    hipError_t e = hipStreamSynchronize(h->last_stream);
    if (e != hipSuccess) return set_hip_error(e, "hipStreamSynchronize");
    DevState st;
    e = hipMemcpy(&st, h->d_state, sizeof st, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return set_hip_error(e, "state readback");
    out->loss_scale = st.loss_scale;
    out->good_steps = st.good_steps;
    out->step = st.step;
    out->skipped_total = st.skipped_total;
    out->consecutive_overflows = st.consecutive_overflows;
    out->last_skipped = st.last_skipped;
    out->last_grad_norm = st.last_grad_norm;
    out->last_clip_coef = st.last_clip_coef;
    out->last_sumsq = st.last_sumsq;
    out->device_loss_scale = &h->d_state->loss_scale;
    return NEOX_OK;
}

extern "C" int neox_zero1_destroy(neox_zero1* h) {
    if (!h) return NEOX_OK;
    hipError_t e = hipStreamSynchronize(h->last_stream);
    free_handle(h);
    if (e != hipSuccess) return set_hip_error(e, "hipStreamSynchronize");
    return NEOX_OK;
}

static void clear_timing(neox_zero1* h) {
    for (auto& s : h->timing)
        for (auto& e : s.ev)
            if (e) (void)hipEventDestroy(e);
    h->timing.clear();
    h->timing_used = 0;
}

extern "C" int neox_zero1_timing_begin(neox_zero1* h, int32_t max_steps, int32_t update_only) {
    if (!h || max_steps < 1 || max_steps > 1000000 || update_only < 0 || update_only > 1)
        return set_error(NEOX_EINVAL, "bad timing request");
    clear_timing(h);
    h->timing_update_only = update_only != 0;
    try {
        h->timing.resize(max_steps);
    } catch (const std::bad_alloc&) {
        return set_error(NEOX_ENOMEM, "timing slots");
    }
    for (auto& s : h->timing)
        for (auto& e : s.ev) e = nullptr;
    for (auto& s : h->timing)
        for (auto& e : s.ev) {
            hipError_t r = hipEventCreateWithFlags(&e, NZ1_TIMING_EVENT_FLAGS);
            if (r != hipSuccess) {
                clear_timing(h);   // no half-made slots: later steps run untimed
                return set_hip_error(r, "hipEventCreate");
            }
        }
    return NEOX_OK;
}

extern "C" int neox_zero1_timing_end(neox_zero1* h, double* ms_sums, int64_t* steps,
                                     double* step_ms, int64_t step_cap) {
    if (!h || !ms_sums || !steps) return set_error(NEOX_EINVAL, "null argument");
    if (step_cap < 0 || (step_cap > 0 && !step_ms)) return set_error(NEOX_EINVAL, "bad step_ms / step_cap");
    ms_sums[0] = ms_sums[1] = ms_sums[2] = 0.0;
    const int first = h->timing_update_only ? 2 : 0;
    for (int64_t i = 0; i < h->timing_used; ++i) {
        auto& s = h->timing[i];
        hipError_t r = hipEventSynchronize(s.ev[5]);
        if (r != hipSuccess) return set_hip_error(r, "hipEventSynchronize");
        for (int k = first; k < 3; ++k) {
            if (k == 1 && h->sl.fused) continue;     // no finalize launch: its time is 0
            float ms = 0.0f;
            r = hipEventElapsedTime(&ms, s.ev[2 * k], s.ev[2 * k + 1]);
            if (r != hipSuccess) return set_hip_error(r, "hipEventElapsedTime");
            ms_sums[k] += ms;
        }
        if (i < step_cap) {
            // the step: from its first timed kernel's start to the update's end
            float ms = 0.0f;
            r = hipEventElapsedTime(&ms, s.ev[2 * first], s.ev[5]);
            if (r != hipSuccess) return set_hip_error(r, "hipEventElapsedTime");
            step_ms[i] = ms;
        }
    }
    *steps = h->timing_used;
    clear_timing(h);
    return NEOX_OK;
}

extern "C" int neox_zero1_update_path(const neox_zero1* h) {
    if (!h) return set_error(NEOX_EINVAL, "handle is NULL");
    return h->sl.flat ? NEOX_PATH_FLAT : NEOX_PATH_CHUNKED;
}

extern "C" const char* neox_zero1_last_error(void) { return g_last_error.c_str(); }
