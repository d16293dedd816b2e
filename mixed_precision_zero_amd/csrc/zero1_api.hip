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

namespace {

thread_local std::string g_last_error = "no error";

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(NEOX_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

// Work-unit sizes (elements), measured best on MI355X: the update wants small blocks
// (2,048 elements: 128 threads x two 16-byte vectors per array) at 2 blocks per CU, the
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
#ifndef NZ1_NORM_BLOCKS_PER_CU
#define NZ1_NORM_BLOCKS_PER_CU 4
#endif
#ifndef NZ1_FLAT_BLOCKS_PER_CU
#define NZ1_FLAT_BLOCKS_PER_CU 2
#endif
// momentum SGD moves 20 B/param over seven streams and prefers more blocks in flight
#ifndef NZ1_FLAT_BLOCKS_PER_CU_SGD
#define NZ1_FLAT_BLOCKS_PER_CU_SGD 4
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
    uint32_t nchunks = 0;          // update work units
    uint32_t nnorm = 0;            // norm-pass work units
    uint32_t norm_blocks = 0;
    uint32_t update_lds = 0;       // LDS reserved per update block (occupancy cap)
    uint32_t norm_lds = 0;         // LDS reserved per norm block
    uint32_t flat_lds = 0;         // LDS reserved per flat-update block
    bool flat = false;             // update runs flat_update_kernel over `span`
    FlatSpan span{};
    uint32_t* d_tile_word = nullptr;
    uint32_t* d_change = nullptr;
    Chunk* d_chunks = nullptr;
    Chunk* d_norm_chunks = nullptr;
    uint32_t nseg = 0;
    uint32_t* d_seg_range = nullptr;   // per segment: [first, end) norm chunk (telemetry)
    double* d_seg_sumsq = nullptr;     // per segment squared norm of the last step
    double* d_partial = nullptr;
    DevState* d_state = nullptr;
    hipStream_t last_stream = nullptr;
    FinalizeArgs fin{};
    UpdateArgs upd_base{};
    // profiling
    std::vector<TimingSlot> timing;
    int64_t timing_used = 0;
    bool timing_update_only = false;
};

// ------------------------------------------------------------------------------------
// configuration
// ------------------------------------------------------------------------------------
extern "C" int neox_zero1_default_config(neox_zero1_config* cfg) {
    if (!cfg) return fail(NEOX_EINVAL, "cfg is NULL");
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
    if (!(c->beta1 >= 0.0 && c->beta1 < 1.0)) return fail(NEOX_EINVAL, "beta1 %g not in [0,1)", c->beta1);
    if (!(c->beta2 >= 0.0 && c->beta2 < 1.0)) return fail(NEOX_EINVAL, "beta2 %g not in [0,1)", c->beta2);
    if (!(std::isfinite(c->eps) && c->eps >= 0.0)) return fail(NEOX_EINVAL, "eps %g", c->eps);
    if (!(std::isfinite(c->weight_decay) && c->weight_decay >= 0.0))
        return fail(NEOX_EINVAL, "weight_decay %g", c->weight_decay);
    if (std::isnan(c->clip_norm) || std::isinf(c->clip_norm))
        return fail(NEOX_EINVAL, "clip_norm %g", c->clip_norm);
    if (!finite_pos(c->predivide_factor)) return fail(NEOX_EINVAL, "predivide_factor %g", c->predivide_factor);
    if (c->dp_world_size < 1) return fail(NEOX_EINVAL, "dp_world_size %d", c->dp_world_size);
    if (c->dtype != NEOX_F16 && c->dtype != NEOX_BF16) return fail(NEOX_EINVAL, "dtype %d", c->dtype);
    if (c->scaler_mode != NEOX_SCALER_DYNAMIC && c->scaler_mode != NEOX_SCALER_STATIC)
        return fail(NEOX_EINVAL, "scaler_mode %d", c->scaler_mode);
    if (c->growth_interval < 1) return fail(NEOX_EINVAL, "growth_interval %d", c->growth_interval);
    if (!finite_pos(c->init_scale) || !std::isfinite((float)c->init_scale) || (float)c->init_scale <= 0.0f)
        return fail(NEOX_EINVAL, "init_scale %g", c->init_scale);
    if (!(std::isfinite(c->growth_factor) && c->growth_factor >= 1.0))
        return fail(NEOX_EINVAL, "growth_factor %g", c->growth_factor);
    if (!(c->backoff_factor > 0.0 && c->backoff_factor <= 1.0))
        return fail(NEOX_EINVAL, "backoff_factor %g", c->backoff_factor);
    if (!finite_pos(c->min_scale) || (float)c->min_scale <= 0.0f || !std::isfinite((float)c->min_scale))
        return fail(NEOX_EINVAL, "min_scale %g", c->min_scale);
    if (c->init_step < 0 || c->init_skipped < 0 || c->init_good_steps < 0 ||
        c->init_consecutive_overflows < 0)
        return fail(NEOX_EINVAL, "negative resume counter");
    if (c->chunk_elems != 0 &&
        (c->chunk_elems % kVec != 0 || c->chunk_elems < 256 || c->chunk_elems > (1u << 24)))
        return fail(NEOX_EINVAL, "chunk_elems %u: multiple of 8 in [256, 2^24]", c->chunk_elems);
    if (c->norm_blocks > (1u << 20)) return fail(NEOX_EINVAL, "norm_blocks %u too large", c->norm_blocks);
    if (c->optimizer != NEOX_OPT_ADAMW && c->optimizer != NEOX_OPT_SGD)
        return fail(NEOX_EINVAL, "optimizer %d", c->optimizer);
    if (c->segment_norms > 1) return fail(NEOX_EINVAL, "segment_norms %u", c->segment_norms);
    if (c->chunked_update > 1) return fail(NEOX_EINVAL, "chunked_update %u", c->chunked_update);
    if (c->segment_norms && c->norm_blocks)
        return fail(NEOX_EINVAL, "segment_norms needs the one-block-per-chunk norm pass (norm_blocks 0)");
    return NEOX_OK;
}

// ------------------------------------------------------------------------------------
// shard partition: interval intersection of each tensor with the rank's range
// ------------------------------------------------------------------------------------
extern "C" int neox_zero1_partition(const uint64_t* tensor_numel, const uint8_t* tensor_decay,
                                    uint64_t ntensors, uint32_t dp_world_size, uint32_t rank,
                                    uint32_t align, neox_shard_segment* out, uint64_t cap,
                                    uint64_t* nseg_out, uint64_t* shard_numel_out) {
    if (!nseg_out || !shard_numel_out) return fail(NEOX_EINVAL, "null output pointer");
    if (ntensors && (!tensor_numel || !tensor_decay)) return fail(NEOX_EINVAL, "null tensor list");
    if (cap && !out) return fail(NEOX_EINVAL, "out is NULL with cap > 0");
    if (dp_world_size == 0 || align == 0) return fail(NEOX_EINVAL, "dp_world_size and align must be >= 1");
    if (rank >= dp_world_size) return fail(NEOX_EINVAL, "rank %u >= dp_world_size %u", rank, dp_world_size);
    uint64_t total = 0;
    for (uint64_t i = 0; i < ntensors; ++i) {
        if (tensor_numel[i] > UINT64_MAX - total) return fail(NEOX_EINVAL, "total numel overflows");
        total += tensor_numel[i];
    }
    const unsigned __int128 unit = (unsigned __int128)dp_world_size * align;
    const unsigned __int128 padded128 = ((unsigned __int128)total + unit - 1) / unit * unit;
    if (padded128 > UINT64_MAX) return fail(NEOX_EINVAL, "padded numel overflows");
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

static void build_chunks(const neox_segment* segs, uint64_t nseg, uint32_t C, std::vector<Chunk>& t) {
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

static int validate_segments(const neox_segment* segs, uint64_t nseg, bool need_v) {
    if (!segs) return fail(NEOX_EINVAL, "segs is NULL");
    if (nseg == 0) return fail(NEOX_EINVAL, "nseg is 0");
    if (nseg > (1u << 31)) return fail(NEOX_EINVAL, "too many segments");
    struct Range { uintptr_t p; uint64_t bytes; uint64_t seg; };
    std::vector<Range> ranges;
    ranges.reserve(nseg * 5);
    for (uint64_t i = 0; i < nseg; ++i) {
        const neox_segment& s = segs[i];
        if (!s.grad || !s.half || !s.master || !s.exp_avg || (need_v && !s.exp_avg_sq))
            return fail(NEOX_EINVAL, "segment %llu: null array", (unsigned long long)i);
        if (s.numel == 0) return fail(NEOX_EINVAL, "segment %llu: numel is 0", (unsigned long long)i);
        if (s.numel > (UINT64_MAX >> 3)) return fail(NEOX_EINVAL, "segment %llu: numel too large", (unsigned long long)i);
        if (((uintptr_t)s.grad & 1u) || ((uintptr_t)s.half & 1u))
            return fail(NEOX_EINVAL, "segment %llu: grad/half not 2-byte aligned", (unsigned long long)i);
        if (((uintptr_t)s.master & 3u) || ((uintptr_t)s.exp_avg & 3u) || ((uintptr_t)s.exp_avg_sq & 3u))
            return fail(NEOX_EINVAL, "segment %llu: FP32 array not 4-byte aligned", (unsigned long long)i);
        if (s.flags & ~NEOX_SEG_DECAY) return fail(NEOX_EINVAL, "segment %llu: unknown flags", (unsigned long long)i);
        ranges.push_back({(uintptr_t)s.half, 2 * s.numel, i});
        ranges.push_back({(uintptr_t)s.master, 4 * s.numel, i});
        ranges.push_back({(uintptr_t)s.exp_avg, 4 * s.numel, i});
        if (need_v) ranges.push_back({(uintptr_t)s.exp_avg_sq, 4 * s.numel, i});
    }
    // written arrays must not overlap each other (sorted sweep)
    std::sort(ranges.begin(), ranges.end(), [](const Range& a, const Range& b) { return a.p < b.p; });
    for (size_t k = 1; k < ranges.size(); ++k)
        if (overlaps(ranges[k - 1].p, ranges[k - 1].bytes, ranges[k].p, ranges[k].bytes))
            return fail(NEOX_EINVAL, "segments %llu and %llu: written arrays overlap",
                        (unsigned long long)ranges[k - 1].seg, (unsigned long long)ranges[k].seg);
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

// The work decomposition of a segment list: what create() uploads and neox_zero1_plan()
// describes.  Validates the config and the segments first.
struct Plan {
    uint32_t C = 0;                        // update chunk length
    uint32_t C1 = 0;                       // norm chunk length
    std::vector<Chunk> table, norm_table;  // update and norm work tables
    bool flat = false;                     // flat partition: the update runs over tiles
    uint64_t numel = 0;
    std::vector<uint32_t> tile_word, change;
};

static int make_plan(const neox_zero1_config* cfg, const neox_segment* segs, uint64_t nseg,
                     Plan& p) {
    if (!cfg) return fail(NEOX_EINVAL, "cfg is NULL");
    int rc = validate_config(cfg);
    if (rc) return rc;
    rc = validate_segments(segs, nseg, cfg->optimizer == NEOX_OPT_ADAMW);
    if (rc) return rc;
    if (cfg->segment_norms && nseg >= (1u << 24))
        return fail(NEOX_EINVAL, "segment_norms supports fewer than 2^24 segments");

    // update chunks of C elements; norm chunks of the smallest multiple of C that is
    // at least kNormChunk
    p.C = cfg->chunk_elems ? cfg->chunk_elems : kDefaultChunk;
    const uint64_t C1_64 = p.C >= kNormChunk ? p.C : (uint64_t)(kNormChunk + p.C - 1) / p.C * p.C;
    p.C1 = C1_64 > (1u << 24) ? p.C : (uint32_t)C1_64;
    for (uint64_t k = 0; k < nseg; ++k) p.numel += segs[k].numel;
    try {
        build_chunks(segs, nseg, p.C, p.table);
        build_chunks(segs, nseg, p.C1, p.norm_table);
    } catch (const std::bad_alloc&) {
        return fail(NEOX_ENOMEM, "host allocation of the chunk table");
    }
    // one block per chunk; the grid's x size in work-items is 32-bit
    if (p.table.size() >= (1ull << 24)) return fail(NEOX_EINVAL, "%zu chunks: raise chunk_elems", p.table.size());

    const bool has_v = cfg->optimizer == NEOX_OPT_ADAMW;
    uint64_t flat_n = 0;
    p.flat = !cfg->chunked_update && cfg->chunk_elems == 0 &&
             flat_layout(segs, nseg, has_v, &flat_n) &&
             (flat_n + kFlatTile - 1) / kFlatTile * kFlatBlock < (1ull << 32);
    if (p.flat) {
        try {
            build_flat_tables(segs, nseg, flat_n, p.tile_word, p.change);
        } catch (const std::bad_alloc&) {
            return fail(NEOX_ENOMEM, "host allocation of the tile table");
        }
    }
    return NEOX_OK;
}

extern "C" int neox_zero1_plan(const neox_zero1_config* cfg, const neox_segment* segs, uint64_t nseg,
                               neox_zero1_plan_t* out, neox_chunk_info* chunks, uint64_t chunk_cap,
                               uint32_t* tile_words, uint64_t word_cap, uint32_t* changes,
                               uint64_t change_cap) {
    if (!out) return fail(NEOX_EINVAL, "out is NULL");
    if ((chunk_cap && !chunks) || (word_cap && !tile_words) || (change_cap && !changes))
        return fail(NEOX_EINVAL, "NULL table with a nonzero capacity");
    Plan p;
    const int rc = make_plan(cfg, segs, nseg, p);
    if (rc) return rc;
    std::memset(out, 0, sizeof *out);
    out->numel = p.numel;
    out->update_chunks = p.table.size();
    out->norm_chunks = p.norm_table.size();
    out->flat_tiles = p.flat ? p.tile_word.size() - 1 : 0;
    out->flat_changes = p.change.size();
    out->chunk_elems = p.C;
    out->norm_chunk_elems = p.C1;
    out->tile_elems = kFlatTile;
    out->update_path = p.flat ? NEOX_PATH_FLAT : NEOX_PATH_CHUNKED;
    for (uint64_t i = 0; i < chunk_cap && i < p.table.size(); ++i) {
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
    if (!out) return fail(NEOX_EINVAL, "out is NULL");
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
    if (!h) return fail(NEOX_ENOMEM, "host allocation of the handle");
    h->cfg = *cfg;
    h->nchunks = (uint32_t)table.size();
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);

    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) { free_handle(h); return hip_fail(e, "hipGetDevice"); }
    int lds_per_cu = 0;
    e = hipDeviceGetAttribute(&lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              h->device);
    if (e != hipSuccess) { free_handle(h); return hip_fail(e, "hipDeviceGetAttribute"); }
    auto reserve = [&](uint32_t per_cu) -> uint32_t {
        return per_cu ? (uint32_t)(lds_per_cu / per_cu) & ~1023u : 0u;
    };
    h->update_lds = reserve(NZ1_UPDATE_BLOCKS_PER_CU);
    h->norm_lds = reserve(NZ1_NORM_BLOCKS_PER_CU);
    h->flat_lds = reserve(cfg->optimizer == NEOX_OPT_SGD ? NZ1_FLAT_BLOCKS_PER_CU_SGD
                                                         : NZ1_FLAT_BLOCKS_PER_CU);
    h->nnorm = (uint32_t)norm_table.size();
    // norm pass: one block per norm chunk unless a smaller striding grid is requested
    uint32_t nb = cfg->norm_blocks ? cfg->norm_blocks : h->nnorm;
    if (nb > h->nnorm) nb = h->nnorm;
    if (nb == 0) nb = 1;
    h->norm_blocks = nb;

    h->nseg = (uint32_t)nseg;
    std::vector<uint32_t> seg_range;
    if (cfg->segment_norms) {
        // norm chunks are built segment by segment, so each segment owns a contiguous range
        seg_range.assign(2 * nseg, 0);
        for (uint32_t c = 0; c < h->nnorm; ++c) {
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
    if (e == hipSuccess) e = hipMalloc(&h->d_state, sizeof(DevState));
    if (e == hipSuccess && flat) e = hipMalloc(&h->d_tile_word, tile_word.size() * sizeof(uint32_t));
    if (e == hipSuccess && flat) e = hipMalloc(&h->d_change, (change.size() + 1) * sizeof(uint32_t));
    if (e != hipSuccess) {
        free_handle(h);
        return e == hipErrorOutOfMemory ? fail(NEOX_ENOMEM, "hipMalloc of library scratch")
                                        : hip_fail(e, "hipMalloc");
    }

    DevState st{};
    st.loss_scale = (float)cfg->init_scale;
    st.good_steps = cfg->init_good_steps;
    st.step = cfg->init_step;
    st.skipped_total = cfg->init_skipped;
    st.consecutive_overflows = cfg->init_consecutive_overflows;
    st.last_skipped = 0;
    st.last_sumsq = 0.0;
    st.last_grad_norm = 0.0f;
    st.last_clip_coef = 1.0f;
    st.inv = unscale_factor(cfg->predivide_factor, (double)cfg->dp_world_size, st.loss_scale);
    st.skip = 1;

    if (!flat)
        e = hipMemcpyAsync(h->d_chunks, table.data(), table.size() * sizeof(Chunk), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(h->d_norm_chunks, norm_table.data(), norm_table.size() * sizeof(Chunk),
                           hipMemcpyHostToDevice, stream);
    if (e == hipSuccess && cfg->segment_norms)
        e = hipMemcpyAsync(h->d_seg_range, seg_range.data(), seg_range.size() * sizeof(uint32_t),
                           hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(h->d_state, &st, sizeof st, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess && flat)
        e = hipMemcpyAsync(h->d_tile_word, tile_word.data(), tile_word.size() * sizeof(uint32_t),
                           hipMemcpyHostToDevice, stream);
    if (e == hipSuccess && flat && !change.empty())
        e = hipMemcpyAsync(h->d_change, change.data(), change.size() * sizeof(uint32_t),
                           hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) { free_handle(h); return hip_fail(e, "upload of the chunk table"); }

    FinalizeArgs& f = h->fin;
    f.clip_norm = cfg->clip_norm;
    f.beta1 = cfg->beta1;
    f.beta2 = cfg->beta2;
    f.growth_factor = cfg->growth_factor;
    f.backoff_factor = cfg->backoff_factor;
    f.predivide_factor = cfg->predivide_factor;
    f.dp_world_size = (double)cfg->dp_world_size;
    f.min_scale = (float)cfg->min_scale;
    f.dynamic = cfg->scaler_mode == NEOX_SCALER_DYNAMIC;
    f.growth_interval = cfg->growth_interval;

    if (flat) {
        h->flat = true;
        FlatSpan& sp = h->span;
        sp.grad = static_cast<const uint16_t*>(segs[0].grad);
        sp.half = static_cast<uint16_t*>(segs[0].half);
        sp.master = segs[0].master;
        sp.m = segs[0].exp_avg;
        sp.v = has_v ? segs[0].exp_avg_sq : nullptr;
        sp.n = flat_n;
        sp.tile_word = h->d_tile_word;
        sp.change = h->d_change;
        sp.ntiles = (uint32_t)(tile_word.size() - 1);
    }

    UpdateArgs& u = h->upd_base;
    u.b1 = (float)cfg->beta1;
    u.omb1 = (float)(1.0 - cfg->beta1);
    u.b2 = (float)cfg->beta2;
    u.omb2 = (float)(1.0 - cfg->beta2);
    u.eps = (float)cfg->eps;
    u.wd = (float)cfg->weight_decay;
    u.lr = 0.0f;

    h->last_stream = stream;
    *out = h;
    return NEOX_OK;
}

// norm pass (+ per-segment sums when enabled)
static hipError_t enqueue_norm(neox_zero1* h, hipStream_t stream, const KernelTiming& t = {}) {
    hipError_t e = launch_norm(h->cfg.dtype, h->d_norm_chunks, h->nnorm, h->norm_blocks,
                               h->d_state, h->d_partial, h->norm_lds, stream, t);
    if (e == hipSuccess && h->cfg.segment_norms)
        e = launch_segment_sumsq(h->d_partial, h->d_seg_range, h->nseg, h->d_seg_sumsq, stream);
    return e;
}

static hipError_t enqueue_update(neox_zero1* h, float lr, hipStream_t stream,
                                 const KernelTiming& t = {}) {
    UpdateArgs u = h->upd_base;
    u.lr = lr;
    if (h->flat)
        return launch_flat_update(h->cfg.dtype, h->cfg.optimizer, h->span, h->d_state, u,
                                  h->flat_lds, stream, t);
    return launch_update(h->cfg.dtype, h->cfg.optimizer, h->d_chunks, h->nchunks, h->d_state, u,
                         h->update_lds, stream, t);
}

extern "C" int neox_zero1_step(neox_zero1* h, float lr, void* hip_stream) {
    if (!h) return fail(NEOX_EINVAL, "handle is NULL");
    if (!std::isfinite(lr)) return fail(NEOX_EINVAL, "lr %g is not finite", (double)lr);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    TimingSlot* ts = nullptr;
    if (h->timing_used < (int64_t)h->timing.size()) ts = &h->timing[h->timing_used++];

    const bool all = ts && !h->timing_update_only;
    KernelTiming tn, tf, tu;
    if (all) {
        tn = {ts->ev[0], ts->ev[1]};
        tf = {ts->ev[2], ts->ev[3]};
    }
    if (ts) tu = {ts->ev[4], ts->ev[5]};
    hipError_t e = enqueue_norm(h, stream, tn);
    if (e == hipSuccess)
        e = launch_finalize(h->d_partial, h->norm_blocks, nullptr, h->d_state, h->fin, stream, tf);
    if (e == hipSuccess) e = enqueue_update(h, lr, stream, tu);
    h->last_stream = stream;
    if (e != hipSuccess) return hip_fail(e, "step launch");
    return NEOX_OK;
}

extern "C" int neox_zero1_step_local(neox_zero1* h, double* local_sumsq, void* hip_stream) {
    if (!h || !local_sumsq) return fail(NEOX_EINVAL, "null argument");
    if ((uintptr_t)local_sumsq & 7u) return fail(NEOX_EINVAL, "local_sumsq not 8-byte aligned");
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    hipError_t e = enqueue_norm(h, stream);
    if (e == hipSuccess) e = launch_reduce(h->d_partial, h->norm_blocks, local_sumsq, stream);
    h->last_stream = stream;
    if (e != hipSuccess) return hip_fail(e, "step_local launch");
    return NEOX_OK;
}

extern "C" int neox_zero1_step_apply(neox_zero1* h, const double* global_sumsq, float lr,
                                     void* hip_stream) {
    if (!h || !global_sumsq) return fail(NEOX_EINVAL, "null argument");
    if ((uintptr_t)global_sumsq & 7u) return fail(NEOX_EINVAL, "global_sumsq not 8-byte aligned");
    if (!std::isfinite(lr)) return fail(NEOX_EINVAL, "lr %g is not finite", (double)lr);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    hipError_t e = launch_finalize(nullptr, 0, global_sumsq, h->d_state, h->fin, stream);
    if (e == hipSuccess) e = enqueue_update(h, lr, stream);
    h->last_stream = stream;
    if (e != hipSuccess) return hip_fail(e, "step_apply launch");
    return NEOX_OK;
}

extern "C" int neox_scaler_set(neox_zero1* h, const neox_scaler_state_t* st, void* hip_stream) {
    if (!h || !st) return fail(NEOX_EINVAL, "null argument");
    if (!(std::isfinite(st->loss_scale) && st->loss_scale > 0.0f))
        return fail(NEOX_EINVAL, "loss_scale %g", (double)st->loss_scale);
    if (st->good_steps < 0 || st->step < 0 || st->skipped_total < 0 || st->consecutive_overflows < 0)
        return fail(NEOX_EINVAL, "negative counter");
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    hipError_t e = launch_set_state(h->d_state, st->loss_scale, st->good_steps, st->step,
                                    st->skipped_total, st->consecutive_overflows,
                                    h->fin.predivide_factor, h->fin.dp_world_size, stream);
    h->last_stream = stream;
    if (e != hipSuccess) return hip_fail(e, "scaler_set launch");
    return NEOX_OK;
}

extern "C" int neox_zero1_segment_sumsq(neox_zero1* h, double* out, uint64_t nseg) {
    if (!h || !out) return fail(NEOX_EINVAL, "null argument");
    if (!h->cfg.segment_norms) return fail(NEOX_EINVAL, "handle created without segment_norms");
    if (nseg != h->nseg) return fail(NEOX_EINVAL, "nseg %llu != %u", (unsigned long long)nseg, h->nseg);
    hipError_t e = hipStreamSynchronize(h->last_stream);
    if (e == hipSuccess) e = hipMemcpy(out, h->d_seg_sumsq, nseg * sizeof(double), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "segment_sumsq readback");
    return NEOX_OK;
}

extern "C" int neox_scaler_state(neox_zero1* h, neox_scaler_state_t* out) {
    if (!h || !out) return fail(NEOX_EINVAL, "null argument");
    hipError_t e = hipStreamSynchronize(h->last_stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    DevState st;
    e = hipMemcpy(&st, h->d_state, sizeof st, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "state readback");
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
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
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
        return fail(NEOX_EINVAL, "bad timing request");
    clear_timing(h);
    h->timing_update_only = update_only != 0;
    try {
        h->timing.resize(max_steps);
    } catch (const std::bad_alloc&) {
        return fail(NEOX_ENOMEM, "timing slots");
    }
    for (auto& s : h->timing)
        for (auto& e : s.ev) e = nullptr;
    for (auto& s : h->timing)
        for (auto& e : s.ev) {
            hipError_t r = hipEventCreateWithFlags(&e, NZ1_TIMING_EVENT_FLAGS);
            if (r != hipSuccess) {
                clear_timing(h);   // no half-made slots: later steps run untimed
                return hip_fail(r, "hipEventCreate");
            }
        }
    return NEOX_OK;
}

extern "C" int neox_zero1_timing_end(neox_zero1* h, double* ms_sums, int64_t* steps) {
    if (!h || !ms_sums || !steps) return fail(NEOX_EINVAL, "null argument");
    ms_sums[0] = ms_sums[1] = ms_sums[2] = 0.0;
    for (int64_t i = 0; i < h->timing_used; ++i) {
        auto& s = h->timing[i];
        hipError_t r = hipEventSynchronize(s.ev[5]);
        if (r != hipSuccess) return hip_fail(r, "hipEventSynchronize");
        for (int k = h->timing_update_only ? 2 : 0; k < 3; ++k) {
            float ms = 0.0f;
            r = hipEventElapsedTime(&ms, s.ev[2 * k], s.ev[2 * k + 1]);
            if (r != hipSuccess) return hip_fail(r, "hipEventElapsedTime");
            ms_sums[k] += ms;
        }
    }
    *steps = h->timing_used;
    clear_timing(h);
    return NEOX_OK;
}

extern "C" int neox_zero1_update_path(const neox_zero1* h) {
    if (!h) return fail(NEOX_EINVAL, "handle is NULL");
    return h->flat ? NEOX_PATH_FLAT : NEOX_PATH_CHUNKED;
}

extern "C" const char* neox_zero1_last_error(void) { return g_last_error.c_str(); }
