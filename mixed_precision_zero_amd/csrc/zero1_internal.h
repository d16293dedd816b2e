// zero1_internal.h -- types shared by the host side and the gfx950 kernels of the
// ZeRO-1 mixed-precision Adam step.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nz1 {

constexpr int kBlock = 256;   // threads per block of the norm, finalize and telemetry kernels
// Threads per block of the norm pass when it runs as at most kFuseMaxParts large blocks
// (one per CU) so that the update can take the step's decisions itself; see make_plan.
// Measured on MI355X (215M-element shard, same process, us per norm pass): 256 threads
// 103, 512 65.6-66.2, 768 65.7-67.0, 1,024 67.4-67.9; 512 with 12 or 16 loads in flight
// per thread 64.9-65.4 or 122 (a Pythia-410M rank: 512 16.3-17.0, 1,024 16.9-17.9, 512
// with 12 loads 18.4-19.1).
#ifndef NZ1_NORM_BIG_BLOCK
#define NZ1_NORM_BIG_BLOCK 512
#endif
constexpr int kNormBigBlock = NZ1_NORM_BIG_BLOCK;
constexpr int kVec = 8;       // elements per thread-vector: one 16-byte load of halves

enum : uint32_t {
    CH_DECAY = 1u,   // elements of this chunk receive decoupled weight decay
    CH_VEC = 2u,     // all five arrays are 16-byte aligned at the chunk start
};

// One unit of work: up to chunk_elems consecutive elements of one segment.  The five
// pointers already point at the chunk's first element, so a block needs a single
// 64-byte scalar load to find its work.
struct alignas(64) Chunk {
    const uint16_t* grad;
    uint16_t* half;
    float* master;
    float* m;
    float* v;
    uint32_t len;
    uint32_t flags;
    uint32_t seg;
    uint32_t pad_;
};
static_assert(sizeof(Chunk) == 64, "Chunk is one 64-byte scalar load");

// Device-resident step state.  The host never needs to know whether a step was
// skipped: the finalize kernel writes the decision here and the update kernel reads it.
struct alignas(64) DevState {
    // persistent scaler / optimizer counters
    float loss_scale;            // scale the next gradient carries
    int32_t good_steps;
    int64_t step;                // applied steps t
    int64_t skipped_total;
    int32_t consecutive_overflows;
    int32_t last_skipped;
    double last_sumsq;
    float last_grad_norm;
    float last_clip_coef;
    // handed from the finalize to the passes
    float inv;                   // fp32(f / (D * S)) for the next norm pass
    int32_t pad_[3];
    // what the update reads, in one 16-byte block (one scalar load in the chunked update)
    int32_t skip;                // this step's decision
    float gscale;                // this step's unscale factor times clip coefficient
    float rbc1;                  // 1 / (1 - beta1^t)
    float rsbc2;                 // 1 / sqrt(1 - beta2^t)
};
static_assert(offsetof(DevState, skip) % 16 == 0, "update fields share one 16-byte load");

// Flat layout: the segments, in order, tile five contiguous arrays whose first elements
// are 16-byte aligned.  Work unit: one tile of kFlatTile elements per block.  Measured
// best on MI355X: 128 threads x 2 vectors (2,048-element tiles) at 2 blocks per CU on
// long grids; fewer tiles in flight per CU keep the chip's open DRAM rows few, and the
// block's single round trip keeps that low occupancy from exposing latency.  (Grids of
// up to 48 blocks per CU, 64 for momentum SGD, run 4 blocks per CU instead; see
// lds_reserve.)
#ifndef NZ1_FLAT_BLOCK
#define NZ1_FLAT_BLOCK 128
#endif
#ifndef NZ1_FLAT_UNROLL
#define NZ1_FLAT_UNROLL 2
#endif
constexpr int kFlatBlock = NZ1_FLAT_BLOCK;                       // threads per block
constexpr int kFlatUnroll = NZ1_FLAT_UNROLL;                     // thread-vectors per thread
constexpr uint32_t kFlatTile = kFlatBlock * kFlatUnroll * kVec;  // elements per block
struct FlatSpan {
    const uint16_t* grad;
    uint16_t* half;
    float* master;
    float* m;
    float* v;                      // null for momentum SGD
    uint64_t n;                    // elements
    // ntiles + 1 words: bit 0 = decay flag of the tile's first element, bits 1.. = index
    // in `change` of the tile's first flag change; word T+1 ends tile T's list
    const uint32_t* tile_word;
    const uint32_t* change;        // in-tile offsets (1 .. kFlatTile-1) where the flag flips
    uint32_t ntiles;
};

struct FinalizeArgs {
    double clip_norm;
    double beta1, beta2;
    double growth_factor, backoff_factor;
    double predivide_factor;
    double dp_world_size;
    float min_scale;
    int32_t dynamic;
    int32_t growth_interval;
};

struct UpdateArgs {
    float b1, omb1, b2, omb2, eps, wd, lr;
};

// A norm pass of at most this many blocks hands its partials straight to the update,
// which then takes the step's decisions itself (no finalize launch): flat partitions,
// whose norm pass runs as at most this many large blocks when the shard is not small,
// and other layouts below ~2M elements whose segments add few norm chunks (see
// make_plan).  0 = always a separate finalize.
constexpr uint32_t kFuseMaxParts = 256;
#ifndef NZ1_UPDATE_DECIDES
#define NZ1_UPDATE_DECIDES 1
#endif
constexpr bool kUpdateDecides = NZ1_UPDATE_DECIDES;
// Small shards split the norm pass into at least about this many blocks (shorter norm
// chunks, down to the update chunk length).  On the 1M-element shard: 11.4-11.5 us per
// step at 64, 11.9-12.1 at 16, 12.7-12.8 at 256 (whose fused update sums four waves of
// partials), 12.5-13.5 with a separate finalize (same process, alternating builds).
#ifndef NZ1_NORM_TARGET_BLOCKS
#define NZ1_NORM_TARGET_BLOCKS 64
#endif
constexpr uint32_t kNormTargetBlocks = NZ1_NORM_TARGET_BLOCKS;

// Shards of at most this many elements read the gradient in the norm pass with
// cache-allocating loads, so the update's second read of it hits the chip's 256 MB
// Infinity Cache; larger shards use non-temporal loads (their gradient does not stay
// resident, and allocating it slows the norm pass: 215M elements 110-117 against 64 us).
// Measured on MI355X with a 2 GB copy between steps (us per step, non-temporal /
// cache-allocating): 1M 18.2 / 17.8, 2M 26.7 / 26.1, 4M 38.0 / 36.8, 8M 57.6 / 56.0, 16M
// 106.6 / 103.0, 24M 144.4 / 142.4, 44M 242 / 245, 215M 1103-1110 / 1137-1140.
#ifndef NZ1_NORM_CACHED_MAX
#define NZ1_NORM_CACHED_MAX (1ull << 24)
#endif
constexpr uint64_t kNormCachedMax = NZ1_NORM_CACHED_MAX;

// Optional timing of one launch: both null, or two events that receive the kernel's own
// start and stop time from its dispatch (no marker packets between kernels).
struct KernelTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// What an update needs to take the step's decisions itself (small norm grids): the norm
// pass's nparts <= kFuseMaxParts partials, its snapshot of the pre-step state, and the
// state block that block 0 writes.
struct FuseIn {
    const double* partial;
    uint32_t nparts;
    const DevState* snap;
    DevState* st;
    FinalizeArgs fin;
};

// Launchers (zero1_kernels.hip).  Each returns the hipError_t of its launch.
// snap (optional): the norm pass copies the pre-step state there for a fused update.
// nt_loads: non-temporal gradient loads (else cache-allocating; see kNormCachedMax).
// big: kNormBigBlock threads per block (else kBlock).
hipError_t launch_norm(int dtype, bool nt_loads, bool big, const Chunk* chunks, uint32_t nchunks,
                       uint32_t blocks, const DevState* st, double* partial, DevState* snap,
                       uint32_t lds_reserve, hipStream_t stream, const KernelTiming& t = {});
// The finalize sums partial[0, nparts) in a fixed order (the norm pass's partials, or the
// ranks' squared norms of a split step), then takes the step's decisions.
hipError_t launch_finalize(const double* partial, uint32_t nparts, DevState* st,
                           const FinalizeArgs& a, hipStream_t stream, const KernelTiming& t = {});
hipError_t launch_reduce(const double* partial, uint32_t nparts, double* out, hipStream_t stream);
hipError_t launch_segment_sumsq(const double* partial, const uint32_t* range, uint32_t nseg,
                                double* out, hipStream_t stream);
hipError_t launch_set_state(DevState* st, float scale, int32_t good_steps, int64_t step,
                            int64_t skipped, int32_t consecutive, double predivide, double dp,
                            hipStream_t stream);
// fuse: null (the finalize ran; the update reads its decision from st) or the inputs of
// the update's own decision.
hipError_t launch_update(int dtype, int optimizer, const Chunk* chunks, uint32_t nchunks,
                         const DevState* st, const UpdateArgs& a, const FuseIn* fuse,
                         uint32_t lds_reserve, hipStream_t stream, const KernelTiming& t = {});
hipError_t launch_flat_update(int dtype, int optimizer, const FlatSpan& f, const DevState* st,
                              const UpdateArgs& a, const FuseIn* fuse, uint32_t lds_reserve,
                              hipStream_t stream, const KernelTiming& t = {});

// Static LDS (bytes) of the norm kernel: launch reservations subtract it so that the
// requested number of blocks per CU really fits.
// Static LDS of the norm kernel at kBlock and at kNormBigBlock threads per block.
hipError_t norm_static_lds(uint32_t* bytes, uint32_t* big_bytes);

// The unscale factor for scale s, computed in double and rounded once to FP32; the
// host (initial state) and the finalize kernel evaluate the same expression.
__host__ __device__ inline float unscale_factor(double predivide, double dp, float s) {
    return (float)(predivide / (dp * (double)s));
}

}  // namespace nz1

// ------------------------------------------------------------------------------------
// Host side shared by the C-ABI translation units (zero1_api.hip, zero1_noalloc.hip).
// ------------------------------------------------------------------------------------
#include "neox_zero1.h"

#include <vector>

namespace nz1 {

// Records the message for neox_zero1_last_error() on this thread and returns code.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int set_hip_error(hipError_t e, const char* what);

// The work decomposition of a segment list: what create() uploads and neox_zero1_plan()
// describes.
struct Plan {
    uint32_t C = 0;                        // update chunk length
    uint32_t C1 = 0;                       // norm chunk length
    std::vector<Chunk> table, norm_table;  // update and norm work tables
    uint64_t nchunks = 0;                  // update chunks (table.size() when it is built)
    bool flat = false;                     // flat partition: the update runs over tiles
    bool norm_big = false;                 // the norm pass runs kNormBigBlock-thread blocks
    uint64_t numel = 0;
    std::vector<uint32_t> tile_word, change;
};
// Validates the config and the segments, then builds the tables.  The update chunk table
// of a flat partition, which the flat update does not read, is built only when
// `want_table` asks for it.  NEOX_OK or an error code (the message recorded).
int make_plan(const neox_zero1_config* cfg, const neox_segment* segs, uint64_t nseg, Plan& p,
              bool want_table = false);

// Launch constants derived from a validated config.
FinalizeArgs finalize_args(const neox_zero1_config& cfg);
UpdateArgs update_args(const neox_zero1_config& cfg);   // lr left at 0
// The device state block before the first step of a run: scaler counters as given,
// unscale factor for `scale`, no decision yet (skip set).
DevState initial_state(const neox_zero1_config& cfg, float scale, int32_t good_steps,
                       int64_t step, int64_t skipped, int32_t consecutive);

// Dynamic LDS each pass's blocks reserve (only to cap blocks per CU) on one device.
struct LdsReserve {
    uint32_t norm = 0, norm_big = 0, update = 0, flat = 0;
};
// update_blocks: the update grid (flat tiles or chunk-table entries), which sets how many
// update blocks share a CU.
int lds_reserve(int device, int optimizer, uint64_t update_blocks, LdsReserve* out);

// Everything one step launches, with device addresses resolved: what a handle keeps and
// what the allocation-free entry point assembles in its scratch.
struct StepLaunch {
    int dtype = 0, optimizer = 0;
    bool norm_nt = true;           // non-temporal gradient loads in the norm pass
    bool norm_big = false;         // kNormBigBlock-thread norm blocks
    const Chunk* norm_chunks = nullptr;
    uint32_t nnorm = 0, norm_blocks = 0;
    double* partial = nullptr;            // norm_blocks doubles
    DevState* st = nullptr;
    DevState* snap = nullptr;             // pre-step state copy (fused steps)
    bool fused = false;                   // norm_blocks <= kFuseMaxParts: no finalize launch
    FinalizeArgs fin{};
    UpdateArgs upd{};
    bool flat = false;
    FlatSpan span{};                      // flat update
    const Chunk* chunks = nullptr;        // chunked update
    uint32_t nchunks = 0;
    LdsReserve lds{};
    // per-segment telemetry after the norm pass (all null / 0 when off)
    const uint32_t* seg_range = nullptr;
    double* seg_sumsq = nullptr;
    uint32_t nseg = 0;
};
// norm -> finalize (unless fused) -> update on stream; t3: null, or timings of the three
// kernels (the finalize's is not used when fused).
hipError_t enqueue_step(const StepLaunch& s, float lr, hipStream_t stream, const KernelTiming* t3);
// the update alone after a finalize has taken the decision (split step)
hipError_t enqueue_update_only(const StepLaunch& s, float lr, hipStream_t stream);
// Whether the split step's update takes the decisions itself from nranks values: at most
// kFuseMaxParts of them, and a layout whose update decides (a flat partition, or a norm
// grid small enough that the single step's update decides too).
bool split_update_decides(const StepLaunch& s, uint32_t nranks);

}  // namespace nz1
