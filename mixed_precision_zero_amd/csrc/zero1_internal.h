// zero1_internal.h -- types shared by the host side and the gfx950 kernels of the
// ZeRO-1 mixed-precision Adam step.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nz1 {

constexpr int kBlock = 256;   // threads per block of the norm, finalize and telemetry kernels
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
// best on MI355X: 128 threads x 2 vectors (2,048-element tiles) at 2 blocks per CU;
// fewer tiles in flight per CU keep the chip's open DRAM rows few, and the block's
// single round trip keeps that low occupancy from exposing latency.
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

// Optional timing of one launch: both null, or two events that receive the kernel's own
// start and stop time from its dispatch (no marker packets between kernels).
struct KernelTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// Launchers (zero1_kernels.hip).  Each returns the hipError_t of its launch.
hipError_t launch_norm(int dtype, const Chunk* chunks, uint32_t nchunks, uint32_t blocks,
                       const DevState* st, double* partial, uint32_t lds_reserve,
                       hipStream_t stream, const KernelTiming& t = {});
hipError_t launch_finalize(const double* partial, uint32_t nparts, const double* sumsq_in,
                           DevState* st, const FinalizeArgs& a, hipStream_t stream,
                           const KernelTiming& t = {});
hipError_t launch_reduce(const double* partial, uint32_t nparts, double* out, hipStream_t stream);
hipError_t launch_segment_sumsq(const double* partial, const uint32_t* range, uint32_t nseg,
                                double* out, hipStream_t stream);
hipError_t launch_set_state(DevState* st, float scale, int32_t good_steps, int64_t step,
                            int64_t skipped, int32_t consecutive, double predivide, double dp,
                            hipStream_t stream);
hipError_t launch_update(int dtype, int optimizer, const Chunk* chunks, uint32_t nchunks,
                         const DevState* st, const UpdateArgs& a, uint32_t lds_reserve,
                         hipStream_t stream, const KernelTiming& t = {});
hipError_t launch_flat_update(int dtype, int optimizer, const FlatSpan& f, const DevState* st,
                              const UpdateArgs& a, uint32_t lds_reserve, hipStream_t stream,
                              const KernelTiming& t = {});

// The unscale factor for scale s, computed in double and rounded once to FP32; the
// host (initial state) and the finalize kernel evaluate the same expression.
__host__ __device__ inline float unscale_factor(double predivide, double dp, float s) {
    return (float)(predivide / (dp * (double)s));
}

}  // namespace nz1
