// stream_probe.hip -- attainable-bandwidth probes for the benchmark (see
// include/neox_stream_probe.h).  They share no code with the step's kernels on purpose:
// each is a self-contained restatement of an access pattern.
#include "neox_stream_probe.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <string>

namespace {

thread_local std::string g_err = "no error";

int fail(int code, const char* msg) {
    g_err = msg;
    return code;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool NTS, typename T>
__device__ __forceinline__ void put(T* p, T v) {
    if constexpr (NTS) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <bool NTS>
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, uint64_t nvec) {
    const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < nvec) put<NTS>(dst + i, src[i]);
}

// The update's access pattern: tiles of NT * U 8-element vectors walked last-to-first,
// U vectors per thread, the step's arithmetic replaced by a few multiplies; NTS:
// non-temporal stores.
template <int NT, int U, bool NTS>
__global__ __launch_bounds__(NT) void pattern_kernel(const u32x4* __restrict__ g,
                                                     u32x4* __restrict__ h,
                                                     f32x4* __restrict__ w,
                                                     f32x4* __restrict__ m,
                                                     f32x4* __restrict__ v, uint64_t nvec) {
    const uint64_t tile = gridDim.x - 1 - blockIdx.x;
    const uint64_t base = tile * (uint64_t)(NT * U);
    u32x4 G[U];
    f32x4 W[U][2], M[U][2], V[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t i = base + u * NT + threadIdx.x;
        if (i < nvec) {
            G[u] = g[i];
            W[u][0] = w[2 * i]; W[u][1] = w[2 * i + 1];
            M[u][0] = m[2 * i]; M[u][1] = m[2 * i + 1];
            V[u][0] = v[2 * i]; V[u][1] = v[2 * i + 1];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t i = base + u * NT + threadIdx.x;
        if (i < nvec) {
            const float gs = __uint_as_float(G[u].x << 16) * 1e-30f;
            put<NTS>(w + 2 * i, W[u][0] + gs); put<NTS>(w + 2 * i + 1, W[u][1] + gs);
            put<NTS>(m + 2 * i, M[u][0] * 0.9f); put<NTS>(m + 2 * i + 1, M[u][1] * 0.9f);
            put<NTS>(v + 2 * i, V[u][0] * 0.95f); put<NTS>(v + 2 * i + 1, V[u][1] * 0.95f);
            const u32x4 hh = {__float_as_uint(W[u][0].x) >> 16, __float_as_uint(W[u][0].z) >> 16,
                              __float_as_uint(W[u][1].x) >> 16, __float_as_uint(W[u][1].z) >> 16};
            put<NTS>(h + i, hh);
        }
    }
}

template <int NT, int U>
void launch_pattern(const void* grad, void* half, float* master, float* exp_avg, float* exp_avg_sq,
                    uint64_t n, uint32_t lds, bool nts, hipStream_t stream) {
    const uint64_t nvec = n / 8;
    const uint64_t tiles = (nvec + NT * U - 1) / (NT * U);
    if (nts)
        pattern_kernel<NT, U, true><<<(uint32_t)tiles, NT, lds, stream>>>(
            (const u32x4*)grad, (u32x4*)half, (f32x4*)master, (f32x4*)exp_avg, (f32x4*)exp_avg_sq, nvec);
    else
        pattern_kernel<NT, U, false><<<(uint32_t)tiles, NT, lds, stream>>>(
            (const u32x4*)grad, (u32x4*)half, (f32x4*)master, (f32x4*)exp_avg, (f32x4*)exp_avg_sq, nvec);
}

bool a16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" int neox_probe_copy(const void* src, void* dst, uint64_t bytes, int32_t nt_stores,
                               void* hip_stream) {
    if (!src || !dst || bytes == 0 || bytes % 16 || !a16(src) || !a16(dst))
        return fail(-1, "copy probe: null, unaligned or bad size");
    const uint64_t nvec = bytes / 16;
    const uint64_t grid = (nvec + 255) / 256;
    if (grid > 0xFFFFFFFFull / 256) return fail(-1, "copy probe: too large");
    if (nt_stores)
        copy_kernel<true><<<(uint32_t)grid, 256, 0, (hipStream_t)hip_stream>>>(
            (const u32x4*)src, (u32x4*)dst, nvec);
    else
        copy_kernel<false><<<(uint32_t)grid, 256, 0, (hipStream_t)hip_stream>>>(
            (const u32x4*)src, (u32x4*)dst, nvec);
    return hipGetLastError() == hipSuccess ? 0 : fail(-2, "copy probe launch failed");
}

extern "C" int neox_probe_update_pattern(const void* grad, void* half, float* master,
                                         float* exp_avg, float* exp_avg_sq, uint64_t n,
                                         int32_t threads, int32_t vectors, int32_t blocks_per_cu,
                                         int32_t nt_stores, void* hip_stream) {
    if (!grad || !half || !master || !exp_avg || !exp_avg_sq || n == 0 || n % 8)
        return fail(-1, "pattern probe: null or n not a positive multiple of 8");
    if (!a16(grad) || !a16(half) || !a16(master) || !a16(exp_avg) || !a16(exp_avg_sq))
        return fail(-1, "pattern probe: arrays must be 16-byte aligned");
    if ((threads != 64 && threads != 128 && threads != 256 && threads != 512) ||
        (vectors != 1 && vectors != 2 && vectors != 4) || blocks_per_cu < 0 || blocks_per_cu > 16)
        return fail(-1, "pattern probe: threads 64/128/256/512, vectors 1/2/4, blocks_per_cu 0..16");
    const uint64_t tiles = (n / 8 + (uint64_t)threads * vectors - 1) / ((uint64_t)threads * vectors);
    if (tiles * (uint64_t)threads > 0xFFFFFFFFull) return fail(-1, "pattern probe: too large");
    uint32_t lds = 0;
    if (blocks_per_cu) {
        int dev = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess)
            return fail(-2, "pattern probe: device query failed");
        lds = (uint32_t)(per_cu / blocks_per_cu) & ~1023u;   // caps the blocks sharing a CU
    }
    hipStream_t st = (hipStream_t)hip_stream;
#define NZP_CASE(T, V)                                                                        \
    if (threads == T && vectors == V) {                                                       \
        launch_pattern<T, V>(grad, half, master, exp_avg, exp_avg_sq, n, lds, nt_stores, st); \
        return hipGetLastError() == hipSuccess ? 0 : fail(-2, "pattern probe launch failed"); \
    }
    NZP_CASE(64, 1) NZP_CASE(64, 2) NZP_CASE(64, 4)
    NZP_CASE(128, 1) NZP_CASE(128, 2) NZP_CASE(128, 4)
    NZP_CASE(256, 1) NZP_CASE(256, 2) NZP_CASE(256, 4)
    NZP_CASE(512, 1) NZP_CASE(512, 2) NZP_CASE(512, 4)
#undef NZP_CASE
    return fail(-1, "pattern probe: unreachable shape");
}

extern "C" const char* neox_probe_last_error(void) { return g_err.c_str(); }
